// Head-dimension 64 instantiation of the backward kernels (fa_bwd_kernels.h),
// in a source of its own so each head dimension compiles separately.
#include "fa_bwd_kernels.h"

namespace fa92 {

bool bwd_launch_d64(const BwdParams& p, int B, hipStream_t s) { return launch_bwd<64>(p, B, s); }

}  // namespace fa92
