// Head-dimension 64 instantiation of the backward kernels (fa_bwd_kernels.h).
// This source is compiled with the MFMA results kept in VGPRs
// (-amdgpu-mfma-vgpr-form): at d = 64 the dK/dV kernel then needs no
// AGPR<->VGPR copies and the backward runs 8-15% faster; at d = 128 the same
// flag costs 2%, so fa_bwd.hip is compiled without it.
#include "fa_bwd_kernels.h"

namespace fa92 {

bool bwd_launch_d64(const BwdParams& p, int B, hipStream_t s) { return launch_bwd<64>(p, B, s); }

}  // namespace fa92
