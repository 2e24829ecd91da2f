#!/usr/bin/env python3
"""Writes fa_fwd_d128_loop.inc (and its clobber list, fa_fwd_d128_clobbers.inc):
the per-item body of fa_fwd_d128_kernel (bf16, d = 128, contiguous
self-attention) as one gfx950 inline-asm program.  The build runs this
script before compiling.

Why asm: the body is a software pipeline whose value is the exact interleave
of matrix-core and vector work inside one wave -- the exponentials of one key
block issue between the MFMAs of the next block's scores and of the previous
block's P.V -- and a fixed register plan (O accumulators and Q in AGPRs;
scores, probabilities, row sums and LDS operands in VGPRs) that the compiler
does not keep.

What it computes is the online softmax of the tiled exact attention forward
(FlashAttention pages: the forward pass with running max m, running sum l
and rescaled accumulator; exp2 with the scale folded into log2 units):
every wave owns 64 query rows (two 32-row tiles A and B) and visits the key
blocks of 64 keys.  Iteration i of the block loop (one workgroup barrier
each) runs two phases:
  X: MFMAs of S(i) = K_i Q^T for both tiles       | softmax of (i-1, tile B)
  Y: MFMAs of O^T += V_{i-1}^T P^T for both tiles | softmax of (i,   tile A)
so each softmax runs beside the MFMAs of another block; each K and V^T
operand read from LDS feeds both tiles.  K and V blocks are staged two
iterations ahead into three LDS slots each with direct-to-LDS loads spread
over the X phase.  The row max is lazy: exponentials use the running
reference max and a block whose fp32 row sum exceeds 2^20 (or is not
finite: first block, masked rows) takes an out-of-line path that moves the
reference, rescales the state and redoes the block.  Only the wave's last key
block can hold hidden keys (causal diagonal, key padding, N not a multiple of
64); its softmax masks them.

Hazards the hardware does not interlock are kept apart by the schedule
(results of MFMA, transcendental and dot instructions); check_hazards()
fails generation on the ones a schedule change could reintroduce.

Usage: python3 gen_fwd_d128_loop.py [--debug | --profile] [--out DIR]
  --debug    register-dump epilogue instead of O / LSE (debug builds)
  --profile  shader-clock marks per phase, dumped instead of O / LSE
"""
import os

# ---------------------------------------------------------------- registers
S_A = 0                       # S tile A: v[0:31]  (key tile kt at +16kt)
S_B = (32, 64)                # S tile B, by parity of the block: v[32:63], v[64:95]
P_A = (96, 112)               # P^T tile A (bf16 pairs), by parity: 16 regs, chunk pc at +4pc
P_B = 128                     # P^T tile B: v[128:143]
RING = 144                    # LDS operand ring: 8 slots of 4 VGPRs, v[144:175]
NSLOT = 8
ET = 198                      # exp temporaries v[198:205]
M = {"A": 176, "B": 179}      # reference max (log2 units), per row
LE = {"A": 178, "B": 181}     # row sum of the fp32 probabilities (per lane half)
RE = {"A": 182, "B": 184}     # fp32 block sums, two partial sums each
T = 186                       # slow-path / epilogue temporaries v[186:190]
NINF = 191                    # -inf
ONES = 192                    # 0x3f803f80: a pair of bf16 ones
# Row sums of the bf16-rounded probabilities (they normalise O), two partial
# sums per lane and tile, accumulated with v_dot2c after the phase's last
# MFMA: dot instructions do not overlap MFMAs, so inside the interleaved
# stream they would stall it.
LV = {"A": (177, 193), "B": (180, 194)}
NVGPR = 206                   # v[0:205] are clobbered

ACC = {"A": 0, "B": 64}       # O^T accumulators: a[0:63] tile A, a[64:127] tile B (dt at +16dt)
QA = {"A": 128, "B": 160}     # Q tiles (MFMA B operand), ks at +4ks: a[128:191]
NAGPR = 192

# SGPRs (clobbered): s[64:67] K rsrc (next block to stage), s[68:71] V rsrc,
# s[72:75] Q / O rsrc, s[76:79] LSE rsrc, s80 block counter i, s81 scratch;
# LDS slot byte offsets of iteration i: s56 = (i%3)*SLOT, s57 = ((i+1)%3)*SLOT,
# s58 = ((i+2)%3)*SLOT, s59 scratch; s60 / s61: M0 bases of this iteration's
# K / V staging.
SK, SV, SQ, SL, SI = 64, 68, 72, 76, 80
SR0, SR1, SR2, SRT, SMK, SMV = 56, 57, 58, 59, 60, 61
SGPRS = list(range(56, 62)) + list(range(64, 82))

KROW = 272                    # K row stride in LDS (bytes): 256 + 16
VROW = 320                    # V row stride in LDS (bytes): 256 + 64
SLOT = 20480                  # bytes per K or V slot (64 rows, padded)
VBASE = 3 * SLOT              # three K slots, then three V slots
LDS_BYTES = 6 * SLOT
KRD, VRD = 196, 197           # LDS read bases of this iteration's K and V slots

LOOKAHEAD = 6                 # LDS operands requested ahead of their MFMAs (< NSLOT - 1)
LIMIT_SUM = "0x49800000"      # 2^20


def v(r, n=1):
    return f"v{r}" if n == 1 else f"v[{r}:{r + n - 1}]"


def a(r, n=1):
    return f"a{r}" if n == 1 else f"a[{r}:{r + n - 1}]"


def s(r, n=1):
    return f"s{r}" if n == 1 else f"s[{r}:{r + n - 1}]"


PROF_BUCKETS = ["vmwait", "barrier", "loads", "X", "Y", "idle", "epi", "total"]
PROF = False                  # set by --profile: clock marks at phase boundaries


def mark(bucket):
    """Profile builds: add the shader clocks since the last mark to a bucket."""
    if not PROF:
        return []
    b = 82 + PROF_BUCKETS.index(bucket)
    return ["s_memtime s[92:93]", "s_waitcnt lgkmcnt(0)", "s_sub_u32 s94, s92, s90",
            f"s_add_u32 s{b}, s{b}, s94", "s_mov_b64 s[90:91], s[92:93]"]


class Prog:
    def __init__(self):
        self.main = []
        self.cold = []      # out-of-line slow paths
        self.nlabel = 0

    def label(self, stem):
        self.nlabel += 1
        return f".Lfa{stem}{self.nlabel}_%="

    def emit(self, *ins):
        self.main.extend(ins)


# ------------------------------------------------------------ softmax (VALU)
# Lags (in MFMA slots) of each step of one score element e after its fma at
# slot e: the exponential, the fp32 add and the bf16 pack of its pair.  One
# element enters per slot, so each slot holds one exponential and two or
# three full-rate VALU operations, which issue while the slot's 32-cycle MFMA
# runs; every result is read a slot or more after it is written (an
# exponential's result needs a wait state).
LAG_EXP, LAG_ADD, LAG_CVT = 1, 2, 2


def softmax_slots(tile, sreg, preg, base, masked):
    """VALU work of one block's softmax for one 32-row tile, as a list of
    slots (one per MFMA of the phase it runs beside, extra slots after it):
    mask (last block only), p = 2^(s*c - base), P^T packed to bf16, fp32
    block sum in RE[tile] and bf16-rounded block sum in RE[tile]+2."""
    re0, re1 = RE[tile], RE[tile] + 1
    nslot = 32 + LAG_ADD + 1
    # each slot: its exponential first, so that the rest of the slot sits
    # between it and the reads of its result when slots are issued back to back
    exps = [[] for _ in range(nslot)]
    slots = [[] for _ in range(nslot)]
    lim = "%[limA]" if tile == "A" else "%[limB]"
    for e in range(32):
        pc, w, j = e // 8, (e % 8) // 2, e % 2
        reg = sreg + 16 * (pc // 2) + 8 * (pc % 2) + 2 * w + j
        t = ET + e % 8
        if masked:
            idx = 32 * (pc // 2) + 16 * (pc % 2) + 2 * w + j   # key offset less 8*half
            slots[e] += [f"v_cmp_gt_i32_e32 vcc, {idx}, {lim}",
                         f"v_cndmask_b32_e32 {v(reg)}, {v(reg)}, {v(NINF)}, vcc"]
        slots[e].append(f"v_fma_f32 {v(t)}, {v(reg)}, %[c], -{v(base)}")
        exps[e + LAG_EXP].append(f"v_exp_f32_e32 {v(t)}, {v(t)}")
        acc = re0 if j == 0 else re1
        if e < 2:
            slots[e + LAG_ADD].append(f"v_mov_b32_e32 {v(acc)}, {v(t)}")
        else:
            slots[e + LAG_ADD].append(f"v_add_f32_e32 {v(acc)}, {v(acc)}, {v(t)}")
        if j == 1:
            pr = preg + 4 * pc + w
            slots[e + LAG_CVT].append(f"v_cvt_pk_bf16_f32 {v(pr)}, {v(t - 1)}, {v(t)}")
    slots[32 + LAG_ADD].append(f"v_add_f32_e32 {v(re0)}, {v(re0)}, {v(re1)}")
    return [x + y for x, y in zip(exps, slots)]


def softmax_valu(tile, sreg, preg, base, masked):
    return [ins for slot in softmax_slots(tile, sreg, preg, base, masked) for ins in slot]


def slow_path(prog, tile, sreg, preg, back):
    """Out-of-line full step for one tile's block: row max of the scores,
    move the reference max, rescale O, l and le by 2^(m_old - m_new), redo
    the exponentials against the new reference (0 for a row with no visible
    key yet) and add the block sums."""
    lab = prog.label("slow" + tile)
    c = prog.cold
    c.append(f"{lab}:")
    c.extend(["s_nop 15", "s_nop 15", "s_nop 15"])      # outstanding MFMAs retire
    t0, t1, t2, t3, t4 = T, T + 1, T + 2, T + 3, T + 4
    c.append(f"v_max3_f32 {v(t0)}, {v(sreg)}, {v(sreg + 1)}, {v(sreg + 2)}")
    r = 3
    while r < 32:
        if r + 1 < 32:
            c.append(f"v_max3_f32 {v(t0)}, {v(t0)}, {v(sreg + r)}, {v(sreg + r + 1)}")
            r += 2
        else:
            c.append(f"v_max_f32_e32 {v(t0)}, {v(t0)}, {v(sreg + r)}")
            r += 1
    c.append(f"v_mov_b32_e32 {v(t1)}, {v(t0)}")
    c.append("s_nop 1")
    c.append(f"v_permlane32_swap_b32_e32 {v(t0)}, {v(t1)}")
    c.append("s_nop 1")
    c.append(f"v_max_f32_e32 {v(t0)}, {v(t0)}, {v(t1)}")          # row max of raw scores
    c.append(f"v_mul_f32_e32 {v(t0)}, %[c], {v(t0)}")
    c.append(f"v_max_f32_e32 {v(t2)}, {v(M[tile])}, {v(t0)}")     # m_new
    c.append(f"v_sub_f32_e32 {v(t3)}, {v(M[tile])}, {v(t2)}")
    c.append(f"v_exp_f32_e32 {v(t3)}, {v(t3)}")
    c.append(f"v_cmp_eq_f32_e32 vcc, {v(M[tile])}, {v(t2)}")
    c.append(f"v_cndmask_b32_e64 {v(t3)}, {v(t3)}, 1.0, vcc")      # alpha
    acc = ACC[tile]
    for g in range(0, 64, 8):
        for k in range(8):
            c.append(f"v_accvgpr_read_b32 {v(ET + k)}, {a(acc + g + k)}")
        for k in range(8):
            c.append(f"v_mul_f32_e32 {v(ET + k)}, {v(t3)}, {v(ET + k)}")
        for k in range(8):
            c.append(f"v_accvgpr_write_b32 {a(acc + g + k)}, {v(ET + k)}")
    c.append("s_nop 2")                      # partial sums were last written by dot instructions
    for r in LV[tile]:
        c.append(f"v_mul_f32_e32 {v(r)}, {v(t3)}, {v(r)}")
    c.append(f"v_mul_f32_e32 {v(LE[tile])}, {v(t3)}, {v(LE[tile])}")
    c.append(f"v_mov_b32_e32 {v(M[tile])}, {v(t2)}")
    c.append(f"v_cmp_eq_f32_e32 vcc, 0xff800000, {v(t2)}")
    c.append(f"v_cndmask_b32_e64 {v(t4)}, {v(t2)}, 0, vcc")        # base
    c.extend(softmax_valu(tile, sreg, preg, t4, False))
    c.append(f"v_add_f32_e32 {v(LE[tile])}, {v(LE[tile])}, {v(RE[tile])}")
    c.append(f"s_branch {back}")
    return lab


def check(prog, tile, sreg, preg):
    """Fast-path test of a tile's block sums; the slow path returns here."""
    back = prog.label("back" + tile)
    lab = slow_path(prog, tile, sreg, preg, back)
    out = [f"v_cmp_nge_f32_e32 vcc, {LIMIT_SUM}, {v(RE[tile])}",
           "s_nop 1",
           f"s_cbranch_vccnz {lab}",
           f"v_add_f32_e32 {v(LE[tile])}, {v(LE[tile])}, {v(RE[tile])}",
           f"{back}:"]
    # bf16-rounded row sums of this block's P^T into the two partial sums
    for r in range(16):
        out.append(f"v_dot2c_f32_bf16_e32 {v(LV[tile][r % 2])}, {v(ONES)}, {v(preg + r)}")
    return out


# ------------------------------------------------------- one loop iteration
def k_operands():
    """The 16 K operands of S(i) in issue order: (ks, kt), one ds_read_b128
    (offsets within the slot; the slot is in the address register)."""
    ops = []
    for ks in range(8):
        for kt in range(2):
            off = kt * 32 * KROW + 32 * ks
            ops.append(("K", (ks, kt), [("ds_read_b128", 0, off)]))
    return ops


def v_operands():
    """The 16 V^T operands of P.V in issue order: (pc, dt), two transposing
    8-byte reads (keys +0..3 and +4..7 of the lane's 8)."""
    ops = []
    for pc in range(4):
        for dt in range(4):
            reads = []
            for half in range(2):
                off = (16 * pc + 4 * half) * VROW + 64 * dt
                reads.append(("ds_read_b64_tr_b16", 2 * half, off))
            ops.append(("V", (pc, dt), reads))
    return ops


LOAD_AT = [1 + 3 * g for g in range(10)]   # X-phase MFMAs after which the staging groups go


def k_prefetch():
    """End of an iteration whose successor computes S: point the K read base
    at the next K slot and request that iteration's first LOOKAHEAD operands.
    K(i+1) was staged in iteration i-1 and the barrier that opened iteration
    i waited for all staging, so every wave's part of it has landed."""
    out = [f"v_add_u32_e32 {v(KRD)}, {s(SR1)}, %[kaddr]"]
    for k, (_, _, reads) in enumerate(k_operands()[:LOOKAHEAD]):
        for ins, sub, off in reads:
            out.append(f"{ins} {v(RING + 4 * (k % NSLOT) + sub, 4)}, {v(KRD)} offset:{off}")
    return out


def iteration(prog, p, do_s, sm_b, do_pv, sm_a, prefetched=False, prefetch_next=False):
    """Instructions of one block-loop iteration with parity p.
    do_s: S(i) MFMAs; sm_b: None | 'plain' | 'masked' softmax of (i-1, B);
    do_pv: P.V of block i-1; sm_a: softmax of (i, A)."""
    ops = (k_operands() if do_s else []) + (v_operands() if do_pv else [])
    out = []
    issued = []            # (operand index, number of read instructions)

    def issue(k):
        kind, _, reads = ops[k]
        slot = RING + 4 * (k % NSLOT)
        addr = v(KRD) if kind == "K" else v(VRD)
        for ins, sub, off in reads:
            n = 4 if ins == "ds_read_b128" else 2
            out.append(f"{ins} {v(slot + sub, n)}, {addr} offset:{off}")
        issued.append((k, len(reads)))

    def wait_for(k):
        after = 0
        seen = False
        for kk, n in issued:
            if seen:
                after += n
            if kk == k:
                seen = True
        assert seen
        out.append(f"s_waitcnt lgkmcnt({min(after, 15)})")

    nxt = 0
    if prefetched:
        assert do_s
        for k in range(LOOKAHEAD):
            issued.append((k, 1))
        nxt = LOOKAHEAD
    for _ in range(min(LOOKAHEAD, len(ops)) - nxt):
        issue(nxt)
        nxt += 1

    def phase(mfmas, slots, first_valu_nop, loads):
        """Slot 0 before the first MFMA, slot m + 1 after MFMA m; staging
        group g after MFMA LOAD_AT[g]."""
        nonlocal nxt
        if not mfmas:
            for sl in slots:
                out.extend(sl)
            for g in loads:
                out.extend(g)
            return
        if slots:
            if first_valu_nop:
                out.append("s_nop 11")       # scores of tile A were just written by MFMA
            out.extend(slots[0])
        started = set()
        for m, (k, text) in enumerate(mfmas):
            if k not in started:
                wait_for(k)
                started.add(k)
                if nxt < len(ops):
                    issue(nxt)
                    nxt += 1
            out.append(text)
            if m + 1 < len(slots):
                out.extend(slots[m + 1])
            for g, at in enumerate(LOAD_AT):
                if g < len(loads) and at == min(m, len(mfmas) - 1) and m < len(mfmas):
                    out.extend(loads[g])
        for sl in slots[len(mfmas) + 1:]:
            out.extend(sl)
        for g, at in enumerate(LOAD_AT):
            if g < len(loads) and at >= len(mfmas):
                out.extend(loads[g])

    # phase X
    x_mfma = []
    if do_s:
        sb = S_B[p]
        for k in range(16):
            ks, kt = ops[k][1]
            ring = RING + 4 * (k % NSLOT)
            for tile, sreg in (("A", S_A), ("B", sb)):
                d = sreg + 16 * kt
                src_c = "0" if ks == 0 else v(d, 16)
                x_mfma.append((k, f"v_mfma_f32_32x32x16_bf16 {v(d, 16)}, {v(ring, 4)}, "
                                  f"{a(QA[tile] + 4 * ks, 4)}, {src_c}"))
    x_valu = softmax_slots("B", S_B[1 - p], P_B, M["B"], sm_b == "masked") if sm_b else []
    loads = iteration_loads()
    phase(x_mfma, x_valu, False, loads if do_s else [])
    if sm_b:
        out.extend(check(prog, "B", S_B[1 - p], P_B))
    out.extend(mark("X"))

    # phase Y
    y_mfma = []
    if do_pv:
        base = 16 if do_s else 0
        for j in range(16):
            k = base + j
            pc, dt = ops[k][1]
            ring = RING + 4 * (k % NSLOT)
            for tile, preg in (("A", P_A[1 - p]), ("B", P_B)):
                acc = ACC[tile] + 16 * dt
                y_mfma.append((k, f"v_mfma_f32_32x32x16_bf16 {a(acc, 16)}, {v(ring, 4)}, "
                                  f"{v(preg + 4 * pc, 4)}, {a(acc, 16)}"))
        if sm_b:
            out.append("s_nop 4")            # P^T of tile B was just written by VALU
    y_valu = softmax_slots("A", S_A, P_A[p], M["A"], sm_a == "masked") if sm_a else []
    if sm_a and do_s and not do_pv:
        out.append("s_nop 15")               # scores of tile A were just written by MFMA
    phase(y_mfma, y_valu, bool(sm_a and do_s and do_pv), [] if do_s else loads)
    if sm_a:
        out.extend(check(prog, "A", S_A, P_A[p]))
    out.extend(mark("Y"))
    if prefetch_next:
        out.extend(k_prefetch())
    assert nxt == len(ops)
    return out


# ------------------------------------------------------------ direct loads
def stage_groups(kind, base=None):
    """This wave's share (5 of 20 KiB) of staging one 64-key block of K or V
    into an LDS slot with direct-to-LDS loads, as 5 instruction groups, and
    the advance of the buffer resource to the next block.  Lane offsets in
    the operands place row padding; reads past the buffer range give zeros
    (blocks past the last one stage zeros into a free slot)."""
    rs = SK if kind == "K" else SV
    mbase = base if base else s(SMK if kind == "K" else SMV)
    groups = [[f"s_add_u32 m0, {mbase}, {u * 4096}", "s_nop 0",
               f"buffer_load_dwordx4 %[{kind.lower()}o{u}], {s(rs, 4)}, 0 offen lds"]
              for u in range(5)]
    # base += 64 rows, bytes left -= 64 rows (not below 0)
    groups[-1] += [f"s_add_u32 {s(rs)}, {s(rs)}, 0x4000",
                   f"s_addc_u32 {s(rs + 1)}, {s(rs + 1)}, 0",
                   f"s_sub_i32 {s(rs + 2)}, {s(rs + 2)}, 0x4000",
                   f"s_max_i32 {s(rs + 2)}, {s(rs + 2)}, 0"]
    return groups


def stage(kind, base=None):
    return [i for g in stage_groups(kind, base) for i in g]


def iteration_loads():
    """Staging of iteration i: K(i+2) into K slot (i+2)%3 and V(i+1) into V
    slot (i+1)%3, both free since the barrier that opened the iteration
    (they held K(i-1) and V(i-2), last read in iteration i-1)."""
    return stage_groups("K") + stage_groups("V")


# ------------------------------------------------------------------ program
DEBUG_VGPRS = list(range(0, 64)) + list(range(96, 112)) + list(range(128, 144)) + list(range(176, 182))  # 102 registers


def build(debug=False):
    prog = Prog()
    e = prog.emit
    # the previous item's waves may still read LDS slots this item restages
    e("s_barrier")
    if PROF:
        e(*[f"s_mov_b32 s{82 + i}, 0" for i in range(len(PROF_BUCKETS))],
          "s_memtime s[90:91]", "s_waitcnt lgkmcnt(0)", "s_mov_b64 s[96:97], s[90:91]")
    # rsrc words: base lo, base hi (stride 0), bytes, raw dword format
    for base, lo, hi, nb in ((SK, "klo", "khi", "kbytes"), (SV, "vlo", "vhi", "vbytes"),
                             (SQ, "qlo", "qhi", "qbytes"), (SL, "llo", "lhi", "lbytes")):
        e(f"s_mov_b32 {s(base)}, %[{lo}]", f"s_and_b32 {s(base + 1)}, %[{hi}], 0xffff",
          f"s_mov_b32 {s(base + 2)}, %[{nb}]", f"s_mov_b32 {s(base + 3)}, 0x20000")
    # K(0), K(1) and V(0) into slot 0, 1 and 0 first (their latency overlaps
    # the rest of the set-up); the loop's slot rotation then starts from
    # (0, 1, 2)
    done = prog.label("done")
    staged = prog.label("staged")
    e("s_cmp_gt_i32 %[nblk], 0", f"s_cbranch_scc0 {staged}")
    e(*stage("K", "%[ldsk]"))
    e(f"s_add_u32 {s(SMK)}, %[ldsk], {SLOT}", *stage("K"))
    e(*stage("V", "%[ldsv]"))
    e(f"s_mov_b32 {s(SR0)}, {2 * SLOT}", f"s_mov_b32 {s(SR1)}, 0", f"s_mov_b32 {s(SR2)}, {SLOT}")
    e(f"{staged}:")
    # Q rows of both tiles into AGPRs (B operand of S^T = K Q^T)
    for tile, qo in (("A", "%[qoff0]"), ("B", "%[qoff1]")):
        for ks in range(8):
            e(f"buffer_load_dwordx4 {a(QA[tile] + 4 * ks, 4)}, {qo}, {s(SQ, 4)}, 0 offen "
              f"offset:{32 * ks}")
    e(f"v_mov_b32_e32 {v(ONES)}, 0x3f803f80", f"v_mov_b32_e32 {v(NINF)}, 0xff800000",
      *[f"v_mov_b32_e32 {v(r)}, 0" for t in ("A", "B") for r in LV[t]])
    for tile in ("A", "B"):
        e(f"v_mov_b32_e32 {v(M[tile])}, 0xff800000", f"v_mov_b32_e32 {v(LE[tile])}, 0")
    for r in range(ACC["A"], ACC["B"] + 64):
        e(f"v_accvgpr_write_b32 {a(r)}, 0")
    e("s_cmp_gt_i32 %[nblk], 0", f"s_cbranch_scc0 {done}")
    e(f"s_mov_b32 {s(SI)}, 0")

    top = prog.label("top")
    nxt = prog.label("next")
    # every block staged so far must have landed: after this barrier K(i),
    # V(i-1) and K(i+1) are visible to all waves (the end of iteration i reads
    # K(i+1) ahead of the next barrier)
    def opening():
        """Barrier that opens an iteration, then the slot rotation."""
        return ["s_waitcnt vmcnt(0)", *mark("vmwait"), "s_barrier", *mark("barrier"),
                f"s_mov_b32 {s(SRT)}, {s(SR0)}", f"s_mov_b32 {s(SR0)}, {s(SR1)}",
                f"s_mov_b32 {s(SR1)}, {s(SR2)}", f"s_mov_b32 {s(SR2)}, {s(SRT)}",
                f"s_add_u32 {s(SMK)}, %[ldsk], {s(SR2)}", f"s_add_u32 {s(SMV)}, %[ldsv], {s(SR1)}",
                f"v_add_u32_e32 {v(KRD)}, {s(SR0)}, %[kaddr]",
                f"v_add_u32_e32 {v(VRD)}, {s(SR2)}, %[vaddr]"]
    e(f"{top}:", *opening())
    # this wave's part of iteration i (jlast = its last key block, -1: none);
    # every variant stages its share of K(i+1) and V(i)
    labs = {k: prog.label(k) for k in ("first", "firstm", "st0", "st1", "last0", "last1",
                                       "tail0", "tail1", "idle0", "idle1")}
    e(*mark("loads"),
      "s_cmp_lt_i32 %[jlast], 0", "s_cbranch_scc1 .Lfaidle_%=",                   # no key block
      f"s_add_i32 {s(SI + 1)}, %[jlast], 1",
      f"s_cmp_gt_i32 {s(SI)}, {s(SI + 1)}", "s_cbranch_scc1 .Lfaidle_%=",       # done, idle
      f"s_cmp_eq_u32 {s(SI)}, 0", f"s_cbranch_scc0 .Lfanotfirst_%=",
      "s_cmp_eq_u32 %[jlast], 0", f"s_cbranch_scc1 {labs['firstm']}",
      f"s_branch {labs['first']}",
      ".Lfanotfirst_%=:",
      f"s_bitcmp1_b32 {s(SI)}, 0", "s_cbranch_scc1 .Lfaodd_%=",
      f"s_cmp_lt_i32 {s(SI)}, %[jlast]", f"s_cbranch_scc1 {labs['st0']}",
      f"s_cmp_eq_u32 {s(SI)}, %[jlast]", f"s_cbranch_scc1 {labs['last0']}",
      f"s_branch {labs['tail0']}",
      ".Lfaodd_%=:",
      f"s_cmp_lt_i32 {s(SI)}, %[jlast]", f"s_cbranch_scc1 {labs['st1']}",
      f"s_cmp_eq_u32 {s(SI)}, %[jlast]", f"s_cbranch_scc1 {labs['last1']}",
      f"s_branch {labs['tail1']}",
      ".Lfaidle_%=:",
      f"s_bitcmp1_b32 {s(SI)}, 0", f"s_cbranch_scc1 {labs['idle1']}",
      f"s_branch {labs['idle0']}")
    # (name, parity, S MFMAs, softmax B, P.V, softmax A, operands prefetched,
    #  prefetch for the next iteration)
    variants = [("first", 0, True, None, False, "plain", False, True),
                ("firstm", 0, True, None, False, "masked", False, False),
                ("st0", 0, True, "plain", True, "plain", True, True),
                ("st1", 1, True, "plain", True, "plain", True, True),
                ("last0", 0, True, "plain", True, "masked", True, False),
                ("last1", 1, True, "plain", True, "masked", True, False),
                ("tail0", 0, False, "masked", True, None, False, False),
                ("tail1", 1, False, "masked", True, None, False, False)]
    counted = prog.label("counted")
    for name, p, do_s, sm_b, do_pv, sm_a, pre, pre_next in variants:
        e(f"{labs[name]}:")
        e(*iteration(prog, p, do_s, sm_b, do_pv, sm_a, pre, pre_next))
        if name in ("st0", "st1"):
            # steady state: while the next iteration is steady too, open it
            # here and go straight to its code (the other parity)
            e(*mark("idle"), f"s_add_u32 {s(SI)}, {s(SI)}, 1",
              f"s_cmp_lt_i32 {s(SI)}, %[jlast]", f"s_cbranch_scc0 {counted}",
              *opening(), *mark("loads"), f"s_branch {labs['st1' if name == 'st0' else 'st0']}")
        else:
            e(f"s_branch {nxt}")
    for p in (0, 1):
        e(f"{labs['idle%d' % p]}:", *stage("K"), *stage("V"), f"s_branch {nxt}")
    e(f"{nxt}:", *mark("idle"), f"s_add_u32 {s(SI)}, {s(SI)}, 1",
      f"{counted}:", f"s_cmp_le_i32 {s(SI)}, %[nblk]", f"s_cbranch_scc1 {top}")
    e(f"{done}:")

    # epilogue: O = acc / l (bf16), LSE = (m + log2 le) * ln 2; rows past N and
    # lanes of the upper half (LSE) address past the buffer ranges
    e("s_waitcnt vmcnt(0) lgkmcnt(0)", "s_nop 15", "s_nop 15", "s_nop 15")
    e(f"s_mov_b32 {s(SQ)}, %[olo]", f"s_and_b32 {s(SQ + 1)}, %[ohi], 0xffff",
      f"s_mov_b32 {s(SQ + 2)}, %[qbytes]", f"s_mov_b32 {s(SQ + 3)}, 0x20000")
    if PROF:
        e(*mark("epi"), "s_sub_u32 s89, s90, s96")
        for i in range(len(PROF_BUCKETS)):
            e(f"v_mov_b32_e32 {v(T)}, s{82 + i}",
              f"buffer_store_dword {v(T)}, %[dbg], {s(SQ, 4)}, 0 offen offset:{i * 256}")
        e("s_waitcnt vmcnt(0)")
        return prog
    if debug:
        # register dump (debug builds only): the listed VGPRs, then a[0:127]
        e(f"s_mov_b32 {s(SI + 1)}, 0")
        for r in DEBUG_VGPRS:
            e(f"buffer_store_dword {v(r)}, %[dbg], {s(SQ, 4)}, {s(SI + 1)} offen",
              f"s_add_u32 {s(SI + 1)}, {s(SI + 1)}, 256")
        for r in range(128):
            e(f"v_accvgpr_read_b32 {v(T)}, {a(r)}", "s_nop 1",
              f"buffer_store_dword {v(T)}, %[dbg], {s(SQ, 4)}, {s(SI + 1)} offen",
              f"s_add_u32 {s(SI + 1)}, {s(SI + 1)}, 256", "s_waitcnt vmcnt(0)")
        e("s_waitcnt vmcnt(0)")
        return prog
    for t, tile in enumerate(("A", "B")):
        t0, t1, t2, t3, t4 = T, T + 1, T + 2, T + 3, T + 4
        e("s_nop 2", f"v_add_f32_e32 {v(t0)}, {v(LV[tile][0])}, {v(LV[tile][1])}",
          f"v_mov_b32_e32 {v(t1)}, {v(t0)}", "s_nop 1",
          f"v_permlane32_swap_b32_e32 {v(t0)}, {v(t1)}", "s_nop 1",
          f"v_add_f32_e32 {v(t0)}, {v(t0)}, {v(t1)}")              # l
        e(f"v_mov_b32_e32 {v(t2)}, {v(LE[tile])}", f"v_mov_b32_e32 {v(t3)}, {v(LE[tile])}",
          "s_nop 1",
          f"v_permlane32_swap_b32_e32 {v(t2)}, {v(t3)}",
          "s_nop 1",
          f"v_add_f32_e32 {v(t2)}, {v(t2)}, {v(t3)}",               # le
          f"v_rcp_f32_e32 {v(t4)}, {v(t0)}",
          f"v_cmp_lt_f32_e32 vcc, 0, {v(t0)}",
          f"v_cndmask_b32_e64 {v(t4)}, 0, {v(t4)}, vcc",            # 1/l or 0
          f"v_log_f32_e32 {v(t2)}, {v(t2)}",
          "s_nop 1",                                                # transcendental result
          f"v_add_f32_e32 {v(t2)}, {v(M[tile])}, {v(t2)}",
          f"v_mul_f32_e32 {v(t2)}, 0x3f317218, {v(t2)}",
          f"v_cndmask_b32_e32 {v(t2)}, {v(NINF)}, {v(t2)}, vcc",
          f"buffer_store_dword {v(t2)}, %[loff{t}], {s(SL, 4)}, 0 offen")
        oo = f"%[ooff{t}]"
        for dt in range(4):
            for q in range(4):
                base = 64 * t + 16 * dt + 4 * q   # scratch (S and P registers), distinct per store
                ar0 = ACC[tile] + 16 * dt + 4 * q
                regs = [base, base + 1, base + 2]
                e(f"v_accvgpr_read_b32 {v(regs[0])}, {a(ar0)}",
                  f"v_accvgpr_read_b32 {v(regs[1])}, {a(ar0 + 1)}",
                  f"v_mul_f32_e32 {v(regs[0])}, {v(t4)}, {v(regs[0])}",
                  f"v_mul_f32_e32 {v(regs[1])}, {v(t4)}, {v(regs[1])}",
                  f"v_cvt_pk_bf16_f32 {v(regs[0])}, {v(regs[0])}, {v(regs[1])}",
                  f"v_accvgpr_read_b32 {v(regs[1])}, {a(ar0 + 2)}",
                  f"v_accvgpr_read_b32 {v(regs[2])}, {a(ar0 + 3)}",
                  f"v_mul_f32_e32 {v(regs[1])}, {v(t4)}, {v(regs[1])}",
                  f"v_mul_f32_e32 {v(regs[2])}, {v(t4)}, {v(regs[2])}",
                  f"v_cvt_pk_bf16_f32 {v(regs[1])}, {v(regs[1])}, {v(regs[2])}",
                  f"buffer_store_dwordx2 {v(regs[0], 2)}, {oo}, {s(SQ, 4)}, 0 offen "
                  f"offset:{64 * dt + 16 * q}")
    e("s_waitcnt vmcnt(0)")
    return prog


TRANS = ("v_exp_f32", "v_log_f32", "v_rcp_f32")


def regs_read(ins):
    """VGPR numbers an instruction reads (sources only; rough but enough for
    the checks below)."""
    import re
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return set()
    ops = [o.strip() for o in parts[1].split(",")]
    srcs = ops[1:] if not parts[0].startswith(("buffer_store", "ds_write")) else ops
    out = set()
    for o in srcs:
        m = re.fullmatch(r"-?v(\d+)", o)
        if m:
            out.add(int(m.group(1)))
        m = re.fullmatch(r"v\[(\d+):(\d+)\]", o)
        if m:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def check_hazards(lines):
    """A transcendental result read by the very next instruction needs a wait
    state; fail generation if the schedule ever produces that."""
    for i in range(len(lines) - 1):
        a, b = lines[i], lines[i + 1]
        if a.startswith(TRANS):
            dst = int(a.split()[1].rstrip(",")[1:])
            if dst in regs_read(b):
                raise SystemExit(f"trans hazard at line {i}: {a!r} -> {b!r}")


def main():
    import sys
    global PROF
    debug = "--debug" in sys.argv
    PROF = "--profile" in sys.argv
    prog = build(debug)
    lines = prog.main + [f"s_branch .Lfaend_%="] + prog.cold + [".Lfaend_%=:"]
    check_hazards(lines)
    here = os.path.dirname(os.path.abspath(__file__))
    name = "fa_fwd_d128_loop_debug.inc" if (debug or PROF) else "fa_fwd_d128_loop.inc"
    if "--out" in sys.argv:
        here = sys.argv[sys.argv.index("--out") + 1]
    with open(os.path.join(here, name), "w") as f:
        f.write("// Generated by gen_fwd_d128_loop.py -- do not edit.\n")
        f.write(f"// {len(prog.main)} hot-path lines, {len(prog.cold)} out-of-line lines.\n")
        for ln in lines:
            f.write(f'"{ln}\\n"\n')
    cname = "fa_fwd_d128_clobbers_debug.inc" if (debug or PROF) else "fa_fwd_d128_clobbers.inc"
    with open(os.path.join(here, cname), "w") as f:
        f.write("// Generated by gen_fwd_d128_loop.py -- do not edit.\n")
        sg = SGPRS + (list(range(82, 98)) if PROF else [])
        names = [f'"v{i}"' for i in range(NVGPR)] + [f'"a{i}"' for i in range(NAGPR)] + \
                [f'"s{i}"' for i in sg] + ['"m0"', '"vcc"', '"scc"', '"memory"']
        for i in range(0, len(names), 16):
            f.write(", ".join(names[i:i + 16]) + ("," if i + 16 < len(names) else "") + "\n")


if __name__ == "__main__":
    main()
