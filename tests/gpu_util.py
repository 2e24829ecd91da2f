"""Helpers shared by the GPU parity tests (upload, run, compare)."""
import sys

import numpy as np

from fa_inputs import bf16_bits_to_f32

# Tolerances.  fp32: O max-abs 1e-4.  bf16 inputs with fp32 accumulation:
# O max-abs 1e-2 and relative Frobenius 5e-3.  LSE: 1e-4 (fp32) and 1e-3
# (bf16); rows with no visible key must give LSE = -inf and O = 0 exactly.
TOL = {
    "f32": {"o_abs": 1e-4, "o_relf": None, "lse_abs": 1e-4},
    "bf16": {"o_abs": 1e-2, "o_relf": 5e-3, "lse_abs": 1e-3},
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(x, scale, mask_kind, sentinel=True):
    """Upload generated inputs, run the matching entry point, return fp64 O, LSE."""
    import torch

    import exact_attention_92_amd as fa
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    kv = None
    if x.get("kv_lens") is not None:
        kv = torch.from_numpy(np.asarray(x["kv_lens"], dtype=np.int32)).cuda()
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if sentinel:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    fn = fa.fa_fwd if q.dtype == torch.bfloat16 else fa.fa_fwd_f32
    fn(q, k, v, o, lse, scale, mask_kind, kv)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def o_to_f64(o):
    import torch
    if o.dtype == torch.bfloat16:
        bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return o.cpu().numpy().astype(np.float64)


def compare(O, L, Or, Lr, dtype, what=""):
    """Assert parity of O and LSE against the oracle; returns the error stats."""
    tol = TOL[dtype]
    assert not np.isnan(O).any(), f"{what}: O has unwritten (NaN) elements"
    assert not np.isnan(L).any(), f"{what}: LSE has unwritten (NaN) elements"
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty), f"{what}: LSE -inf pattern differs"
    if empty.any():
        assert np.all(L[empty] == -np.inf) and np.all(O[empty] == 0.0), f"{what}: empty rows"
    err = np.abs(O - Or)
    stats = {"o_abs": float(err.max(initial=0.0))}
    nrm = np.linalg.norm(Or)
    stats["o_relf"] = float(np.linalg.norm(O - Or) / nrm) if nrm > 0 else 0.0
    stats["lse_abs"] = float(np.abs(L[~empty] - Lr[~empty]).max(initial=0.0))
    def room(k):   # share of the bar still unused (negative: over the bar)
        return "" if tol[k] is None else f" ({100.0 * (1.0 - stats[k] / tol[k]):.0f}% headroom)"
    say(f"  {what}: max|dO|={stats['o_abs']:.3e}{room('o_abs')} "
        f"relF={stats['o_relf']:.3e}{room('o_relf')} "
        f"max|dLSE|={stats['lse_abs']:.3e}{room('lse_abs')}")
    assert stats["o_abs"] <= tol["o_abs"], (what, stats)
    if tol["o_relf"] is not None:
        assert stats["o_relf"] <= tol["o_relf"], (what, stats)
    assert stats["lse_abs"] <= tol["lse_abs"], (what, stats)
    return stats


# Backward tolerances (bf16 inputs, fp32 accumulation), per element: the
# standard bound for a rounded sum of products, |err| <= k u (A + |ref|),
# with u = 2^-8 the bf16 unit roundoff and A the sum of the absolute values
# of the terms (the oracle's magnitudes).  The kernel rounds one factor of
# every term to bf16 (P for dV, dS for dQ and dK: relative error <= u), the
# row sum D inherits the bf16 rounding of O (magnitude terms of the oracle
# carry it into dS), and the result is rounded once more (u |ref|); fp32
# accumulation and the exp2/LSE errors are ~1e-6 relative, far below u.
# k = 2 covers these with room.  An element whose terms are all zero (a key
# nobody sees, a row that sees nothing) must come out exactly 0.  On the
# named workloads (millions of elements, little cancellation in bulk) each
# tensor's relative Frobenius error must also stay below 1e-2: independent
# roundings give ~u/sqrt(3) ~ 2.3e-3 each, adding in quadrature.  Tiny cases
# can be dominated by cancellation (two visible keys: dS_0 = -dS_1), where
# that ratio says nothing and the element bound alone applies.
U_BF16 = 2.0 ** -8
TOL_BWD = {"k": 2.0, "relf": 1e-2}


def run_bwd_gpu(x, scale, mask_kind, sentinel=True):
    """Forward then backward on the GPU; returns fp64 dq, dk, dv, dp_rowsum
    (and the forward's O, LSE)."""
    import torch

    import exact_attention_92_amd as fa
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    kv = None
    if x.get("kv_lens") is not None:
        kv = torch.from_numpy(np.asarray(x["kv_lens"], dtype=np.int32)).cuda()
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa.fa_fwd(q, k, v, o, lse, scale, mask_kind, kv)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dps = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if sentinel:
        for t in (dq, dk, dv, dps):
            t.fill_(float("nan"))
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dps, scale, mask_kind, kv)
    torch.cuda.synchronize()
    return {"dq": o_to_f64(dq), "dk": o_to_f64(dk), "dv": o_to_f64(dv),
            "dps": dps.cpu().numpy().astype(np.float64),
            "o": o_to_f64(o), "lse": lse.cpu().numpy().astype(np.float64)}


def compare_grads(g, ref, mag, what="", keys=("dq", "dk", "dv"), bulk=False):
    """Assert backward parity of ``g`` against fp64 ``ref`` with the
    per-element bound above (``mag``: the oracle's magnitudes)."""
    stats = {}
    for name in keys:
        got, want, a = g[name], ref[name], mag[name]
        assert not np.isnan(got).any(), f"{what}: {name} has unwritten (NaN) elements"
        assert not np.isnan(want).any() and not np.isnan(a).any(), f"{what}: {name} reference"
        err = np.abs(got - want)
        bound = TOL_BWD["k"] * U_BF16 * (a + np.abs(want))
        zero = bound == 0
        assert np.all(err[zero] == 0.0), (what, name, "elements with no terms must be 0")
        ratio = float(np.max(err[~zero] / bound[~zero], initial=0.0))
        nrm = float(np.linalg.norm(want))
        relf = float(np.linalg.norm(got - want) / nrm) if nrm > 0 else 0.0
        stats[name] = (relf, ratio)
        assert ratio <= 1.0, (what, name, "element bound", stats[name])
        if bulk:
            assert relf <= TOL_BWD["relf"], (what, name, "relative Frobenius", stats[name])
    say(f"  {what}: " + " ".join(f"{n}: relF={a:.2e} err/bound={b:.2f}"
                                 for n, (a, b) in stats.items()))
    return stats


def compare_bound(O, L, ref, what):
    """Element-wise parity of a bf16 forward with probabilities rounded to
    bf16: |err| <= 2^-8 |O_ref| (O's own rounding) + (2^-7 + 1e-5) (P|V|)
    (P rounded to bf16 and normalised by the sum of the rounded values, fp32
    sums), relative Frobenius <= 5e-3, LSE within 1e-3; rows without a
    visible key exactly O = 0, LSE = -inf; no unwritten (NaN) element.
    ``ref`` is (O_ref, LSE_ref, P|V|) from the oracle's ``magnitudes``; O is
    laid out as LSE's rows followed by d."""
    Or, Lr, M = ref
    assert not np.isnan(O).any() and not np.isnan(L).any(), f"{what}: unwritten elements"
    empty = ~np.isfinite(Lr)
    assert np.array_equal(~np.isfinite(L), empty), f"{what}: LSE -inf pattern"
    assert np.all(O[empty] == 0.0) and np.all(L[empty] == -np.inf), f"{what}: empty rows"
    err = np.abs(O - Or)
    bound = 2.0 ** -8 * np.abs(Or) + (2.0 ** -7 + 1e-5) * M
    zero = bound == 0
    assert np.all(err[zero] == 0.0), what
    ratio = float(np.max(err[~zero] / bound[~zero], initial=0.0))
    nrm = np.linalg.norm(Or)
    relf = float(np.linalg.norm(O - Or) / nrm) if nrm > 0 else 0.0
    lerr = float(np.abs(L[~empty] - Lr[~empty]).max(initial=0.0))
    say(f"  {what}: err/bound={ratio:.2f} relF={relf:.2e} max|dLSE|={lerr:.2e}")
    assert ratio <= 1.0 and relf <= 5e-3 and lerr <= 1e-3, (what, ratio, relf, lerr)
