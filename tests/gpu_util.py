"""Helpers for the GPU parity tests: numpy <-> torch device tensors and the comparison rules."""
from __future__ import annotations

import numpy as np
import torch

POISON = 0xFFFF  # BF16 bit pattern (a NaN) written into outputs before a call
TOL = 5e-3       # max|gpu - oracle| / max|oracle| per expert block


def dev():
    return torch.device("cuda:0")


def u16(a: np.ndarray) -> torch.Tensor:
    """BF16 bits (uint16) -> bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 numpy bits (synchronises)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def poison_bf16(rows: int, cols: int) -> torch.Tensor:
    return torch.full((rows, cols), -1, dtype=torch.int16, device=dev()).view(torch.bfloat16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_gemm(got_bits: np.ndarray, ref_acc: np.ndarray, topk_flat: np.ndarray, E: int, rows=None,
               tol: float = TOL, label: str = ""):
    """Per expert block: max|gpu - oracle| / max|oracle| <= tol over the expert's checked rows (all N
    columns); an all-zero oracle block needs an all-zero GPU block.  Rows of invalid routes must still be
    poison.  ``rows`` restricts the check to the listed route indices (sampled checking)."""
    ids = np.asarray(topk_flat).reshape(-1)
    R = ids.size
    valid = (ids >= 0) & (ids < E)
    check_rows = np.arange(R) if rows is None else np.asarray(rows)
    worst = 0.0
    for e in np.unique(ids[check_rows][valid[check_rows]]):
        rr = check_rows[ids[check_rows] == e]
        g = bf16_to_f64(got_bits[rr])
        r = ref_acc[rr]
        assert not np.any(np.isnan(g)), "%s expert %d: unwritten (poison) output in a routed row" % (label, e)
        den = np.abs(r).max()
        if den == 0:
            assert np.all(g == 0), "%s expert %d: oracle block is zero, GPU is not" % (label, e)
            continue
        ratio = np.abs(g - r).max() / den
        worst = max(worst, ratio)
        assert ratio <= tol, "%s expert %d: error ratio %.3g > %.3g" % (label, e, ratio, tol)
    inv = check_rows[~valid[check_rows]]
    if inv.size:
        assert np.all(got_bits[inv] == POISON), "%s: a row of a non-local route was written" % label
    return worst


def silu(g):
    return g / (1.0 + np.exp(-g))


def check_act(got_bits: np.ndarray, gu_ref: np.ndarray, topk_flat: np.ndarray, E: int, rows=None,
              tol: float = TOL, label: str = ""):
    """SiLU*mul output h against the oracle's binary64 gate/up accumulators gu_ref [R, 2I].

    The bar follows from the GEMM bar: per expert block the gate and up values may each be off by
    dg = tol * max|g| and du = tol * max|u| (max over the block), and silu has slope at most 1.1, so
        |h - silu(g) u| <= 1.1 |u| dg + (|silu(g)| + 1.1 dg) du + 2^-8 |h|
    elementwise, the last term being the BF16 rounding of h.  A gate/up column mix-up or a wrong row
    exceeds it by about 1/tol.  Rows of non-local routes must keep their poison."""
    ids = np.asarray(topk_flat).reshape(-1)
    R = ids.size
    I = gu_ref.shape[1] // 2
    valid = (ids >= 0) & (ids < E)
    check_rows = np.arange(R) if rows is None else np.asarray(rows)
    worst = 0.0
    for e in np.unique(ids[check_rows][valid[check_rows]]):
        rr = check_rows[ids[check_rows] == e]
        g, u = gu_ref[rr, :I], gu_ref[rr, I:]
        h = bf16_to_f64(got_bits[rr])
        assert not np.any(np.isnan(h)), "%s expert %d: unwritten (poison) output in a routed row" % (label, e)
        dg, du = tol * np.abs(g).max(), tol * np.abs(u).max()
        ref = silu(g) * u
        bound = 1.1 * np.abs(u) * dg + (np.abs(silu(g)) + 1.1 * dg) * du + 2.0 ** -8 * np.abs(ref) + 1e-30
        err = np.abs(h - ref)
        worst = max(worst, float((err / bound).max()))
        assert np.all(err <= bound), "%s expert %d: activation error beyond the derived bound (worst %.3g x)" % (
            label, e, (err / bound).max())
    inv = check_rows[~valid[check_rows]]
    if inv.size:
        assert np.all(got_bits[inv] == POISON), "%s: a row of a non-local route was written" % label
    return worst


# Fused expert MLP bar, per token t: max|gpu - oracle| <= FUSED_TOL * S_t with S_t = sum_j |tw[t,j]| * max|y_j|
# over the token's valid routes j (y_j: the oracle's binary32 down-projection row of route t*k + j).  S_t is the
# scale the token's weighted sum is built from: the combine adds the routes' errors with weights tw, so
# normalising by max|out_t| instead would make the bar depend on how far the k weighted rows cancel.  Derived
# from the GEMM bar (5e-3 of an output's scale, BF16 output rounding included): the GPU's y_j is the down GEMM's
# BF16 output, so it carries that GEMM's own error with its rounding (at most 5e-3) plus the gate_up error passed
# on through h (silu*mul has slope of about 1, the down GEMM is linear; at most 5e-3), and the single BF16
# rounding of the output adds at most 2^-9 |out_t| <= 2^-9 S_t.  The oracle keeps y binary32.
FUSED_TOL = 1e-2 + 2.0 ** -9


def check_fused(got_bits: np.ndarray, out_acc: np.ndarray, y: np.ndarray, tw: np.ndarray, ids: np.ndarray, E: int,
                tol: float = FUSED_TOL, label: str = ""):
    """Fused MLP output [T,H] (BF16 bits) against the oracle's combine accumulators out_acc [T,H] (before the
    final rounding) to the bar above; tokens without a valid route must be all zero.  Returns (worst error /
    S_t, worst error / max|out_t|), the second only reported."""
    ids = np.asarray(ids)
    T, k = ids.shape
    g = bf16_to_f64(got_bits)
    worst, worst_plain = 0.0, 0.0
    for t in range(T):
        valid = (ids[t] >= 0) & (ids[t] < E)
        if not valid.any():
            assert np.all(got_bits[t] == 0), "%s token %d without a local route must be zero" % (label, t)
            continue
        scale = sum(abs(float(tw[t, j])) * np.abs(y[t * k + j]).max() for j in range(k) if valid[j])
        err = np.abs(g[t] - out_acc[t]).max()
        if scale == 0.0:
            assert err == 0.0, "%s token %d" % (label, t)
            continue
        ratio = err / scale
        worst = max(worst, ratio)
        den = np.abs(out_acc[t]).max()
        if den > 0:
            worst_plain = max(worst_plain, err / den)
        assert ratio <= tol, "%s token %d: error %.3g of S_t (bar %.3g)" % (label, t, ratio, tol)
    return worst, worst_plain
