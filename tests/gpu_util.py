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
