"""Seeded synthetic inputs for the W4A16 MoE grouped GEMM.

This module holds input generation only: random draws, the shapes of the
workloads, and routing draws.  It contains none of the method's arithmetic
(no dequantisation, no routing preparation, no products), so the oracle and
the HIP library can both consume its outputs without sharing code.  Random
values are rounded to BF16 by torch's own dtype cast.

Draw recipe (one ``numpy.random.default_rng(seed)`` per workload):
  x      ~ N(0, 1), rounded to BF16;
  codes  uniform integers 0..15, one per byte (upper nibble zero);
  scales uniform in [0.005, 0.02], rounded to BF16;
  routes distinct experts per token, uniform (or as each workload states).

All arrays are numpy; BF16 values are carried as their uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED_BASE = 20260


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float values to BF16 with torch's cast; return uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rng_for(cfg_index: int, salt: int = 0) -> np.random.Generator:
    return np.random.default_rng(SEED_BASE + cfg_index + 1000 * salt)


def activations(rng: np.random.Generator, rows: int, K: int) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal((rows, K), dtype=np.float32))


def codes(rng: np.random.Generator, E: int, N: int, K: int) -> np.ndarray:
    return rng.integers(0, 16, size=(E, N, K), dtype=np.uint8)


def scales(rng: np.random.Generator, E: int, N: int, K: int, lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    assert K % 32 == 0
    return to_bf16_bits(rng.uniform(lo, hi, size=(E, N, K // 32)).astype(np.float32))


def mxfp4_scales(rng: np.random.Generator, E: int, N: int, K: int, lo: int = 118, hi: int = 126) -> np.ndarray:
    """E8M0 scale bytes uniform in [lo, hi] (2^-9 .. 2^-1 by default): uint8 [E,N,K/32]."""
    return rng.integers(lo, hi + 1, (E, N, K // 32), dtype=np.uint8)


def uniform_topk(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """Distinct experts per token, uniform without replacement: int32 [T, k]."""
    if T == 0:
        return np.zeros((0, k), np.int32)
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)


def local_share(global_ids: np.ndarray, local_experts: int) -> np.ndarray:
    """Expert-parallel share of one GPU: global ids below ``local_experts`` stay, others become -1."""
    out = global_ids.astype(np.int32).copy()
    out[out >= local_experts] = -1
    return out


def zipf_local_topk(rng: np.random.Generator, T: int, k: int, n_global: int = 384, n_local: int = 48,
                    s: float = 1.1, forced_empty: int = 4) -> np.ndarray:
    """Skewed prefill routing for one GPU's share of experts.

    Global expert popularity is (1 + rank)^-s.  Local expert j gets rank
    8j + 4 (a stratified eighth of the popularity range); the other ranks go to
    the non-local experts in a seeded permutation.  The last ``forced_empty``
    local experts get weight 0.  Each token draws k distinct experts by
    weighted sampling without replacement (Efraimidis-Spirakis keys
    u^(1/w), largest k).  Returns int32 [T, k] with non-local routes as -1.
    """
    stride = n_global // n_local
    ranks = np.empty(n_global, np.int64)
    local_ranks = stride * np.arange(n_local) + stride // 2
    ranks[:n_local] = local_ranks
    others = np.setdiff1d(np.arange(n_global), local_ranks)
    ranks[n_local:] = rng.permutation(others)
    w = (1.0 + ranks.astype(np.float64)) ** (-s)
    if forced_empty:
        w[n_local - forced_empty:n_local] = 0.0
    u = rng.random((T, n_global))
    with np.errstate(divide="ignore"):
        keys = np.where(w > 0, np.log(u) / np.where(w > 0, w, 1.0), -np.inf)
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return local_share(ids, n_local)


def softmax_topk_router(rng: np.random.Generator, T: int, E: int, k: int):
    """Router of the fused MLP workload: BF16 logits ~N(0,1) [T,E] -> fp32 softmax -> top-k (ties to the
    lower index) -> weights renormalised to sum 1.  Returns (ids int32 [T,k], weights float32 [T,k])."""
    import torch

    logits = torch.from_numpy(rng.standard_normal((T, E), dtype=np.float32)).to(torch.bfloat16).float()
    probs = torch.softmax(logits, dim=-1)
    # stable descending sort keeps the lower index first among equal probabilities
    order = torch.sort(probs, dim=-1, descending=True, stable=True).indices[:, :k]
    w = torch.gather(probs, 1, order)
    w = w / w.sum(dim=-1, keepdim=True)
    return order.to(torch.int32).numpy(), w.to(torch.float32).numpy()


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass
class GemmCase:
    """One grouped-GEMM problem: A rows, expert weights, routes."""
    name: str
    A: np.ndarray          # uint16 bf16 bits [rows, K]
    a_row_div: int         # route i reads A row i // a_row_div
    codes: np.ndarray      # uint8 [E, N, K]
    scales: np.ndarray     # uint16 bf16 bits [E, N, K/32]
    topk_ids: np.ndarray   # int32 [T, k]

    @property
    def E(self):
        return self.codes.shape[0]

    @property
    def N(self):
        return self.codes.shape[1]

    @property
    def K(self):
        return self.codes.shape[2]


def tiny_case(seed_salt: int = 0) -> GemmCase:
    """16 tokens, 8 experts, top-2 distinct uniform; W 512x256; x [16,256]; out [32,512]."""
    r = rng_for(1, seed_salt)
    T, E, k, N, K = 16, 8, 2, 512, 256
    ids = uniform_topk(r, T, E, k)
    return GemmCase("tiny", activations(r, T, K), k, codes(r, E, N, K), scales(r, E, N, K), ids)


def qwen3_routes(T: int, seed_salt: int = 0) -> np.ndarray:
    return uniform_topk(rng_for(2, seed_salt + 10 + T), T, 128, 8)


def kimi_decode_routes(T: int, seed_salt: int = 0) -> np.ndarray:
    g = uniform_topk(rng_for(3, seed_salt + 10 + T), T, 384, 8)
    return local_share(g, 48)


def kimi_prefill_routes(T: int = 8192, seed_salt: int = 0) -> np.ndarray:
    return zipf_local_topk(rng_for(4, seed_salt), T, 8)


def deepseek_router(T: int, seed_salt: int = 0):
    return softmax_topk_router(rng_for(5, seed_salt + 10 + T), T, 256, 8)


def expert_weights(cfg_index: int, E: int, N: int, K: int, salt: int = 0):
    r = rng_for(cfg_index, 100 + salt)
    return codes(r, E, N, K), scales(r, E, N, K)


def integer_exact_case(rng: np.random.Generator, T: int, E: int, k: int, N: int, K: int):
    """Inputs whose every partial sum is exact in binary32: scale 2^-4, x in {-2..2}, codes 0..15."""
    x = to_bf16_bits(rng.integers(-2, 3, size=(T, K)).astype(np.float32))
    c = codes(rng, E, N, K)
    s = np.full((E, N, K // 32), 0x3D80, np.uint16)  # bf16 bits of 2^-4
    ids = uniform_topk(rng, T, E, k)
    return x, c, s, ids


def codes_device(seed: int, E: int, N: int, K: int, device):
    """Seeded codes generated on the GPU (for weight sets too large to draw on the host): uint8 [E,N,K]."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(0, 16, (E, N, K), dtype=torch.uint8, device=device, generator=g)


def mxfp4_scales_device(seed: int, E: int, N: int, K: int, device, lo: int = 118, hi: int = 126):
    """Seeded E8M0 scale bytes uniform in [lo, hi] generated on the GPU: uint8 [E,N,K/32]."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, (E, N, K // 32), dtype=torch.uint8, device=device, generator=g)


def scales_device(seed: int, E: int, N: int, K: int, device, lo: float = 0.005, hi: float = 0.02):
    """Seeded BF16 scales uniform in [lo, hi] generated on the GPU: bfloat16 [E,N,K/32]."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    u = torch.rand((E, N, K // 32), dtype=torch.float32, device=device, generator=g)
    return (lo + (hi - lo) * u).to(torch.bfloat16)
