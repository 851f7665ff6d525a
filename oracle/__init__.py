"""Plain CPU oracle for the W4A16 MoE grouped GEMM -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does: it
shares no code with the oracle, and the oracle shares none with it.

The arithmetic lives in ``w4a16_oracle.c`` (plain loops, binary32 or binary64
accumulation, compiled with ``-O2 -ffp-contract=off`` so no multiply-add is
fused).  This module only marshals numpy arrays into it.  Definitions and the
passages they follow are in the C file's header:

* MXFP4 weights ``w = e2m1(c) * 2^(e - 127)`` with one E8M0 scale per 32 k --
  b12x page ("local-inference-lab/b12x pull 479", "Summary") and humans& page
  ("BF16 preserves each local product"), value sets of the OCP formats;
* dequantisation ``w = (q - 8) * s`` with one BF16 scale per 32 k -- Chord page
  ("vLLM x Novita AI: Chord, Faster INT4 MoE for Kimi K2.x"), sections
  "Grouped SM90 kernels" and "H200 and Blackwell indexed decode";
* per-expert product ``out[rows of e] = x[rows of e] @ W[e]^T`` --
  "LegumMagister/nf4-grouped-gemm", section "Usage";
* indexed routing tensors -- Chord page, "Two kernel families", Figure 3;
* fused expert MLP -- humans& page, "Dedicated warps keep the pipeline busy".

Every function here is pinned by ``tests/test_oracle_*.py`` against values
fixed by the definitions and by mathematics (exact rationals, hand-computed
cases, closed forms and invariants), not against itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fused multiply-add, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_oracle(_SRC, _LIB)
    return _LIB


def _bind(lib):
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_bf16_rne.argtypes = [ctypes.c_float]
    lib.orc_bf16_rne_f64.restype = ctypes.c_uint16
    lib.orc_bf16_rne_f64.argtypes = [ctypes.c_double]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_dequant_one.restype = ctypes.c_float
    lib.orc_dequant_one.argtypes = [ctypes.c_uint8, ctypes.c_uint16]
    lib.orc_dequant.restype = None
    lib.orc_dequant.argtypes = [_P, _P, _I, _I, _P, _P]
    lib.orc_route_bounds.restype = None
    lib.orc_route_bounds.argtypes = [_I, _I, _I, _I, _P, _P]
    lib.orc_route_prep.restype = _I
    lib.orc_route_prep.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
    lib.orc_grouped_gemm.restype = None
    lib.orc_grouped_gemm.argtypes = [_P, _I, _P, _P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _I, _I]
    lib.orc_silu.restype = ctypes.c_double
    lib.orc_silu.argtypes = [ctypes.c_double]
    lib.orc_silu_mul.restype = None
    lib.orc_silu_mul.argtypes = [_P, _I, _I, _P]
    lib.orc_combine.restype = None
    lib.orc_combine.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P]
    lib.orc_fused_moe.restype = _I
    lib.orc_fused_moe.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I]
    lib.orc_e2m1.restype = ctypes.c_float
    lib.orc_e2m1.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0.restype = ctypes.c_float
    lib.orc_e8m0.argtypes = [ctypes.c_uint8]
    lib.orc_dequant_mxfp4_one.restype = ctypes.c_float
    lib.orc_dequant_mxfp4_one.argtypes = [ctypes.c_uint8, ctypes.c_uint8]
    lib.orc_dequant_mxfp4.restype = None
    lib.orc_dequant_mxfp4.argtypes = [_P, _P, _I, _I, _P, _P]
    lib.orc_grouped_gemm_fmt.restype = None
    lib.orc_grouped_gemm_fmt.argtypes = [_P, _I, _P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _I, _I]
    lib.orc_fused_moe_fmt.restype = _I
    lib.orc_fused_moe_fmt.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I]
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return os.cpu_count() or 1


class Oracle:
    """The oracle's functions bound to one compiled copy of ``w4a16_oracle.c``."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        self.lib = _bind(ctypes.CDLL(lib_path))

    # ------------------------------------------------------------ scalars
    def bf16_rne(self, f: float) -> int:
        """Round a binary32 value to BF16 bits (nearest, ties to even)."""
        return int(self.lib.orc_bf16_rne(float(np.float32(f))))

    def bf16_rne_f64(self, d: float) -> int:
        """Round a binary64 value to BF16 bits in one step."""
        return int(self.lib.orc_bf16_rne_f64(float(d)))

    def bf16_to_f32(self, h: int) -> float:
        return float(self.lib.orc_bf16_to_f32(int(h)))

    def dequant_one(self, code: int, scale_bf16: int) -> float:
        return float(self.lib.orc_dequant_one(int(code), int(scale_bf16)))

    def silu(self, g: float) -> float:
        return float(self.lib.orc_silu(float(g)))

    def e2m1(self, code: int) -> float:
        return float(self.lib.orc_e2m1(int(code)))

    def e8m0(self, e: int) -> float:
        return float(self.lib.orc_e8m0(int(e)))

    def dequant_mxfp4_one(self, code: int, scale_e8m0: int) -> float:
        return float(self.lib.orc_dequant_mxfp4_one(int(code), int(scale_e8m0)))

    def dequant_mxfp4(self, codes: np.ndarray, scales: np.ndarray):
        """One MXFP4 expert: codes uint8 [N,K], E8M0 scales uint8 [N,K/32] -> (f32 [N,K], bf16 bits [N,K])."""
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.uint8)
        N, K = codes.shape
        assert K % 32 == 0 and scales.shape == (N, K // 32)
        f = np.empty((N, K), np.float32)
        b = np.empty((N, K), np.uint16)
        self.lib.orc_dequant_mxfp4(_ptr(codes), _ptr(scales), N, K, _ptr(f), _ptr(b))
        return f, b

    # ------------------------------------------------------------ arrays
    def dequant(self, codes: np.ndarray, scales: np.ndarray):
        """One expert: codes uint8 [N,K], scales bf16 bits [N,K/32] -> (f32 [N,K], bf16 bits [N,K])."""
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.uint16)
        N, K = codes.shape
        assert K % 32 == 0 and scales.shape == (N, K // 32)
        f = np.empty((N, K), np.float32)
        b = np.empty((N, K), np.uint16)
        self.lib.orc_dequant(_ptr(codes), _ptr(scales), N, K, _ptr(f), _ptr(b))
        return f, b

    def route_bounds(self, T: int, k: int, E: int, block_m: int):
        mp = ctypes.c_int(0)
        mb = ctypes.c_int(0)
        self.lib.orc_route_bounds(T, k, E, block_m, ctypes.byref(mp), ctypes.byref(mb))
        return mp.value, mb.value

    def route_prep(self, topk_ids: np.ndarray, E: int, block_m: int):
        """topk_ids int32 [T,k] -> dict(sorted_ids, expert_ids, num_tokens_padded, expert_offsets, counts)."""
        ids = _c(topk_ids, np.int32)
        T, k = ids.shape
        maxP, maxB = self.route_bounds(T, k, E, block_m)
        sorted_ids = np.empty(max(maxP, 1), np.int32)
        expert_ids = np.empty(max(maxB, 1), np.int32)
        ntp = np.zeros(1, np.int32)
        offs = np.empty(E + 1, np.int32)
        counts = np.empty(max(E, 1), np.int32)
        rc = self.lib.orc_route_prep(_ptr(ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(expert_ids),
                                     _ptr(ntp), _ptr(offs), _ptr(counts))
        assert rc == 0
        return dict(sorted_ids=sorted_ids[:maxP], expert_ids=expert_ids[:maxB],
                    num_tokens_padded=int(ntp[0]), expert_offsets=offs, counts=counts[:E])

    def grouped_gemm(self, A, a_row_div: int, codes, scales, topk_ids, acc64: bool = False, rows=None,
                     nthreads: int | None = None, fmt: str = "int4"):
        """out[i,:] = bf16(sum_k A[i//a_row_div,k] * w[e(i),:,k]) for every valid route i.

        A bf16 bits [*,K]; codes uint8 [E,N,K]; scales [E,N,K/32]: bf16 bits (fmt "int4") or E8M0 bytes
        (fmt "mxfp4"); topk_ids int32 (any shape, flattened to R).  Returns (acc float64 [R,N], NaN where not
        computed; out bf16 bits [R,N], 0xFFFF where not computed).  ``rows`` restricts the work to the listed
        route indices.
        """
        A = _c(A, np.uint16)
        codes = _c(codes, np.uint8)
        fcode = {"int4": 0, "mxfp4": 1}[fmt]
        scales = _c(scales, np.uint16 if fcode == 0 else np.uint8)
        ids = _c(topk_ids, np.int32).reshape(-1)
        E, N, K = codes.shape
        assert A.ndim == 2 and A.shape[1] == K and scales.shape == (E, N, K // 32)
        R = ids.size
        acc = np.full((R, N), np.nan, np.float64)
        out = np.full((R, N), 0xFFFF, np.uint16)
        rows_arr = None if rows is None else _c(rows, np.int32)
        self.lib.orc_grouped_gemm_fmt(_ptr(A), a_row_div, _ptr(codes), _ptr(scales), fcode, E, N, K, _ptr(ids), R,
                                      1 if acc64 else 0, _ptr(acc), _ptr(out), _ptr(rows_arr),
                                      0 if rows_arr is None else rows_arr.size, nthreads or default_threads())
        return acc, out

    def silu_mul(self, gu: np.ndarray):
        """gu float64 [rows, 2I] (pre-rounding values) -> h bf16 bits [rows, I]."""
        gu = _c(gu, np.float64)
        rows, two_i = gu.shape
        h = np.empty((rows, two_i // 2), np.uint16)
        self.lib.orc_silu_mul(_ptr(gu), rows, two_i // 2, _ptr(h))
        return h

    def combine(self, y, tw, topk_ids, E: int, with_acc: bool = False):
        """y float64 [T*k,H] (binary32 values), tw float32 [T,k], ids int32 [T,k] -> bf16 bits [T,H]
        (and, with ``with_acc``, the binary32 accumulators before rounding as float64 [T,H])."""
        y = _c(y, np.float64)
        tw = _c(tw, np.float32)
        ids = _c(topk_ids, np.int32)
        T, k = ids.shape
        H = y.shape[1]
        out = np.empty((T, H), np.uint16)
        acc = np.empty((T, H), np.float64)
        self.lib.orc_combine(_ptr(y), _ptr(tw), _ptr(ids), T, k, E, H, _ptr(out), _ptr(acc))
        return (out, acc) if with_acc else out

    def fused_moe(self, x, topk_ids, tw, c13, s13, c2, s2, nthreads: int | None = None, fmt: str = "int4"):
        """Fused expert MLP; returns (out bf16 bits [T,H], h bf16 bits [R,I], y float64 [R,H]).  Scales as in
        ``grouped_gemm`` for ``fmt``.

        ``self.last_out_acc`` then holds the combine's binary32 accumulators before rounding [T,H]."""
        x = _c(x, np.uint16)
        ids = _c(topk_ids, np.int32)
        tw = _c(tw, np.float32)
        fcode = {"int4": 0, "mxfp4": 1}[fmt]
        sdt = np.uint16 if fcode == 0 else np.uint8
        c13, s13 = _c(c13, np.uint8), _c(s13, sdt)
        c2, s2 = _c(c2, np.uint8), _c(s2, sdt)
        T, k = ids.shape
        E, two_i, H = c13.shape
        I = two_i // 2
        assert c2.shape == (E, H, I) and x.shape == (T, H)
        R = T * k
        out = np.empty((T, H), np.uint16)
        out_acc = np.empty((T, H), np.float64)
        h = np.zeros((R, I), np.uint16)
        y = np.zeros((R, H), np.float64)
        rc = self.lib.orc_fused_moe_fmt(_ptr(x), _ptr(ids), _ptr(tw), T, k, E, H, I, _ptr(c13), _ptr(s13),
                                        _ptr(c2), _ptr(s2), fcode, _ptr(out), _ptr(out_acc), _ptr(h), _ptr(y),
                                        nthreads or default_threads())
        assert rc == 0
        self.last_out_acc = out_acc
        return out, h, y


def compile_oracle(src_path: str, out_path: str) -> str:
    """Compile a copy of the oracle source with the flags the oracle is defined under."""
    tmp = out_path + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-pthread", "-o", tmp, src_path, "-lm"])
    os.replace(tmp, out_path)
    return out_path


def _default() -> Oracle:
    global _lib
    with _lock:
        if _lib is None:
            _lib = Oracle(build())
    return _lib


def __getattr__(name):
    # module-level access to the default oracle's methods: oracle.grouped_gemm(...), ...
    if name in Oracle.__dict__ and not name.startswith("_"):
        return getattr(_default(), name)
    raise AttributeError(name)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact: BF16 is the top half of binary32)."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
