"""Thin Python binding of libw4a16 (ctypes).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU; their device pointers and the
current HIP stream are handed to the C ABI declared in ``include/w4a16.h``.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

FORMAT_INT4 = 0
FORMAT_MXFP4 = 1
KERNEL_DECODE = 1
KERNEL_PREFILL = 2


class W4A16Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("w4a16 error %d: %s" % (code, message))
        self.code = code


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("block_m", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("k_split", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1)]

    def __repr__(self):
        kind = {KERNEL_DECODE: "decode", KERNEL_PREFILL: "prefill"}.get(self.kernel, str(self.kernel))
        tile = ", tile_m=%d" % self.tile_m if self.tile_m else ""
        if self.flags:
            tile += ", flags=%d" % self.flags
        return "Plan(%s, block_m=%d, n_blocks=%d, waves=%d, k_split=%d%s)" % (kind, self.block_m, self.n_blocks,
                                                                            self.waves, self.k_split, tile)


# name -> (restype, argtypes)
_SIGS = {
    "w4a16_last_error": (ctypes.c_char_p, []),
    "w4a16_version": (ctypes.c_char_p, []),
    "w4a16_packed_bytes": (_I, [_I, _I, _I, ctypes.POINTER(_SZ)]),
    "w4a16_pack_weights": (_I, [_P, _P, _I, _I, _I, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "w4a16_packed_bytes_mxfp4": (_I, [_I, _I, _I, ctypes.POINTER(_SZ)]),
    "w4a16_pack_weights_mxfp4": (_I, [_P, _P, _I, _I, _I, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "w4a16_weights_format": (_I, [_P]),
    "w4a16_weights_rebind": (_I, [_P, _P, ctypes.POINTER(_P)]),
    "w4a16_weights_info": (_I, [_P, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I),
                                ctypes.POINTER(_P), ctypes.POINTER(_SZ)]),
    "w4a16_weights_destroy": (None, [_P]),
    "w4a16_dequant": (_I, [_P, _I, _P, _P, _P]),
    "w4a16_route_bounds": (_I, [_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "w4a16_route_prep": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "w4a16_route_prep_workspace_bytes": (_I, [_I, _I, _I, ctypes.POINTER(_SZ)]),
    "w4a16_contiguous_workspace_bytes": (_I, [_I, _P, _P, ctypes.POINTER(_SZ)]),
    "w4a16_grouped_gemm_contiguous": (_I, [_P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "w4a16_masked_workspace_bytes": (_I, [_I, _P, _P, ctypes.POINTER(_SZ)]),
    "w4a16_grouped_gemm_masked": (_I, [_P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "w4a16_route_prep_ws": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "w4a16_plan_select": (_I, [_I, _I, _I, _I, _I, ctypes.c_float, ctypes.POINTER(Plan)]),
    "w4a16_gemm_workspace_bytes": (_I, [ctypes.POINTER(Plan), _I, _I, _I, ctypes.POINTER(_SZ)]),
    "w4a16_grouped_gemm": (_I, [_P, _I, _P, _P, _P, _P, _I, ctypes.POINTER(Plan), _P, _P, _SZ, _P]),
    "w4a16_grouped_gemm_f32": (_I, [_P, _I, _P, _P, _P, _P, _I, ctypes.POINTER(Plan), _P, _P, _SZ, _P]),
    "w4a16_grouped_gemm_silu": (_I, [_P, _I, _P, _P, _P, _P, _I, ctypes.POINTER(Plan), _P, _P, _SZ, _P]),
    "w4a16_silu_mul_f32": (_I, [_P, _I, _I, _P, _P]),
    "w4a16_fused_moe_plans": (_I, [_I, _I, _P, _P, ctypes.POINTER(Plan), ctypes.POINTER(Plan)]),
    "w4a16_offsets_workspace_bytes": (_I, [_I, _P, ctypes.POINTER(Plan), ctypes.POINTER(_SZ)]),
    "w4a16_grouped_gemm_offsets": (_I, [_P, _P, _I, _P, ctypes.POINTER(Plan), _P, _P, _SZ, _P]),
    "w4a16_silu_mul": (_I, [_P, _I, _I, _P, _P]),
    "w4a16_moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "w4a16_moe_combine_bf16": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "w4a16_fused_moe_workspace_bytes": (_I, [_I, _I, _P, _P, ctypes.POINTER(_SZ)]),
    "w4a16_fused_moe": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "w4a16_fused_moe_profiled": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P, _P]),
    "w4a16_fused_moe_plans_hint": (_I, [_I, _I, _P, _P, ctypes.c_float, ctypes.POINTER(Plan), ctypes.POINTER(Plan)]),
    "w4a16_fused_moe_planned_workspace_bytes": (_I, [_I, _I, _P, _P, ctypes.POINTER(Plan), ctypes.POINTER(Plan),
                                                     ctypes.POINTER(_SZ)]),
    "w4a16_fused_moe_planned": (_I, [_P, _P, _P, _I, _I, _P, _P, ctypes.POINTER(Plan), ctypes.POINTER(Plan), _P, _P,
                                     _SZ, _P, _P]),
    "w4a16_fused_moe_noalloc": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _P]),
    "w4a16_validate_routing": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "w4a16_workspace_bytes": (_I, [ctypes.POINTER(Plan), _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
}

ROUTE_BAD_COUNT, ROUTE_BAD_EXPERT, ROUTE_BAD_SLOT, ROUTE_WRONG_EXPERT = 1, 2, 4, 8

_lib = None


def load(path: str = LIB_PATH):
    """Load libw4a16.so (built in-tree by ``weight_only_int4_amd.build``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError("libw4a16.so is not built (%s); run weight_only_int4_amd.build.build()" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != 0:
        raise W4A16Error(rc, load().w4a16_last_error().decode())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def version() -> str:
    return load().w4a16_version().decode()


def symbol_names():
    return list(_SIGS)


# ---------------------------------------------------------------- weights

def packed_bytes(E: int, N: int, K: int, fmt: str = "int4") -> int:
    out = _SZ(0)
    fn = load().w4a16_packed_bytes_mxfp4 if fmt == "mxfp4" else load().w4a16_packed_bytes
    _check(fn(E, N, K, ctypes.byref(out)))
    return out.value


class Weights:
    """A packed weight set: device buffer plus the library's host handle."""

    def __init__(self, handle: int, packed: torch.Tensor, E: int, N: int, K: int):
        self.handle = ctypes.c_void_p(handle)
        self.packed = packed
        self.E, self.N, self.K = E, N, K

    def rebind(self, packed: torch.Tensor) -> "Weights":
        """Handle for another buffer holding a byte-identical copy of this packed image."""
        h = ctypes.c_void_p()
        _check(load().w4a16_weights_rebind(self.handle, _ptr(packed), ctypes.byref(h)))
        return Weights(h.value, packed, self.E, self.N, self.K)

    @property
    def fmt(self) -> str:
        rc = load().w4a16_weights_format(self.handle)
        _check(min(rc, 0))
        return "mxfp4" if rc == FORMAT_MXFP4 else "int4"

    def info(self):
        E, N, K = _I(), _I(), _I()
        p, b = _P(), _SZ()
        _check(load().w4a16_weights_info(self.handle, ctypes.byref(E), ctypes.byref(N), ctypes.byref(K),
                                         ctypes.byref(p), ctypes.byref(b)))
        return E.value, N.value, K.value, p.value, b.value

    def __del__(self):
        if _lib is not None and self.handle:
            _lib.w4a16_weights_destroy(self.handle)
            self.handle = None


def pack_weights(codes: torch.Tensor, scales: torch.Tensor, packed: torch.Tensor | None = None,
                 stream=None) -> Weights:
    """codes uint8 [E,N,K] (low nibble), scales bf16 [E,N,K/32] -> Weights (packed on the GPU)."""
    E, N, K = codes.shape
    nbytes = packed_bytes(E, N, K)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    h = ctypes.c_void_p()
    _check(load().w4a16_pack_weights(_ptr(codes), _ptr(scales), E, N, K, _ptr(packed), packed.numel(),
                                     _stream(stream), ctypes.byref(h)))
    return Weights(h.value, packed, E, N, K)

def pack_weights_mxfp4(codes: torch.Tensor, scales: torch.Tensor, packed: torch.Tensor | None = None,
                       stream=None) -> Weights:
    """MXFP4: codes uint8 [E,N,K] (low nibble: E2M1), scales uint8 [E,N,K/32] (E8M0) -> Weights."""
    E, N, K = codes.shape
    nbytes = packed_bytes(E, N, K, "mxfp4")
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    h = ctypes.c_void_p()
    _check(load().w4a16_pack_weights_mxfp4(_ptr(codes), _ptr(scales), E, N, K, _ptr(packed), packed.numel(),
                                           _stream(stream), ctypes.byref(h)))
    return Weights(h.value, packed, E, N, K)


def dequant(w: Weights, expert: int, want_f32: bool = True, want_bf16: bool = True, stream=None):
    dev = w.packed.device
    f = torch.empty((w.N, w.K), dtype=torch.float32, device=dev) if want_f32 else None
    b = torch.empty((w.N, w.K), dtype=torch.bfloat16, device=dev) if want_bf16 else None
    _check(load().w4a16_dequant(w.handle, expert, _ptr(f), _ptr(b), _stream(stream)))
    return f, b


# ---------------------------------------------------------------- routing

def route_bounds(T: int, k: int, E: int, block_m: int):
    mp, mb = _I(), _I()
    _check(load().w4a16_route_bounds(T, k, E, block_m, ctypes.byref(mp), ctypes.byref(mb)))
    return mp.value, mb.value


def route_prep_workspace_bytes(T: int, k: int, E: int) -> int:
    out = _SZ(0)
    _check(load().w4a16_route_prep_workspace_bytes(T, k, E, ctypes.byref(out)))
    return out.value


def route_prep(topk_ids: torch.Tensor, E: int, block_m: int, stream=None, multi: bool = False) -> dict:
    """topk_ids int32 [T,k] on the GPU -> routing tensors (all on the GPU).  ``multi``: the several-workgroup
    form with its scratch (w4a16_route_prep_ws)."""
    T, k = topk_ids.shape
    maxP, maxB = route_bounds(T, k, E, block_m)
    dev = topk_ids.device
    out = dict(sorted_ids=torch.empty(max(maxP, 1), dtype=torch.int32, device=dev)[:maxP],
               expert_ids=torch.empty(max(maxB, 1), dtype=torch.int32, device=dev)[:maxB],
               num_tokens_padded=torch.empty(1, dtype=torch.int32, device=dev),
               expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               counts=torch.empty(E, dtype=torch.int32, device=dev), block_m=block_m, R=T * k, E=E)
    if multi:
        nbytes = route_prep_workspace_bytes(T, k, E)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        _check(load().w4a16_route_prep_ws(_ptr(topk_ids) if T else None, T, k, E, block_m,
                                          ctypes.c_void_p(out["sorted_ids"].data_ptr()),
                                          ctypes.c_void_p(out["expert_ids"].data_ptr()),
                                          _ptr(out["num_tokens_padded"]), _ptr(out["expert_offsets"]),
                                          _ptr(out["counts"]), _ptr(ws), ws.numel(), _stream(stream)))
        out["_ws"] = ws
        return out
    route_prep_into(topk_ids, E, block_m, out, stream)
    return out


def route_prep_into(topk_ids: torch.Tensor, E: int, block_m: int, out: dict, stream=None):
    T, k = topk_ids.shape
    L = load()
    _check(L.w4a16_route_prep(_ptr(topk_ids) if T else None, T, k, E, block_m,
                              ctypes.c_void_p(out["sorted_ids"].data_ptr()),
                              ctypes.c_void_p(out["expert_ids"].data_ptr()), _ptr(out["num_tokens_padded"]),
                              _ptr(out["expert_offsets"]), _ptr(out["counts"]), _stream(stream)))


# ---------------------------------------------------------------- planning and GEMM

def validate_routing(route: dict, topk_ids: torch.Tensor | None = None, status: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Device-side check of routing tensors (w4a16_validate_routing); returns the int32 status tensor [1] (0 =
    valid, else a bitmask of ROUTE_*), written on the stream without a host read-back."""
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=route["sorted_ids"].device)
    _check(load().w4a16_validate_routing(_ptr(topk_ids) if topk_ids is not None else None, route["R"], route["E"],
                                         route["block_m"], ctypes.c_void_p(route["sorted_ids"].data_ptr()),
                                         ctypes.c_void_p(route["expert_ids"].data_ptr()),
                                         _ptr(route["num_tokens_padded"]), route["sorted_ids"].numel(),
                                         _ptr(status), _stream(stream)))
    return status


def plan_select(T: int, k: int, E: int, N: int, K: int, expected_rows_per_expert: float = 0.0) -> Plan:
    p = Plan()
    _check(load().w4a16_plan_select(T, k, E, N, K, float(expected_rows_per_expert), ctypes.byref(p)))
    return p


PLAN_ONE_LAUNCH = 1  # W4A16_PLAN_ONE_LAUNCH


def make_plan(kernel: str, block_m: int, n_blocks: int, waves: int, k_split: int = 1, tile_m: int = 0,
              flags: int = 0) -> Plan:
    p = Plan()
    p.kernel = KERNEL_DECODE if kernel == "decode" else KERNEL_PREFILL
    p.block_m, p.n_blocks, p.waves, p.k_split, p.tile_m = block_m, n_blocks, waves, k_split, tile_m
    p.flags = flags
    return p


def one_launch(plans):
    """The fused call's (gate_up, down) plans with W4A16_PLAN_ONE_LAUNCH set on the gate_up plan."""
    p13, p2 = plans
    q = Plan.from_buffer_copy(p13)
    q.flags |= PLAN_ONE_LAUNCH
    return q, p2


def two_launches(plans):
    """The fused call's (gate_up, down) plans with W4A16_PLAN_ONE_LAUNCH cleared on the gate_up plan."""
    p13, p2 = plans
    q = Plan.from_buffer_copy(p13)
    q.flags &= ~PLAN_ONE_LAUNCH
    return q, p2


def gemm_workspace_bytes(plan: Plan, R: int, E: int, N: int) -> int:
    out = _SZ(0)
    _check(load().w4a16_gemm_workspace_bytes(ctypes.byref(plan), R, E, N, ctypes.byref(out)))
    return out.value


def zeroed_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace as the library requires it: zero-filled before its first use."""
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def grouped_gemm(A: torch.Tensor, a_row_div: int, w: Weights, route: dict, plan: Plan,
                 out: torch.Tensor | None = None, out_f32: bool = False, ws: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Indexed grouped GEMM; ``route`` from route_prep with plan.block_m.  Returns out [R, N], BF16 (or the
    unrounded binary32 accumulators with ``out_f32``)."""
    R = route["R"]
    if route["block_m"] != plan.block_m:
        raise ValueError("routing was prepared with block_m=%d but the plan uses %d" % (route["block_m"], plan.block_m))
    if route["E"] != w.E:
        raise ValueError("routing was prepared for %d experts but the weights hold %d" % (route["E"], w.E))
    if out is None:
        out = torch.empty((R, w.N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=A.device)
    if ws is None:
        ws = zeroed_workspace(gemm_workspace_bytes(plan, R, w.E, w.N), A.device)
    fn = load().w4a16_grouped_gemm_f32 if out.dtype == torch.float32 else load().w4a16_grouped_gemm
    _check(fn(_ptr(A), a_row_div, w.handle, ctypes.c_void_p(route["sorted_ids"].data_ptr()),
              ctypes.c_void_p(route["expert_ids"].data_ptr()), _ptr(route["num_tokens_padded"]), R,
              ctypes.byref(plan), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def grouped_gemm_silu(A: torch.Tensor, a_row_div: int, w13: Weights, route: dict, plan: Plan,
                      out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Gate/up grouped GEMM with SiLU*mul in the epilogue: h [R, N/2] BF16 from w13 [E, N, K] (gate rows first)."""
    R = route["R"]
    if route["block_m"] != plan.block_m:
        raise ValueError("routing was prepared with block_m=%d but the plan uses %d" % (route["block_m"], plan.block_m))
    if route["E"] != w13.E:
        raise ValueError("routing was prepared for %d experts but the weights hold %d" % (route["E"], w13.E))
    if out is None:
        out = torch.empty((R, w13.N // 2), dtype=torch.bfloat16, device=A.device)
    if ws is None:
        ws = zeroed_workspace(gemm_workspace_bytes(plan, R, w13.E, w13.N), A.device)
    _check(load().w4a16_grouped_gemm_silu(_ptr(A), a_row_div, w13.handle, ctypes.c_void_p(route["sorted_ids"].data_ptr()),
                                          ctypes.c_void_p(route["expert_ids"].data_ptr()),
                                          _ptr(route["num_tokens_padded"]), R, ctypes.byref(plan), _ptr(out), _ptr(ws),
                                          ws.numel(), _stream(stream)))
    return out


def offsets_workspace_bytes(rows_max: int, w: Weights, plan: Plan) -> int:
    out = _SZ(0)
    _check(load().w4a16_offsets_workspace_bytes(rows_max, w.handle, ctypes.byref(plan), ctypes.byref(out)))
    return out.value


def grouped_gemm_offsets(A_sorted: torch.Tensor, expert_offsets: torch.Tensor, w: Weights, plan: Plan,
                         out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    rows_max = A_sorted.shape[0]
    if out is None:
        out = torch.empty((rows_max, w.N), dtype=torch.bfloat16, device=A_sorted.device)
    if ws is None:
        ws = zeroed_workspace(offsets_workspace_bytes(rows_max, w, plan), A_sorted.device)
    _check(load().w4a16_grouped_gemm_offsets(_ptr(A_sorted), _ptr(expert_offsets), rows_max, w.handle,
                                             ctypes.byref(plan), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def contiguous_workspace_bytes(m: int, w: Weights, plan: Plan) -> int:
    out = _SZ(0)
    _check(load().w4a16_contiguous_workspace_bytes(m, w.handle, ctypes.byref(plan), ctypes.byref(out)))
    return out.value


def grouped_gemm_contiguous(A: torch.Tensor, m_indices: torch.Tensor, w: Weights, plan: Plan,
                            out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """Contiguous form: row r of A [m, K] belongs to expert m_indices[r] (-1: padding, row of out untouched)."""
    m = A.shape[0]
    if out is None:
        out = torch.empty((m, w.N), dtype=torch.bfloat16, device=A.device)
    if ws is None:
        ws = zeroed_workspace(contiguous_workspace_bytes(m, w, plan), A.device)
    _check(load().w4a16_grouped_gemm_contiguous(_ptr(A), _ptr(m_indices), m, w.handle, ctypes.byref(plan), _ptr(out),
                                                _ptr(ws), ws.numel(), _stream(stream)))
    return out


def masked_workspace_bytes(max_m: int, w: Weights, plan: Plan) -> int:
    out = _SZ(0)
    _check(load().w4a16_masked_workspace_bytes(max_m, w.handle, ctypes.byref(plan), ctypes.byref(out)))
    return out.value


def grouped_gemm_masked(A: torch.Tensor, masked_m: torch.Tensor, w: Weights, plan: Plan,
                        out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """Masked form: A [E, max_m, K]; rows r < masked_m[e] of expert e are computed into the flat out
    [E*max_m, N]; the other rows of out are untouched."""
    E, max_m, K = A.shape
    if out is None:
        out = torch.empty((E * max_m, w.N), dtype=torch.bfloat16, device=A.device)
    if ws is None:
        ws = zeroed_workspace(masked_workspace_bytes(max_m, w, plan), A.device)
    _check(load().w4a16_grouped_gemm_masked(_ptr(A), _ptr(masked_m), max_m, w.handle, ctypes.byref(plan), _ptr(out),
                                            _ptr(ws), ws.numel(), _stream(stream)))
    return out


# ---------------------------------------------------------------- expert MLP

def silu_mul(gu: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """h = bf16(silu(gate) * up) from gu [rows, 2I] (BF16 or float32, gate columns first)."""
    rows, two_i = gu.shape
    I = two_i // 2
    if out is None:
        out = torch.empty((rows, I), dtype=torch.bfloat16, device=gu.device)
    fn = load().w4a16_silu_mul_f32 if gu.dtype == torch.float32 else load().w4a16_silu_mul
    _check(fn(_ptr(gu), rows, I, _ptr(out), _stream(stream)))
    return out


def moe_combine(y: torch.Tensor, topk_w: torch.Tensor, topk_ids: torch.Tensor, E: int,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Weighted top-k combine of y [T*k, H], binary32 or BF16 (the BF16 entry point for the latter)."""
    T, k = topk_ids.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    fn = load().w4a16_moe_combine_bf16 if y.dtype in (torch.bfloat16, torch.int16) else load().w4a16_moe_combine
    _check(fn(_ptr(y), _ptr(topk_w), _ptr(topk_ids), T, k, E, H, _ptr(out), _stream(stream)))
    return out


def fused_moe_plans(T: int, k: int, w13: Weights, w2: Weights, expected_rows_per_expert: float = 0.0):
    """The fused call's plans; ``expected_rows_per_expert`` > 0 replaces the default T*k/E estimate."""
    p13, p2 = Plan(), Plan()
    if expected_rows_per_expert > 0:
        _check(load().w4a16_fused_moe_plans_hint(T, k, w13.handle, w2.handle, float(expected_rows_per_expert),
                                                 ctypes.byref(p13), ctypes.byref(p2)))
    else:
        _check(load().w4a16_fused_moe_plans(T, k, w13.handle, w2.handle, ctypes.byref(p13), ctypes.byref(p2)))
    return p13, p2


def fused_moe_workspace_bytes(T: int, k: int, w13: Weights, w2: Weights, plans=None) -> int:
    """Workspace of the fused call, for its own plans or for ``plans`` = (gate_up, down)."""
    out = _SZ(0)
    if plans is None:
        _check(load().w4a16_fused_moe_workspace_bytes(T, k, w13.handle, w2.handle, ctypes.byref(out)))
    else:
        _check(load().w4a16_fused_moe_planned_workspace_bytes(T, k, w13.handle, w2.handle, ctypes.byref(plans[0]),
                                                              ctypes.byref(plans[1]), ctypes.byref(out)))
    return out.value


# stage boundaries recorded by w4a16_fused_moe_profiled: routing | gate_up + activation | down | combine
FUSED_STAGES = ("route_prep", "gate_up_silu", "down", "combine")
FUSED_STAGE_EVENTS = len(FUSED_STAGES) + 1


def fused_moe(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, w13: Weights, w2: Weights,
              out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None,
              stage_events=None, plans=None) -> torch.Tensor:
    """Fused expert MLP.  ``stage_events``: FUSED_STAGE_EVENTS torch.cuda.Event objects (timing) or None;
    ``plans``: (gate_up, down) plans to use instead of the call's own (w4a16_fused_moe_planned)."""
    T, k = topk_ids.shape
    if out is None:
        out = torch.empty((T, w2.N), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = zeroed_workspace(fused_moe_workspace_bytes(T, k, w13, w2, plans), x.device)
    ev = None
    if stage_events is not None:
        if len(stage_events) != FUSED_STAGE_EVENTS:
            raise ValueError("stage_events needs %d events" % FUSED_STAGE_EVENTS)
        arr = (ctypes.c_void_p * FUSED_STAGE_EVENTS)(*[ctypes.c_void_p(e.cuda_event) for e in stage_events])
        ev = ctypes.cast(arr, ctypes.c_void_p)
    head = (_ptr(x) if T else None, _ptr(topk_ids) if T else None, _ptr(topk_w) if T else None, T, k, w13.handle,
            w2.handle)
    tail = (_ptr(out) if T else None, _ptr(ws), ws.numel(), _stream(stream))
    if plans is not None:
        _check(load().w4a16_fused_moe_planned(*head, ctypes.byref(plans[0]), ctypes.byref(plans[1]), *tail, ev))
    elif ev is None:
        _check(load().w4a16_fused_moe(*head, *tail))
    else:
        _check(load().w4a16_fused_moe_profiled(*head, *tail, ev))
    return out


NOALLOC_SCRATCH_BYTES = 96 << 20  # W4A16_NOALLOC_SCRATCH_BYTES


def fused_moe_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, w13: Weights, w2: Weights,
                      out: torch.Tensor, stream=None) -> torch.Tensor:
    """Fused expert MLP with every intermediate in the library's static device scratch (w4a16_fused_moe_noalloc):
    no workspace, no allocation; ``out`` is the caller's."""
    T, k = topk_ids.shape
    _check(load().w4a16_fused_moe_noalloc(_ptr(x) if T else None, _ptr(topk_ids) if T else None,
                                          _ptr(topk_w) if T else None, T, k, w13.handle, w2.handle,
                                          _ptr(out) if T else None, _stream(stream)))
    return out
