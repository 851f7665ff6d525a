"""The C-ABI library loads and exports every entry point its header declares; host-side checks
reject bad arguments before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from weight_only_int4_amd import build, lib as L

    if not os.path.exists(L.LIB_PATH):
        build.build()
    return L.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("w4a16_pack_weights", "w4a16_route_prep", "w4a16_grouped_gemm", "w4a16_fused_moe",
                     "w4a16_grouped_gemm_offsets", "w4a16_dequant", "w4a16_plan_select"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    from weight_only_int4_amd import lib as L

    for name in declared_functions():
        assert hasattr(lib, name), "libw4a16.so does not export " + name
        assert name in L._SIGS, "binding has no signature for " + name


def test_packed_bytes(lib):
    from weight_only_int4_amd import lib as L

    # one superblock = 16 rows x 256 k = 2048 code bytes + 256 scale bytes
    assert L.packed_bytes(1, 16, 256) == 2304
    assert L.packed_bytes(8, 512, 256) == 8 * 32 * 2304
    # ragged shapes pad to whole superblocks
    assert L.packed_bytes(2, 17, 288) == 2 * 2 * 2 * 2304
    # 4.5 bits per weight at the Kimi-K2 gate_up shape
    assert L.packed_bytes(1, 4096, 7168) == 4096 * 7168 * 9 // 16


def test_shape_errors(lib):
    from weight_only_int4_amd import lib as L

    with pytest.raises(L.W4A16Error) as ei:
        L.packed_bytes(1, 16, 100)
    assert ei.value.code == -2 and "multiple of 32" in str(ei.value)
    with pytest.raises(L.W4A16Error) as ei:
        L.packed_bytes(0, 16, 64)
    assert ei.value.code == -1
    sz = ctypes.c_size_t(0)
    h = ctypes.c_void_p()
    # pack into a too-small buffer fails before any launch (fake, never dereferenced device pointers)
    rc = lib.w4a16_pack_weights(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 1, 16, 256, ctypes.c_void_p(0x3000),
                                100, None, ctypes.byref(h))
    assert rc == -4 and b"needs 2304" in lib.w4a16_last_error()
    rc = lib.w4a16_pack_weights(None, ctypes.c_void_p(0x2000), 1, 16, 256, ctypes.c_void_p(0x3000), 4096, None,
                                ctypes.byref(h))
    assert rc == -1
    del sz


def test_route_bounds(lib):
    from weight_only_int4_amd import lib as L

    # R = 32 routes, 8 experts, block 16: 32 + 8*15 = 152 -> 160 slots, 10 blocks
    assert L.route_bounds(16, 2, 8, 16) == (160, 10)
    assert L.route_bounds(0, 8, 128, 16) == (0, 0)
    # DeepSeek-V3-like prefill: 4096 tokens x 8, 256 experts, block 128
    assert L.route_bounds(4096, 8, 256, 128) == (65280, 510)
    with pytest.raises(L.W4A16Error):
        L.route_bounds(4, 2, 8, 24)


def test_route_bounds_match_oracle(lib, orc):
    from weight_only_int4_amd import lib as L

    for T, k, E, BM in [(1, 8, 48, 16), (64, 8, 128, 32), (8192, 8, 48, 128), (3, 3, 5, 64)]:
        assert L.route_bounds(T, k, E, BM) == orc.route_bounds(T, k, E, BM)


def test_plan_selector_keys_on_rows_per_expert(lib):
    from weight_only_int4_amd import lib as L

    # Qwen3-like decode: 64 tokens x 8 / 128 experts = 4 rows per expert
    p = L.plan_select(64, 8, 128, 1536, 2048)
    assert p.kernel == L.KERNEL_DECODE and p.block_m == 16
    # same token count, far fewer experts: 64 x 8 / 4 = 128 rows per expert -> prefill, 16-row route blocks
    # gathered into tiles of up to 144 rows
    p = L.plan_select(64, 8, 4, 1536, 2048)
    assert p.kernel == L.KERNEL_PREFILL and (p.block_m, p.tile_m) == (16, 144)
    # an explicit expectation overrides T*k/E: 10 rows stay on the decode kernel, 30 rows take 64-row tiles of
    # 16-row blocks, 48 rows plain 64-row blocks
    p = L.plan_select(64, 8, 128, 1536, 2048, expected_rows_per_expert=10.0)
    assert p.kernel == L.KERNEL_DECODE and (p.block_m, p.tile_m) == (16, 0)
    p = L.plan_select(64, 8, 128, 1536, 2048, expected_rows_per_expert=30.0)
    assert p.kernel == L.KERNEL_PREFILL and (p.block_m, p.tile_m) == (16, 64)
    p = L.plan_select(64, 8, 128, 1536, 2048, expected_rows_per_expert=48.0)
    assert p.kernel == L.KERNEL_PREFILL and (p.block_m, p.tile_m) == (64, 0)
    # one token on a Kimi-K2-like expert share: few workgroups, so K is split across workgroups, in slices of at
    # least 4 stages of 128 k (at most 14 of K = 7168), and the workgroups are narrowed to 2 n-blocks
    p = L.plan_select(1, 8, 48, 4096, 7168, expected_rows_per_expert=1.0 / 48)
    assert p.kernel == L.KERNEL_DECODE and 1 < p.k_split <= 14 and p.n_blocks == 2
    # a Mixtral-like down projection (K = 14336): K split at most 16 ways, workgroups kept at 4 n-blocks
    p = L.plan_select(1, 2, 8, 4096, 14336)
    assert p.kernel == L.KERNEL_DECODE and p.k_split == 16 and p.n_blocks == 4
    # a short K is never split below 8 stages per slice: K = 768 (6 stages) stays whole
    p = L.plan_select(1, 8, 128, 2048, 768)
    assert p.kernel == L.KERNEL_DECODE and p.k_split == 1
    # the 64-token Qwen3-like step fills the machine as it is: 4 n-blocks, K whole
    for N, K in ((1536, 2048), (2048, 768)):
        p = L.plan_select(64, 8, 128, N, K)
        assert (p.kernel, p.n_blocks, p.k_split) == (L.KERNEL_DECODE, 4, 1)
    # memoised: same answer twice
    a = L.plan_select(256, 8, 48, 4096, 7168)
    b = L.plan_select(256, 8, 48, 4096, 7168)
    assert (a.kernel, a.block_m, a.n_blocks, a.waves, a.tile_m) == (b.kernel, b.block_m, b.n_blocks, b.waves, b.tile_m)


def test_plan_validation(lib):
    from weight_only_int4_amd import lib as L

    sz = ctypes.c_size_t(0)
    bad = L.make_plan("decode", 24, 4, 4)
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(bad), 32, 8, 512, ctypes.byref(sz)) == -2
    bad = L.make_plan("prefill", 96, 4, 4)
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(bad), 32, 8, 512, ctypes.byref(sz)) == -2
    bad = L.make_plan("prefill", 64, 4, 4, k_split=17)
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(bad), 32, 8, 512, ctypes.byref(sz)) == -2
    good = L.make_plan("decode", 16, 4, 4)
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(good), 32, 8, 512, ctypes.byref(sz)) == 0
    # plan flags: W4A16_PLAN_ONE_LAUNCH is the only one; the reserved word stays zero
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(L.make_plan("decode", 16, 4, 4, flags=1)), 32, 8, 512,
                                          ctypes.byref(sz)) == 0
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(L.make_plan("decode", 16, 4, 4, flags=2)), 32, 8, 512,
                                          ctypes.byref(sz)) == -1
    bad = L.make_plan("decode", 16, 4, 4)
    bad.reserved[0] = 1
    assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(bad), 32, 8, 512, ctypes.byref(sz)) == -1
    assert sz.value == 0
    # prefill tiles: 64 or 128 rows, taller than the route block only for 32-row blocks; 16-row blocks take
    # tiles of 64 or 144 rows and two n-blocks per wavefront; decode has none
    for args in (("prefill", 32, 2, 4, 1, 96), ("prefill", 64, 2, 4, 1, 128), ("prefill", 128, 2, 4, 1, 64),
                 ("prefill", 32, 2, 4, 1, 0), ("decode", 16, 4, 4, 1, 64), ("prefill", 16, 2, 4, 1, 0),
                 ("prefill", 16, 2, 4, 1, 128), ("prefill", 16, 4, 4, 1, 144), ("prefill", 32, 2, 4, 1, 144)):
        bad = L.make_plan(*args)
        assert lib.w4a16_gemm_workspace_bytes(ctypes.byref(bad), 32, 8, 512, ctypes.byref(sz)) == -2, args
    # a tile list: its length padded to 16 bytes, then two ints per 32-row route block for the tiles and two for
    # the scratch they are built with (R=32, E=8: at most 9 blocks), rounded up to 256 bytes
    tiled = L.make_plan("prefill", 32, 2, 4, 1, 128)
    assert L.gemm_workspace_bytes(tiled, 32, 8, 512) == 256
    assert L.gemm_workspace_bytes(tiled, 32 * 100, 8, 512) == ((4 + 4 * 108) * 4 + 255) // 256 * 256
    assert L.gemm_workspace_bytes(L.make_plan("prefill", 64, 2, 4, 1, 64), 32, 8, 512) == 0
    # prefill split K: one counter per (tile, column tile), then fp32 partial tiles of the tallest tile.  Plain
    # 64-row blocks: one tile per route block (R=32, E=8, 64-row blocks: 32 + 8*63 slots -> 9 blocks); n_blocks 4
    # -> 256 columns, N=512 -> 2 column tiles
    ps = L.make_plan("prefill", 64, 4, 4, k_split=3)
    assert L.gemm_workspace_bytes(ps, 32, 8, 512) == 256 + 9 * 2 * 3 * 64 * 256 * 4
    # 32-row blocks in 128-row tiles: at most ceil(blocks / 4) + owners tiles (R=32, E=8: 9 blocks -> 3 + 8)
    pt = L.make_plan("prefill", 32, 2, 4, 2, 128)
    tl = ((4 + 4 * 9) * 4 + 255) // 256 * 256
    assert L.gemm_workspace_bytes(pt, 32, 8, 512) == 256 + 11 * 4 * 2 * 128 * 128 * 4 + tl
    # 16-row blocks in 144-row tiles (R=32, E=8: 32 + 8*15 slots -> 10 blocks; at most ceil(10 / 9) + 8 tiles),
    # two n-blocks per wavefront -> 128 columns, N=512 -> 4 column tiles
    pt16 = L.make_plan("prefill", 16, 2, 4, 2, 144)
    tl16 = ((4 + 4 * 10) * 4 + 255) // 256 * 256
    assert L.gemm_workspace_bytes(pt16, 32, 8, 512) == 256 + 10 * 4 * 2 * 144 * 128 * 4 + tl16
    assert L.gemm_workspace_bytes(L.make_plan("prefill", 16, 2, 4, 1, 144), 32, 8, 512) == tl16
    # split K: counters (one per route block and column tile) then fp32 partial tiles
    split = L.make_plan("decode", 16, 4, 4, k_split=4)
    # 10 route blocks x 2 column tiles of 256: 20 counters (one 256-byte line), 10*2*4 partial tiles of 16x256
    assert L.gemm_workspace_bytes(split, 32, 8, 512) == 256 + 10 * 2 * 4 * 16 * 256 * 4


def test_bad_handle_is_rejected(lib):
    # a host buffer that is not a handle: rejected on the host, nothing launched
    junk = (ctypes.c_uint32 * 16)()
    f = ctypes.c_void_p(0x1000)
    rc = lib.w4a16_dequant(ctypes.cast(junk, ctypes.c_void_p), 0, f, None, None)
    assert rc == -3 and b"not a w4a16 weight handle" in lib.w4a16_last_error()
    assert lib.w4a16_dequant(None, 0, f, None, None) == -1


def test_workspace_bytes_in_token_terms(lib):
    """w4a16_workspace_bytes(plan, T, k, E, N) is the GEMM workspace of R = T*k routes."""
    from weight_only_int4_amd import lib as L

    split = L.make_plan("decode", 16, 4, 4, k_split=4)
    sz = ctypes.c_size_t(0)
    assert lib.w4a16_workspace_bytes(ctypes.byref(split), 16, 2, 8, 512, ctypes.byref(sz)) == 0
    assert sz.value == L.gemm_workspace_bytes(split, 32, 8, 512)
    assert lib.w4a16_workspace_bytes(ctypes.byref(split), -1, 2, 8, 512, ctypes.byref(sz)) == -1


def test_validate_routing_argument_checks(lib):
    """Argument errors of the device-side routing check are caught on the host, before any launch (the device
    pointers below are never dereferenced)."""
    st = ctypes.c_void_p(0x4000)
    p = ctypes.c_void_p(0x1000)
    assert lib.w4a16_validate_routing(None, 32, 8, 24, p, p, p, 160, st, None) == -2   # block_m not a multiple of 16
    assert lib.w4a16_validate_routing(None, 32, 8, 16, p, p, p, 150, st, None) == -1   # max_padded not whole blocks
    assert lib.w4a16_validate_routing(None, 32, 8, 16, p, p, None, 160, st, None) == -1
    assert lib.w4a16_validate_routing(None, 32, 8, 16, p, p, p, 160, None, None) == -1
    assert lib.w4a16_validate_routing(None, -1, 8, 16, p, p, p, 160, st, None) == -1
    assert b"w4a16_validate_routing" in lib.w4a16_last_error()


def test_noalloc_checks_before_launch(lib):
    """The no-allocation fused call refuses bad arguments on the host (the handle check comes first)."""
    junk = (ctypes.c_uint32 * 16)()
    h = ctypes.cast(junk, ctypes.c_void_p)
    p = ctypes.c_void_p(0x1000)
    assert lib.w4a16_fused_moe_noalloc(p, p, p, 4, 2, h, h, p, None) == -3
    assert lib.w4a16_fused_moe_noalloc(p, p, p, 4, 2, None, None, p, None) == -1
