// C ABI of libw4a16: argument checks, weight handles, the schedule selector
// and the orchestration of the fused expert MLP.  No device memory is
// allocated or read here; every device operation is a launch on the caller's
// stream.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>

#include "w4a16_internal.h"

using namespace w4a16;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return W4A16_OK;
}

int check_launch(hipError_t err, const char* what) {
    if (err != hipSuccess) return fail(W4A16_HIP_ERROR, "%s: launch failed: %s", what, hipGetErrorString(err));
    return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_handle(const w4a16_weights* w, const char* what) {
    if (!w) return fail(W4A16_INVALID_ARG, "%s: weight handle is NULL", what);
    if (w->magic != kHandleMagic) return fail(W4A16_LAYOUT_MISMATCH, "%s: not a w4a16 weight handle", what);
    if (w->layout_version != (uint32_t)kLayoutVersion)
        return fail(W4A16_LAYOUT_MISMATCH, "%s: packed layout version %u, library expects %d", what,
                    w->layout_version, kLayoutVersion);
    return W4A16_OK;
}

void route_bounds(long T, long k, long E, long BM, int* maxP, int* maxB) {
    const long R = T * k;
    const long act = R < E ? R : E;
    const long raw = R + act * (BM - 1);
    const long blocks = (raw + BM - 1) / BM;
    *maxP = (int)(blocks * BM);
    *maxB = (int)blocks;
}

// ----------------------------------------------------------------- planner

int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    return atoi(v);
}

struct Overrides {
    int force_kernel = 0;  // 0 auto, else W4A16_KERNEL_*
    int block_m = 0, n_blocks = 0, waves = 0, k_split = 0, tile_m = -1;
    int one_launch = -1;  // -1 the planner's rule, 0 or 1 forced (fused prefill steps)
};

const Overrides& overrides() {
    static Overrides o = [] {
        Overrides r;
        const char* fk = getenv("W4A16_FORCE_KERNEL");
        if (!fk || !*fk) fk = getenv("W4A16_FORCE_SCHEDULE");  // the same switch under its other name
        if (fk && !strcmp(fk, "decode")) r.force_kernel = W4A16_KERNEL_DECODE;
        if (fk && !strcmp(fk, "prefill")) r.force_kernel = W4A16_KERNEL_PREFILL;
        r.block_m = env_int("W4A16_BLOCK_M", 0);
        r.n_blocks = env_int("W4A16_N_BLOCKS", 0);
        r.waves = env_int("W4A16_WAVES", 0);
        r.k_split = env_int("W4A16_K_SPLIT", 0);
        r.tile_m = env_int("W4A16_TILE_M", -1);
        r.one_launch = env_int("W4A16_ONE_LAUNCH", -1);
        return r;
    }();
    return o;
}

// Decode streams each weight once per route block and applies the scales per
// output row; the prefill kernel dequantises each weight once per tile and
// shares it over the tile's rows.  Measured on the Qwen3-, Kimi- and
// DeepSeek-shaped projections, decode is faster up to about 12 routed rows per
// expert and the prefill kernel from 16 rows on.
constexpr float kDecodeMaxRows = 12.0f;


w4a16_plan select_plan(int T, int k, int E, int N, int K, float rows) {
    const Overrides& ov = overrides();
    w4a16_plan p;
    memset(&p, 0, sizeof(p));
    const int NB = (N + 15) / 16;
    const int nst = (K / 32 + 3) / 4;  // 128-k stages
    int kernel = rows <= kDecodeMaxRows ? W4A16_KERNEL_DECODE : W4A16_KERNEL_PREFILL;
    if (ov.force_kernel) kernel = ov.force_kernel;
    p.kernel = kernel;
    p.k_split = 1;
    if (kernel == W4A16_KERNEL_DECODE) {
        // cover ~1.3x the expected rows in one block so a slightly heavy expert
        // does not spill into a second pass over all of K (Chord page, "Grouped
        // SM90 kernels", masked decode sizing)
        int bm = (int)ceilf(1.3f * rows / 16.0f) * 16;
        p.block_m = bm < 16 ? 16 : (bm > 64 ? 64 : bm);
        p.n_blocks = NB >= 16 ? 4 : (NB >= 8 ? 2 : 1);
        p.waves = 4;
        // expected route blocks: experts that receive at least one row (Poisson estimate)
        const double active = (double)E * (1.0 - exp(-(double)rows));
        const double blocks = active * ceil((double)rows / p.block_m > 1.0 ? (double)rows / p.block_m : 1.0);
        auto waves_of = [&](int nbw) { return blocks * (double)((NB + nbw * p.waves - 1) / (nbw * p.waves)) * p.waves; };
        // slices of at least 8 stages of 128 k over K up to 32 stages (at K = 2048 one or two slices beat four
        // or eight), of at least 4 over longer K (one token on the Kimi-K2 share, K = 7168: 14 slices 21.6 us,
        // 7 slices 23.7, 28 slices 28.3), and at most 16 slices
        int max_ks = nst <= 32 ? nst / 8 : nst / 4;
        if (max_ks < 1) max_ks = 1;
        if (max_ks > 16) max_ks = 16;
        if (p.n_blocks < 4 || waves_of(4) < 512.0) {
            // A grid of fewer than ~2 wavefronts per CU streams better from narrower workgroups (twice the
            // column tiles), and with K split until ~8 wavefronts per CU: on 1-4 tokens, gate_up and down
            // 10-40% faster (measured on the Qwen3-, Kimi-K2-share and DeepSeek-V3-shaped steps).  With a long
            // K (more than 64 stages, a Mixtral-8x7B-shaped down projection) the slices of 4 n-blocks stream
            // better than narrower workgroups (one token: 25.6 us against 30.5).
            if (p.n_blocks == 4 && nst <= 64) p.n_blocks = 2;
            const double waves_total = waves_of(p.n_blocks);
            const int ks = (int)ceil(2048.0 / (waves_total > 1.0 ? waves_total : 1.0));
            p.k_split = ks < 1 ? 1 : (ks > max_ks ? max_ks : ks);
        } else {
            // From ~2 wavefronts per CU on, K whole is fastest (measured on 2-32 tokens: 8-20% faster than 2 or
            // 3 slices), except where 257-384 workgroups leave a second round less than half full and K is
            // long enough (>= 32 stages) for half-length slices to fill it (Kimi-K2 share, 32 tokens: 66.7 us
            // with 2 slices, 73.9 with K whole)
            const double waves_total = waves_of(4);
            p.k_split = (waves_total > 1024.0 && waves_total <= 1536.0 && nst >= 32 && max_ks >= 2) ? 2 : 1;
        }
    } else {
        // 16-row route blocks keep the padding below 16 rows per expert; the workgroup tile gathers up to nine
        // of them so that each dequantised weight feeds up to 144 rows, and an expert of 129-144 rows is one tile
        // rather than two (measured against 32-row blocks in 128-row tiles: -12% on a 4096-token DeepSeek-V3
        // gate_up, -10% on its down projection, also faster from 64 rows per expert on and on Zipf-routed
        // shares).  Below ~56 rows per expert a 64-row tile is faster (more workgroups; a tall tile would mostly
        // hold a few blocks), except that between 40 and 56 rows plain 64-row blocks are (measured; the tile list
        // costs a launch and the padding saved is small there).
        p.waves = 4;
        p.n_blocks = 2;
        if (rows >= 56.0f) {
            p.block_m = 16;
            p.tile_m = 144;
        } else if (rows >= 40.0f) {
            p.block_m = 64;
        } else {
            p.block_m = 16;
            p.tile_m = 64;
        }
        // The prefill kernel can split K across workgroups (explicit plans), but the planner does not: on an
        // 8-expert, 4096 x 14336 projection whose grid holds about one workgroup per CU, two to eight slices
        // were 2-75% slower at 32 to 256 rows per expert (measured), so more workgroups per CU do not help
        // there and the partial tiles cost their traffic.
    }
    if (ov.block_m) p.block_m = ov.block_m;
    if (ov.n_blocks) p.n_blocks = ov.n_blocks;
    if (ov.waves) p.waves = ov.waves;
    if (ov.k_split) p.k_split = ov.k_split;
    if (ov.tile_m >= 0 && p.kernel == W4A16_KERNEL_PREFILL) p.tile_m = ov.tile_m;
    (void)T; (void)k;
    return p;
}

int validate_plan(const w4a16_plan* p, const char* what) {
    if (!p) return fail(W4A16_INVALID_ARG, "%s: plan is NULL", what);
    if (p->reserved[0]) return fail(W4A16_INVALID_ARG, "%s: plan.reserved must be zero", what);
    if (p->flags & ~W4A16_PLAN_ONE_LAUNCH) return fail(W4A16_INVALID_ARG, "%s: unknown plan flags 0x%x", what, p->flags);
    if (p->kernel == W4A16_KERNEL_DECODE) {
        if (p->block_m % 16 || p->block_m < 16 || p->block_m > 64)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: decode block_m %d not in {16,32,48,64}", what, p->block_m);
        if (p->n_blocks != 1 && p->n_blocks != 2 && p->n_blocks != 4)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: decode n_blocks %d not in {1,2,4}", what, p->n_blocks);
        if (p->k_split < 1 || p->k_split > 64)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: decode k_split %d not in 1..64", what, p->k_split);
        if (p->waves != 4) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: decode waves must be 4", what);
        if (p->tile_m != 0) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: decode tile_m must be 0", what);
    } else if (p->kernel == W4A16_KERNEL_PREFILL) {
        if (p->block_m != 16 && p->block_m != 32 && p->block_m != 64 && p->block_m != 128)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill block_m %d not in {16,32,64,128}", what, p->block_m);
        const int tile = p->tile_m ? p->tile_m : p->block_m;
        if (p->block_m == 16) {
            if (tile != 64 && tile != 144)
                return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill tile_m %d with 16-row blocks not in {64,144}", what,
                            tile);
            if (p->n_blocks != 2)
                return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill n_blocks %d with 16-row blocks must be 2", what,
                            p->n_blocks);
        } else {
            if (tile != 64 && tile != 128)
                return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill tile_m %d not in {64,128}", what, tile);
            if (tile != p->block_m && p->block_m != 32)
                return fail(W4A16_UNSUPPORTED_SHAPE,
                            "%s: prefill tile_m %d must equal block_m %d unless block_m is 16 or 32", what, tile,
                            p->block_m);
        }
        if (p->n_blocks != 2 && p->n_blocks != 4)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill n_blocks %d not in {2,4}", what, p->n_blocks);
        if (p->k_split < 1 || p->k_split > 16)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill k_split %d not in 1..16", what, p->k_split);
        if (p->waves != 4) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: prefill waves must be 4", what);
    } else {
        return fail(W4A16_INVALID_ARG, "%s: unknown kernel %d", what, p->kernel);
    }
    return W4A16_OK;
}

// Split-K workspace of one GEMM: arrival counters first (so that GEMMs sharing a
// workspace find them at the same place, all zero), then the partial tiles.
// A prefill plan whose workgroup tile spans several route blocks also needs a tile list after the split-K area:
// its length (one int, padded to 16 bytes), then (first block, blocks) per tile, at most one tile per block,
// then two ints per block of scratch the list is built with.
struct GemmWs {
    size_t counter_bytes, partial_bytes, tile_bytes, total;
};

bool tiled_prefill(const w4a16_plan& p) {
    return p.kernel == W4A16_KERNEL_PREFILL && prefill_tile_rows(p) != p.block_m;
}

GemmWs gemm_ws(const Shape& sh, const w4a16_plan& p, int max_blocks) {
    GemmWs g;
    g.counter_bytes = align_up(sizeof(unsigned) * (decode_counters(sh, p, max_blocks) +
                                                   prefill_counters(sh, p, max_blocks)), 256);
    g.partial_bytes = align_up(sizeof(float) * (decode_partial_floats(sh, p, max_blocks) +
                                                prefill_partial_floats(sh, p, max_blocks)), 256);
    g.tile_bytes = tiled_prefill(p) ? align_up(sizeof(int32_t) * (4 + 4 * (size_t)max_blocks), 256) : 0;
    g.total = g.counter_bytes + g.partial_bytes + g.tile_bytes;
    return g;
}

// counters at ws, partials at ws + partial_offset, the tile list at tiles
void bind_ws(GemmArgs& a, const GemmWs& g, void* ws, size_t partial_offset, void* tiles) {
    if (g.counter_bytes + g.partial_bytes) {
        a.counters = static_cast<unsigned*>(ws);
        a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + partial_offset);
    }
    if (g.tile_bytes) {
        a.tile_count = static_cast<int32_t*>(tiles);
        a.tiles = static_cast<int32_t*>(tiles) + 4;
        a.tile_scratch = a.tiles + 2 * (size_t)a.max_blocks;
    }
}

// standalone layout: counters | partials | tile list
void bind_ws(GemmArgs& a, const GemmWs& g, void* ws) {
    bind_ws(a, g, ws, g.counter_bytes, static_cast<char*>(ws) + g.counter_bytes + g.partial_bytes);
}

hipError_t run_gemm(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    return p.kernel == W4A16_KERNEL_DECODE ? launch_gemm_decode(a, p, s) : launch_gemm_prefill(a, p, s);
}

// Workspace carve-up of the fused expert MLP.
struct FusedLayout {
    int maxP, maxB;
    size_t off_sorted, off_eids, off_ntp, off_offsets, off_counts, off_h, off_y, off_split, off_tiles, off_route,
        total;
};

// The split-K area goes first so its counters sit at a fixed place regardless of the route block.
// The two GEMMs run one after the other on one stream, so they share one tile-list area.
FusedLayout fused_layout(int T, int k, int E, int H, int I, int BM, size_t split_bytes, size_t tile_bytes) {
    FusedLayout f;
    route_bounds(T, k, E, BM, &f.maxP, &f.maxB);
    const size_t R = (size_t)T * k;
    size_t o = 0;
    f.off_split = o;  o = align_up(o + split_bytes, 256);
    f.off_tiles = o;  o = align_up(o + tile_bytes, 256);
    f.off_route = o;  o = align_up(o + sizeof(int32_t) * route_prep_scratch_ints((int)R, E), 256);
    f.off_sorted = o; o = align_up(o + sizeof(int32_t) * (size_t)f.maxP, 256);
    f.off_eids = o;   o = align_up(o + sizeof(int32_t) * (size_t)f.maxB, 256);
    f.off_ntp = o;    o = align_up(o + sizeof(int32_t), 256);
    f.off_offsets = o; o = align_up(o + sizeof(int32_t) * (size_t)(E + 1), 256);
    f.off_counts = o; o = align_up(o + sizeof(int32_t) * (size_t)E, 256);
    f.off_h = o;      o = align_up(o + sizeof(uint16_t) * R * I, 256);
    f.off_y = o;      o = align_up(o + sizeof(uint16_t) * R * H, 256);  // y in BF16
    f.total = o;
    return f;
}

}  // namespace

extern "C" {

const char* w4a16_last_error(void) { return g_last_error.c_str(); }

const char* w4a16_version(void) { return "libw4a16 0.1 (packed layout 1, gfx950)"; }

int w4a16_packed_bytes(int E, int N, int K, size_t* bytes) {
    if (!bytes) return fail(W4A16_INVALID_ARG, "w4a16_packed_bytes: bytes is NULL");
    if (E < 1 || N < 1) return fail(W4A16_INVALID_ARG, "w4a16_packed_bytes: E=%d N=%d must be >= 1", E, N);
    if (K < 32 || K % 32) return fail(W4A16_UNSUPPORTED_SHAPE, "w4a16_packed_bytes: K=%d must be a positive multiple of 32", K);
    *bytes = packed_bytes(make_shape(E, N, K));
    return ok();
}

int w4a16_pack_weights(const uint8_t* codes, const uint16_t* scales, int E, int N, int K, void* packed,
                       size_t packed_bytes_avail, hipStream_t s, w4a16_weights** out) {
    const char* what = "w4a16_pack_weights";
    if (!codes || !scales || !packed || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    size_t need = 0;
    int rc = w4a16_packed_bytes(E, N, K, &need);
    if (rc) return rc;
    if (packed_bytes_avail < need)
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: packed buffer has %zu bytes, needs %zu", what, packed_bytes_avail, need);
    if (!aligned16(packed)) return fail(W4A16_INVALID_ARG, "%s: packed buffer must be 16-byte aligned", what);
    if (((uintptr_t)codes & 7u) != 0) return fail(W4A16_INVALID_ARG, "%s: codes must be 8-byte aligned", what);
    w4a16_weights* w = new (std::nothrow) w4a16_weights;
    if (!w) return fail(W4A16_INVALID_ARG, "%s: out of host memory", what);
    w->magic = kHandleMagic;
    w->layout_version = kLayoutVersion;
    w->shape = make_shape(E, N, K);
    w->packed = packed;
    w->bytes = need;
    rc = check_launch(launch_pack(codes, scales, w->shape, packed, s), what);
    if (rc) {
        delete w;
        return rc;
    }
    *out = w;
    return ok();
}

int w4a16_packed_bytes_mxfp4(int E, int N, int K, size_t* bytes) {
    if (!bytes) return fail(W4A16_INVALID_ARG, "w4a16_packed_bytes_mxfp4: bytes is NULL");
    if (E < 1 || N < 1) return fail(W4A16_INVALID_ARG, "w4a16_packed_bytes_mxfp4: E=%d N=%d must be >= 1", E, N);
    if (K < 32 || K % 32)
        return fail(W4A16_UNSUPPORTED_SHAPE, "w4a16_packed_bytes_mxfp4: K=%d must be a positive multiple of 32", K);
    *bytes = packed_bytes(make_shape(E, N, K, kFmtMxfp4));
    return ok();
}

int w4a16_pack_weights_mxfp4(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, void* packed,
                             size_t packed_bytes_avail, hipStream_t s, w4a16_weights** out) {
    const char* what = "w4a16_pack_weights_mxfp4";
    if (!codes || !scales || !packed || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    size_t need = 0;
    int rc = w4a16_packed_bytes_mxfp4(E, N, K, &need);
    if (rc) return rc;
    if (packed_bytes_avail < need)
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: packed buffer has %zu bytes, needs %zu", what, packed_bytes_avail, need);
    if (!aligned16(packed)) return fail(W4A16_INVALID_ARG, "%s: packed buffer must be 16-byte aligned", what);
    if (((uintptr_t)codes & 7u) != 0) return fail(W4A16_INVALID_ARG, "%s: codes must be 8-byte aligned", what);
    w4a16_weights* w = new (std::nothrow) w4a16_weights;
    if (!w) return fail(W4A16_INVALID_ARG, "%s: out of host memory", what);
    w->magic = kHandleMagic;
    w->layout_version = kLayoutVersion;
    w->shape = make_shape(E, N, K, kFmtMxfp4);
    w->packed = packed;
    w->bytes = need;
    rc = check_launch(launch_pack_mxfp4(codes, scales, w->shape, packed, s), what);
    if (rc) {
        delete w;
        return rc;
    }
    *out = w;
    return ok();
}

int w4a16_weights_format(const w4a16_weights* w) {
    int rc = check_handle(w, "w4a16_weights_format");
    if (rc) return rc;
    return w->shape.fmt;
}

int w4a16_weights_rebind(const w4a16_weights* w, void* packed, w4a16_weights** out) {
    int rc = check_handle(w, "w4a16_weights_rebind");
    if (rc) return rc;
    if (!packed || !out) return fail(W4A16_INVALID_ARG, "w4a16_weights_rebind: NULL pointer argument");
    if (!aligned16(packed)) return fail(W4A16_INVALID_ARG, "w4a16_weights_rebind: packed buffer must be 16-byte aligned");
    w4a16_weights* n = new (std::nothrow) w4a16_weights(*w);
    if (!n) return fail(W4A16_INVALID_ARG, "w4a16_weights_rebind: out of host memory");
    n->packed = packed;
    *out = n;
    return ok();
}

int w4a16_weights_info(const w4a16_weights* w, int* E, int* N, int* K, void** packed, size_t* bytes) {
    int rc = check_handle(w, "w4a16_weights_info");
    if (rc) return rc;
    if (E) *E = w->shape.E;
    if (N) *N = w->shape.N;
    if (K) *K = w->shape.K;
    if (packed) *packed = w->packed;
    if (bytes) *bytes = w->bytes;
    return ok();
}

void w4a16_weights_destroy(w4a16_weights* w) {
    if (w && w->magic == kHandleMagic) {
        w->magic = 0;
        delete w;
    }
}

int w4a16_dequant(const w4a16_weights* w, int expert, float* out_f32, uint16_t* out_bf16, hipStream_t s) {
    const char* what = "w4a16_dequant";
    int rc = check_handle(w, what);
    if (rc) return rc;
    if (expert < 0 || expert >= w->shape.E)
        return fail(W4A16_INVALID_ARG, "%s: expert %d outside [0,%d)", what, expert, w->shape.E);
    if (!out_f32 && !out_bf16) return fail(W4A16_INVALID_ARG, "%s: both outputs are NULL", what);
    return check_launch(launch_dequant(w->packed, w->shape, expert, out_f32, out_bf16, s), what);
}

int w4a16_route_bounds(int T, int k, int E, int block_m, int* max_padded, int* max_blocks) {
    if (!max_padded || !max_blocks) return fail(W4A16_INVALID_ARG, "w4a16_route_bounds: NULL output");
    if (T < 0 || k < 1 || E < 1) return fail(W4A16_INVALID_ARG, "w4a16_route_bounds: T=%d k=%d E=%d", T, k, E);
    if (block_m < 16 || block_m % 16)
        return fail(W4A16_UNSUPPORTED_SHAPE, "w4a16_route_bounds: block_m %d must be a positive multiple of 16", block_m);
    if ((long)T * k > (1L << 30)) return fail(W4A16_UNSUPPORTED_SHAPE, "w4a16_route_bounds: T*k too large");
    route_bounds(T, k, E, block_m, max_padded, max_blocks);
    return ok();
}

int w4a16_route_prep(const int32_t* topk_ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                     int32_t* expert_ids, int32_t* num_tokens_padded, int32_t* expert_offsets, int32_t* counts,
                     hipStream_t s) {
    const char* what = "w4a16_route_prep";
    int maxP, maxB;
    int rc = w4a16_route_bounds(T, k, E, block_m, &maxP, &maxB);
    if (rc) return rc;
    if (E > W4A16_MAX_EXPERTS) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: E=%d exceeds %d", what, E, W4A16_MAX_EXPERTS);
    if ((T > 0 && !topk_ids) || (maxP > 0 && !sorted_ids) || (maxB > 0 && !expert_ids) || !num_tokens_padded ||
        !expert_offsets || !counts)
        return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    return check_launch(launch_route_prep(topk_ids, T * k, E, block_m, maxP, maxB, sorted_ids, expert_ids,
                                          num_tokens_padded, expert_offsets, counts, s),
                        what);
}

int w4a16_route_prep_workspace_bytes(int T, int k, int E, size_t* bytes) {
    if (!bytes || T < 0 || k < 1 || E < 1 || (long)T * k > INT32_MAX)
        return fail(W4A16_INVALID_ARG, "w4a16_route_prep_workspace_bytes: T=%d k=%d E=%d", T, k, E);
    *bytes = sizeof(int32_t) * route_prep_scratch_ints(T * k, E);
    return ok();
}

int w4a16_route_prep_ws(const int32_t* topk_ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                        int32_t* expert_ids, int32_t* num_tokens_padded, int32_t* expert_offsets, int32_t* counts,
                        void* ws, size_t ws_bytes, hipStream_t s) {
    const char* what = "w4a16_route_prep_ws";
    int maxP, maxB;
    int rc = w4a16_route_bounds(T, k, E, block_m, &maxP, &maxB);
    if (rc) return rc;
    if (E > W4A16_MAX_EXPERTS) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: E=%d exceeds %d", what, E, W4A16_MAX_EXPERTS);
    if ((T > 0 && !topk_ids) || (maxP > 0 && !sorted_ids) || (maxB > 0 && !expert_ids) || !num_tokens_padded ||
        !expert_offsets || !counts)
        return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    const size_t need = sizeof(int32_t) * route_prep_scratch_ints(T * k, E);
    if (need && (!ws || ws_bytes < need))
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, needs %zu", what, ws_bytes, need);
    if (need && ((uintptr_t)ws & 3u)) return fail(W4A16_INVALID_ARG, "%s: workspace must be 4-byte aligned", what);
    return check_launch(launch_route_prep_scratch(topk_ids, T * k, E, block_m, maxP, maxB, sorted_ids, expert_ids,
                                                  num_tokens_padded, expert_offsets, counts,
                                                  need ? static_cast<int32_t*>(ws) : nullptr, s),
                        what);
}

int w4a16_validate_routing(const int32_t* topk_ids, int R, int E, int block_m, const int32_t* sorted_ids,
                           const int32_t* expert_ids, const int32_t* num_tokens_padded, int max_padded,
                           int32_t* status, hipStream_t s) {
    const char* what = "w4a16_validate_routing";
    if (R < 0 || E < 1 || max_padded < 0) return fail(W4A16_INVALID_ARG, "%s: R=%d E=%d max_padded=%d", what, R, E, max_padded);
    if (block_m < 16 || block_m % 16)
        return fail(W4A16_UNSUPPORTED_SHAPE, "%s: block_m %d must be a positive multiple of 16", what, block_m);
    if (max_padded % block_m) return fail(W4A16_INVALID_ARG, "%s: max_padded %d not a multiple of block_m", what, max_padded);
    if (!num_tokens_padded || !status || (max_padded > 0 && (!sorted_ids || !expert_ids)))
        return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    return check_launch(launch_route_validate(topk_ids, R, E, block_m, sorted_ids, expert_ids, num_tokens_padded,
                                              max_padded, status, s),
                        what);
}

int w4a16_plan_select(int T, int k, int E, int N, int K, float expected_rows_per_expert, w4a16_plan* out) {
    if (!out) return fail(W4A16_INVALID_ARG, "w4a16_plan_select: out is NULL");
    if (T < 0 || k < 1 || E < 1 || N < 1 || K < 32 || K % 32)
        return fail(W4A16_INVALID_ARG, "w4a16_plan_select: bad shape T=%d k=%d E=%d N=%d K=%d", T, k, E, N, K);
    const float rows = expected_rows_per_expert > 0 ? expected_rows_per_expert : (float)T * k / (float)E;
    typedef std::tuple<int, int, int, int, int, float> Key;
    static std::mutex mu;
    static std::map<Key, w4a16_plan> memo;
    const Key key(T, k, E, N, K, rows);
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = memo.find(key);
        if (it != memo.end()) {
            *out = it->second;
            return ok();
        }
    }
    w4a16_plan p = select_plan(T, k, E, N, K, rows);
    int rc = validate_plan(&p, "w4a16_plan_select (after environment overrides)");
    if (rc) return rc;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (memo.size() > 4096) memo.clear();
        memo[key] = p;
    }
    *out = p;
    return ok();
}

int w4a16_gemm_workspace_bytes(const w4a16_plan* p, int R, int E, int N, size_t* bytes) {
    int rc = validate_plan(p, "w4a16_gemm_workspace_bytes");
    if (rc) return rc;
    if (!bytes || R < 0 || E < 1 || N < 1) return fail(W4A16_INVALID_ARG, "w4a16_gemm_workspace_bytes: bad argument");
    int maxP, maxB;
    route_bounds(R, 1, E, p->block_m, &maxP, &maxB);
    *bytes = gemm_ws(make_shape(E, N, 32), *p, maxB).total;
    return ok();
}

int w4a16_workspace_bytes(const w4a16_plan* p, int T, int k, int E, int N, size_t* bytes) {
    if (T < 0 || k < 1 || (long)T * k > INT32_MAX)
        return fail(W4A16_INVALID_ARG, "w4a16_workspace_bytes: T=%d k=%d", T, k);
    return w4a16_gemm_workspace_bytes(p, T * k, E, N, bytes);
}

// Shapes the prefill kernel cannot address (its buffer resources reach below 2 GiB).
static int check_prefill_shape(const char* what, const GemmArgs& a, const w4a16_plan& p) {
    if (p.kernel == W4A16_KERNEL_PREFILL && !prefill_supported(a))
        return fail(W4A16_UNSUPPORTED_SHAPE,
                    "%s: the prefill kernel needs one expert's packed weights and the activation matrix below 2 GiB",
                    what);
    return W4A16_OK;
}

// MXFP4 weights run on the 16-row register-streaming decode kernel and on the prefill kernel.
static int check_format_plan(const char* what, const w4a16_weights* w, const w4a16_plan& p) {
    if (w->shape.fmt == kFmtMxfp4 && p.kernel == W4A16_KERNEL_DECODE && p.block_m != 16)
        return fail(W4A16_UNSUPPORTED_SHAPE, "%s: MXFP4 weights need decode block_m 16 (plan has %d)", what,
                    p.block_m);
    return W4A16_OK;
}

// W4A16_VALIDATE=1: the GEMM calls that take routing tensors check them on the device first and synchronise to
// read the status (a debugging mode).  The status word lives in a small static device array.
static __device__ int32_t validate_status[1];

static bool validate_mode() {
    static const bool on = [] {
        const char* v = getenv("W4A16_VALIDATE");
        return v && *v && strcmp(v, "0") != 0;
    }();
    return on;
}

static int validate_now(const char* what, const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntp,
                        int R, int E, int block_m, int max_padded, hipStream_t s) {
    void* st = nullptr;
    hipError_t err = hipGetSymbolAddress(&st, HIP_SYMBOL(validate_status));
    if (err == hipSuccess)
        err = launch_route_validate(nullptr, R, E, block_m, sorted_ids, expert_ids, ntp, max_padded,
                                    static_cast<int32_t*>(st), s);
    int32_t status = 0;
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err == hipSuccess) err = hipMemcpy(&status, st, sizeof(status), hipMemcpyDeviceToHost);
    if (err != hipSuccess) return fail(W4A16_HIP_ERROR, "%s: routing validation failed: %s", what, hipGetErrorString(err));
    if (status)
        return fail(W4A16_INVALID_ARG, "%s: routing tensors invalid (W4A16_VALIDATE status 0x%x)", what, (unsigned)status);
    return W4A16_OK;
}

static int grouped_gemm_impl(const char* what, const uint16_t* A, int a_row_div, const w4a16_weights* w,
                             const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntp, int R,
                             const w4a16_plan* p, void* out, int out_mode, void* ws, size_t ws_bytes,
                             hipStream_t s) {
    int rc = check_handle(w, what);
    if (rc) return rc;
    rc = validate_plan(p, what);
    if (rc) return rc;
    rc = check_format_plan(what, w, *p);
    if (rc) return rc;
    if (R < 0 || a_row_div < 1) return fail(W4A16_INVALID_ARG, "%s: R=%d a_row_div=%d", what, R, a_row_div);
    if (R == 0) return ok();
    if (R % a_row_div) return fail(W4A16_INVALID_ARG, "%s: R=%d not a multiple of a_row_div=%d", what, R, a_row_div);
    if (!A || !sorted_ids || !expert_ids || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    if (!aligned16(A)) return fail(W4A16_INVALID_ARG, "%s: A must be 16-byte aligned", what);
    if (out_mode == kOutAct) {
        if (w->shape.N % 32)
            return fail(W4A16_UNSUPPORTED_SHAPE, "%s: N=%d must be a multiple of 32 (gate and up halves of whole n-blocks)",
                        what, w->shape.N);
        if (p->n_blocks < 2) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: plan.n_blocks must be at least 2", what);
    }
    int maxP, maxB;
    route_bounds(R / a_row_div, a_row_div, w->shape.E, p->block_m, &maxP, &maxB);
    const GemmWs g = gemm_ws(w->shape, *p, maxB);
    if (g.total && (!ws || ws_bytes < g.total))
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, needs %zu", what, ws_bytes, g.total);
    if (g.total && !aligned16(ws)) return fail(W4A16_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);
    GemmArgs a{A, a_row_div, w->packed, w->shape, sorted_ids, expert_ids, R, maxB, out, out_mode};
    a.ntp = ntp;
    rc = check_prefill_shape(what, a, *p);
    if (rc) return rc;
    if (validate_mode() && ntp) {
        rc = validate_now(what, sorted_ids, expert_ids, ntp, R, w->shape.E, p->block_m, maxP, s);
        if (rc) return rc;
    }
    bind_ws(a, g, ws);
    return check_launch(run_gemm(a, *p, s), what);
}

int w4a16_grouped_gemm(const uint16_t* A, int a_row_div, const w4a16_weights* w, const int32_t* sorted_ids,
                       const int32_t* expert_ids, const int32_t* num_tokens_padded, int R, const w4a16_plan* p,
                       uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s) {
    return grouped_gemm_impl("w4a16_grouped_gemm", A, a_row_div, w, sorted_ids, expert_ids, num_tokens_padded, R, p,
                             out, kOutBf16, ws, ws_bytes, s);
}

int w4a16_grouped_gemm_f32(const uint16_t* A, int a_row_div, const w4a16_weights* w, const int32_t* sorted_ids,
                           const int32_t* expert_ids, const int32_t* num_tokens_padded, int R, const w4a16_plan* p,
                           float* out, void* ws, size_t ws_bytes, hipStream_t s) {
    return grouped_gemm_impl("w4a16_grouped_gemm_f32", A, a_row_div, w, sorted_ids, expert_ids, num_tokens_padded, R,
                             p, out, kOutF32, ws, ws_bytes, s);
}

int w4a16_grouped_gemm_silu(const uint16_t* A, int a_row_div, const w4a16_weights* w13, const int32_t* sorted_ids,
                            const int32_t* expert_ids, const int32_t* num_tokens_padded, int R, const w4a16_plan* p,
                            uint16_t* h, void* ws, size_t ws_bytes, hipStream_t s) {
    return grouped_gemm_impl("w4a16_grouped_gemm_silu", A, a_row_div, w13, sorted_ids, expert_ids, num_tokens_padded,
                             R, p, h, kOutAct, ws, ws_bytes, s);
}

// Offsets-form workspace: [split-K area][sorted_ids][expert_ids][num_tokens_padded].
static size_t offsets_layout(int rows_max, const w4a16_weights* w, const w4a16_plan* p, size_t* off_sorted,
                             size_t* off_eids, size_t* off_ntp, int* maxP, int* maxB, GemmWs* g) {
    route_bounds(rows_max, 1, w->shape.E, p->block_m, maxP, maxB);
    *g = gemm_ws(w->shape, *p, *maxB);
    *off_sorted = g->total;
    *off_eids = *off_sorted + align_up(sizeof(int32_t) * (size_t)*maxP, 256);
    *off_ntp = *off_eids + align_up(sizeof(int32_t) * (size_t)*maxB, 256);
    return *off_ntp + 256;
}

int w4a16_offsets_workspace_bytes(int rows_max, const w4a16_weights* w, const w4a16_plan* p, size_t* bytes) {
    const char* what = "w4a16_offsets_workspace_bytes";
    int rc = check_handle(w, what);
    if (rc) return rc;
    rc = validate_plan(p, what);
    if (rc) return rc;
    if (!bytes || rows_max < 0) return fail(W4A16_INVALID_ARG, "%s: bad argument", what);
    size_t a, b, c;
    int maxP, maxB;
    GemmWs g;
    *bytes = offsets_layout(rows_max, w, p, &a, &b, &c, &maxP, &maxB, &g);
    return ok();
}

int w4a16_grouped_gemm_offsets(const uint16_t* A_sorted, const int32_t* expert_offsets, int rows_max,
                               const w4a16_weights* w, const w4a16_plan* p, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t s) {
    const char* what = "w4a16_grouped_gemm_offsets";
    int rc = check_handle(w, what);
    if (rc) return rc;
    rc = validate_plan(p, what);
    if (rc) return rc;
    rc = check_format_plan(what, w, *p);
    if (rc) return rc;
    if (rows_max < 0) return fail(W4A16_INVALID_ARG, "%s: rows_max=%d", what, rows_max);
    if (w->shape.E > W4A16_MAX_EXPERTS) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: too many experts", what);
    if (rows_max == 0) return ok();
    size_t off_sorted, off_eids, off_ntp;
    int maxP, maxB;
    GemmWs g;
    const size_t need = offsets_layout(rows_max, w, p, &off_sorted, &off_eids, &off_ntp, &maxP, &maxB, &g);
    if (!ws || ws_bytes < need)
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, needs %zu", what, ws_bytes, need);
    if (!aligned16(ws)) return fail(W4A16_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);
    if (!A_sorted || !expert_offsets || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    if (!aligned16(A_sorted)) return fail(W4A16_INVALID_ARG, "%s: A_sorted must be 16-byte aligned", what);
    int32_t* sorted_ids = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off_sorted);
    int32_t* expert_ids = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off_eids);
    int32_t* ntp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off_ntp);
    GemmArgs a{A_sorted, 1, w->packed, w->shape, sorted_ids, expert_ids, rows_max, maxB, out, kOutBf16};
    a.ntp = ntp;
    rc = check_prefill_shape(what, a, *p);
    if (rc) return rc;
    rc = check_launch(launch_offsets_to_route(expert_offsets, w->shape.E, rows_max, p->block_m, maxP, maxB, sorted_ids,
                                              expert_ids, ntp, s),
                      what);
    if (rc) return rc;
    bind_ws(a, g, ws);
    return check_launch(run_gemm(a, *p, s), what);
}

// Masked form: rows [e*max_m, e*max_m + masked_m[e]) of a [E*max_m, K] activation block belong to expert e; the
// routing tensors are built on the device in the offsets-form workspace layout.
int w4a16_masked_workspace_bytes(int max_m, const w4a16_weights* w, const w4a16_plan* p, size_t* bytes) {
    const char* what = "w4a16_masked_workspace_bytes";
    int rc = check_handle(w, what);
    if (rc) return rc;
    if (max_m < 0 || (long)max_m * w->shape.E > INT32_MAX)
        return fail(W4A16_INVALID_ARG, "%s: max_m=%d", what, max_m);
    return w4a16_offsets_workspace_bytes(max_m * w->shape.E, w, p, bytes);
}

int w4a16_grouped_gemm_masked(const uint16_t* A, const int32_t* masked_m, int max_m, const w4a16_weights* w,
                              const w4a16_plan* p, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s) {
    const char* what = "w4a16_grouped_gemm_masked";
    int rc = check_handle(w, what);
    if (rc) return rc;
    rc = validate_plan(p, what);
    if (rc) return rc;
    rc = check_format_plan(what, w, *p);
    if (rc) return rc;
    const int E = w->shape.E;
    if (max_m < 0 || (long)max_m * E > INT32_MAX) return fail(W4A16_INVALID_ARG, "%s: max_m=%d", what, max_m);
    if (E > W4A16_MAX_EXPERTS) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: too many experts", what);
    if (max_m == 0) return ok();
    const int rows = max_m * E;
    size_t off_sorted, off_eids, off_ntp;
    int maxP, maxB;
    GemmWs g;
    const size_t need = offsets_layout(rows, w, p, &off_sorted, &off_eids, &off_ntp, &maxP, &maxB, &g);
    if (!ws || ws_bytes < need)
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, needs %zu", what, ws_bytes, need);
    if (!aligned16(ws)) return fail(W4A16_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);
    if (!A || !masked_m || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    if (!aligned16(A)) return fail(W4A16_INVALID_ARG, "%s: A must be 16-byte aligned", what);
    int32_t* sorted_ids = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off_sorted);
    int32_t* expert_ids = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off_eids);
    int32_t* ntp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off_ntp);
    GemmArgs a{A, 1, w->packed, w->shape, sorted_ids, expert_ids, rows, maxB, out, kOutBf16};
    a.ntp = ntp;
    rc = check_prefill_shape(what, a, *p);
    if (rc) return rc;
    rc = check_launch(launch_masked_to_route(masked_m, E, max_m, p->block_m, maxP, maxB, sorted_ids, expert_ids, ntp, s),
                      what);
    if (rc) return rc;
    bind_ws(a, g, ws);
    return check_launch(run_gemm(a, *p, s), what);
}

// Contiguous form: row r of A belongs to expert m_indices[r] (-1, or any id outside [0,E): a padding row).  The
// rows are sorted by expert on the device exactly as routes are (one route per row), so neither the grouping nor
// the padding of the rows matters.  Workspace: [GEMM workspace][sorted_ids][expert_ids][num_tokens_padded]
// [expert_offsets][counts][routing scratch].
static size_t contiguous_layout(int m, const w4a16_weights* w, const w4a16_plan* p, size_t* off, int* maxP, int* maxB,
                                GemmWs* g) {
    const int E = w->shape.E;
    route_bounds(m, 1, E, p->block_m, maxP, maxB);
    *g = gemm_ws(w->shape, *p, *maxB);
    off[0] = g->total;                                                          // sorted_ids
    off[1] = off[0] + align_up(sizeof(int32_t) * (size_t)*maxP, 256);          // expert_ids
    off[2] = off[1] + align_up(sizeof(int32_t) * (size_t)*maxB, 256);          // num_tokens_padded
    off[3] = off[2] + 256;                                                      // expert_offsets
    off[4] = off[3] + align_up(sizeof(int32_t) * (size_t)(E + 1), 256);        // counts
    off[5] = off[4] + align_up(sizeof(int32_t) * (size_t)E, 256);              // routing scratch
    return off[5] + align_up(sizeof(int32_t) * route_prep_scratch_ints(m, E), 256);
}

int w4a16_contiguous_workspace_bytes(int m, const w4a16_weights* w, const w4a16_plan* p, size_t* bytes) {
    const char* what = "w4a16_contiguous_workspace_bytes";
    int rc = check_handle(w, what);
    if (rc) return rc;
    rc = validate_plan(p, what);
    if (rc) return rc;
    if (!bytes || m < 0) return fail(W4A16_INVALID_ARG, "%s: bad argument", what);
    size_t off[6];
    int maxP, maxB;
    GemmWs g;
    *bytes = contiguous_layout(m, w, p, off, &maxP, &maxB, &g);
    return ok();
}

int w4a16_grouped_gemm_contiguous(const uint16_t* A, const int32_t* m_indices, int m, const w4a16_weights* w,
                                  const w4a16_plan* p, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s) {
    const char* what = "w4a16_grouped_gemm_contiguous";
    int rc = check_handle(w, what);
    if (rc) return rc;
    rc = validate_plan(p, what);
    if (rc) return rc;
    rc = check_format_plan(what, w, *p);
    if (rc) return rc;
    const int E = w->shape.E;
    if (m < 0) return fail(W4A16_INVALID_ARG, "%s: m=%d", what, m);
    if (E > W4A16_MAX_EXPERTS) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: too many experts", what);
    if (m == 0) return ok();
    size_t off[6];
    int maxP, maxB;
    GemmWs g;
    const size_t need = contiguous_layout(m, w, p, off, &maxP, &maxB, &g);
    if (!ws || ws_bytes < need)
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, needs %zu", what, ws_bytes, need);
    if (!aligned16(ws)) return fail(W4A16_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);
    if (!A || !m_indices || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    if (!aligned16(A)) return fail(W4A16_INVALID_ARG, "%s: A must be 16-byte aligned", what);
    char* base = static_cast<char*>(ws);
    int32_t* sorted_ids = reinterpret_cast<int32_t*>(base + off[0]);
    int32_t* expert_ids = reinterpret_cast<int32_t*>(base + off[1]);
    int32_t* ntp = reinterpret_cast<int32_t*>(base + off[2]);
    GemmArgs a{A, 1, w->packed, w->shape, sorted_ids, expert_ids, m, maxB, out, kOutBf16};
    a.ntp = ntp;
    rc = check_prefill_shape(what, a, *p);
    if (rc) return rc;
    rc = check_launch(launch_route_prep_scratch(m_indices, m, E, p->block_m, maxP, maxB, sorted_ids, expert_ids, ntp,
                                                reinterpret_cast<int32_t*>(base + off[3]),
                                                reinterpret_cast<int32_t*>(base + off[4]),
                                                reinterpret_cast<int32_t*>(base + off[5]), s),
                      what);
    if (rc) return rc;
    bind_ws(a, g, ws);
    return check_launch(run_gemm(a, *p, s), what);
}

int w4a16_silu_mul(const uint16_t* gu, int rows, int I, uint16_t* h, hipStream_t s) {
    if (rows < 0 || I < 2 || I % 2) return fail(W4A16_INVALID_ARG, "w4a16_silu_mul: rows=%d I=%d (I must be even)", rows, I);
    if (rows == 0) return ok();
    if (!gu || !h) return fail(W4A16_INVALID_ARG, "w4a16_silu_mul: NULL pointer argument");
    if (((uintptr_t)gu & 3u) || ((uintptr_t)h & 3u)) return fail(W4A16_INVALID_ARG, "w4a16_silu_mul: buffers must be 4-byte aligned");
    return check_launch(launch_silu_mul(gu, rows, I, h, s), "w4a16_silu_mul");
}

int w4a16_silu_mul_f32(const float* gu, int rows, int I, uint16_t* h, hipStream_t s) {
    if (rows < 0 || I < 2 || I % 2) return fail(W4A16_INVALID_ARG, "w4a16_silu_mul_f32: rows=%d I=%d (I must be even)", rows, I);
    if (rows == 0) return ok();
    if (!gu || !h) return fail(W4A16_INVALID_ARG, "w4a16_silu_mul_f32: NULL pointer argument");
    if (((uintptr_t)gu & 7u) || ((uintptr_t)h & 3u)) return fail(W4A16_INVALID_ARG, "w4a16_silu_mul_f32: misaligned buffer");
    return check_launch(launch_silu_mul_f32(gu, rows, I, h, s), "w4a16_silu_mul_f32");
}

int w4a16_moe_combine(const float* y, const float* topk_w, const int32_t* topk_ids, int T, int k, int E, int H,
                      uint16_t* out, hipStream_t s) {
    if (T < 0 || k < 1 || E < 1 || H < 2 || H % 2)
        return fail(W4A16_INVALID_ARG, "w4a16_moe_combine: T=%d k=%d E=%d H=%d (H must be even)", T, k, E, H);
    if (T == 0) return ok();
    if (!y || !topk_w || !topk_ids || !out) return fail(W4A16_INVALID_ARG, "w4a16_moe_combine: NULL pointer argument");
    if (((uintptr_t)y & 7u) || ((uintptr_t)out & 3u)) return fail(W4A16_INVALID_ARG, "w4a16_moe_combine: misaligned buffer");
    return check_launch(launch_combine(y, topk_w, topk_ids, T, k, E, H, out, s), "w4a16_moe_combine");
}

int w4a16_moe_combine_bf16(const uint16_t* y, const float* topk_w, const int32_t* topk_ids, int T, int k, int E, int H,
                           uint16_t* out, hipStream_t s) {
    if (T < 0 || k < 1 || E < 1 || H < 2 || H % 2)
        return fail(W4A16_INVALID_ARG, "w4a16_moe_combine_bf16: T=%d k=%d E=%d H=%d (H must be even)", T, k, E, H);
    if (T == 0) return ok();
    if (!y || !topk_w || !topk_ids || !out)
        return fail(W4A16_INVALID_ARG, "w4a16_moe_combine_bf16: NULL pointer argument");
    if (((uintptr_t)y & 3u) || ((uintptr_t)out & 3u))
        return fail(W4A16_INVALID_ARG, "w4a16_moe_combine_bf16: misaligned buffer");
    return check_launch(launch_combine_bf16(y, topk_w, topk_ids, T, k, E, H, out, s), "w4a16_moe_combine_bf16");
}

// A decode step of 16-row blocks on the register-streaming kernel with at most kSelfRouteMaxRoutes routes routes its
// rows inside the gate_up kernel (every gate_up workgroup reads all the ids into LDS, so larger steps keep the
// routing launch).  With W4A16_PLAN_ONE_LAUNCH on the gate_up plan such a step also runs down in the same launch (down's
// workgroups of a route block start once gate_up has stored that block's rows of h; both route in-kernel) when
// down's plan is one too and both weight sets have one format.

static bool fused_self_route(int R, int E, const GemmArgs& g13, const w4a16_plan& p13) {
    return p13.kernel == W4A16_KERNEL_DECODE && p13.block_m == 16 && R <= kSelfRouteMaxRoutes &&
           E <= W4A16_MAX_EXPERTS && decode_reg_supported(g13, p13);
}

// Fused workspace.  Zero at rest, from offset 0: the sync words of the one-launch step (if it runs as one launch)
// and the split-K counters.  Two GEMMs in one launch each get their own split-K area; two GEMMs in consecutive
// launches share one (counters at the start, sized for the larger).  Then the routing tensors and intermediates.
struct FusedPlan {
    FusedLayout f;
    bool one_launch;
    size_t off_sync, off_c13, off_p13, off_c2, off_p2;  // one launch: both split areas; else off_c13/off_p13 shared
    size_t zero_bytes;                                   // [0, zero_bytes) holds everything that is zero at rest
};

static FusedPlan fused_full_layout(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                                   const w4a16_plan& p13, const w4a16_plan& p2) {
    const int E = w13->shape.E, H = w13->shape.K, I = w2->shape.K;
    const int R = T * k;
    int maxP, maxB;
    route_bounds(T, k, E, p13.block_m, &maxP, &maxB);
    const GemmWs a = gemm_ws(w13->shape, p13, maxB), b = gemm_ws(w2->shape, p2, maxB);
    GemmArgs g13{nullptr, k, nullptr, w13->shape, nullptr, nullptr, R, maxB, nullptr, kOutAct};
    GemmArgs g2{nullptr, 1, nullptr, w2->shape, nullptr, nullptr, R, maxB, nullptr, kOutBf16};
    FusedPlan fp;
    fp.one_launch = (p13.flags & W4A16_PLAN_ONE_LAUNCH) &&
                    ((fused_self_route(R, E, g13, p13) && decode_fused_supported(g13, p13, g2, p2)) ||
                     prefill_fused_supported(g13, p13, g2, p2));
    size_t head;
    if (fp.one_launch) {
        fp.off_sync = 0;
        fp.off_c13 = align_up(sizeof(unsigned) * (2 * (size_t)maxB + 1), 256);
        fp.off_c2 = fp.off_c13 + a.counter_bytes;
        fp.zero_bytes = fp.off_c2 + b.counter_bytes;
        fp.off_p13 = fp.zero_bytes;
        fp.off_p2 = fp.off_p13 + a.partial_bytes;
        head = fp.off_p2 + b.partial_bytes;
    } else {
        const size_t cb = a.counter_bytes > b.counter_bytes ? a.counter_bytes : b.counter_bytes;
        const size_t pb = a.partial_bytes > b.partial_bytes ? a.partial_bytes : b.partial_bytes;
        fp.off_sync = 0;
        fp.off_c13 = fp.off_c2 = 0;
        fp.off_p13 = fp.off_p2 = cb;
        fp.zero_bytes = cb;
        head = cb + pb;
    }
    const size_t tile_bytes = a.tile_bytes > b.tile_bytes ? a.tile_bytes : b.tile_bytes;
    fp.f = fused_layout(T, k, E, H, I, p13.block_m, head, tile_bytes);
    return fp;
}

// The two weight handles form an expert MLP and the two plans can run it: each valid on its own, one route block
// height (one set of routing tensors), one kernel family, n-blocks in pairs for the gate_up activation, one tile
// height for prefill, and decode plans of MXFP4 weights on 16-row blocks.
static int check_fused_plans(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                             const w4a16_plan* p13, const w4a16_plan* p2, const char* what) {
    int rc = check_handle(w13, what);
    if (rc) return rc;
    rc = check_handle(w2, what);
    if (rc) return rc;
    if (T < 0 || k < 1) return fail(W4A16_INVALID_ARG, "%s: T=%d k=%d", what, T, k);
    const int E = w13->shape.E, H = w13->shape.K, I = w2->shape.K;
    if (w2->shape.E != E || w13->shape.N != 2 * I || w2->shape.N != H)
        return fail(W4A16_LAYOUT_MISMATCH, "%s: w13 is [%d,%d,%d] and w2 is [%d,%d,%d]; need [E,2I,H] and [E,H,I]", what,
                    w13->shape.E, w13->shape.N, w13->shape.K, w2->shape.E, w2->shape.N, w2->shape.K);
    if (E > W4A16_MAX_EXPERTS) return fail(W4A16_UNSUPPORTED_SHAPE, "%s: E=%d exceeds %d", what, E, W4A16_MAX_EXPERTS);
    if (!p13 || !p2) return fail(W4A16_INVALID_ARG, "%s: plan is NULL", what);
    rc = validate_plan(p13, what);
    if (!rc) rc = validate_plan(p2, what);
    if (rc) return rc;
    if (p13->kernel != p2->kernel || p13->block_m != p2->block_m)
        return fail(W4A16_INVALID_ARG, "%s: gate_up and down plans must share kernel and block_m (one routing)", what);
    if (p13->n_blocks < 2) return fail(W4A16_INVALID_ARG, "%s: gate_up plan needs n_blocks >= 2", what);
    if (p13->kernel == W4A16_KERNEL_PREFILL && prefill_tile_rows(*p13) != prefill_tile_rows(*p2))
        return fail(W4A16_INVALID_ARG, "%s: prefill plans must share tile_m (one tile list)", what);
    rc = check_format_plan(what, w13, *p13);
    if (!rc) rc = check_format_plan(what, w2, *p2);
    return rc;
}

int w4a16_fused_moe_planned_workspace_bytes(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                                            const w4a16_plan* gate_up, const w4a16_plan* down, size_t* bytes) {
    const char* what = "w4a16_fused_moe_workspace_bytes";
    if (!bytes) return fail(W4A16_INVALID_ARG, "%s: bytes is NULL", what);
    int rc = check_fused_plans(T, k, w13, w2, gate_up, down, what);
    if (rc) return rc;
    *bytes = fused_full_layout(T, k, w13, w2, *gate_up, *down).f.total;
    return ok();
}

int w4a16_fused_moe_workspace_bytes(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2, size_t* bytes) {
    w4a16_plan p13, p2;
    int rc = w4a16_fused_moe_plans(T, k, w13, w2, &p13, &p2);
    if (rc) return rc;
    return w4a16_fused_moe_planned_workspace_bytes(T, k, w13, w2, &p13, &p2, bytes);
}

int w4a16_fused_moe_plans(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2, w4a16_plan* gate_up,
                          w4a16_plan* down) {
    return w4a16_fused_moe_plans_hint(T, k, w13, w2, 0.f, gate_up, down);
}

int w4a16_fused_moe_plans_hint(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                               float expected_rows_per_expert, w4a16_plan* gate_up, w4a16_plan* down) {
    const char* what = "w4a16_fused_moe_plans";
    int rc = check_handle(w13, what);
    if (rc) return rc;
    rc = check_handle(w2, what);
    if (rc) return rc;
    if (!gate_up || !down || k < 1 || T < 0) return fail(W4A16_INVALID_ARG, "%s: bad argument", what);
    const int E = w13->shape.E, H = w13->shape.K, I = w2->shape.K;
    w4a16_plan p13, p2;
    rc = w4a16_plan_select(T, k, E, 2 * I, H, expected_rows_per_expert, &p13);
    if (rc) return rc;
    rc = w4a16_plan_select(T, k, E, H, I, expected_rows_per_expert, &p2);
    if (rc) return rc;
    if (p13.n_blocks < 2) p13.n_blocks = 2;  // the activation epilogue pairs a gate and an up n-block
    p2.block_m = p13.block_m;  // both projections share one set of routing tensors
    p2.kernel = p13.kernel;
    if (p2.kernel == W4A16_KERNEL_PREFILL) {
        if (p2.n_blocks != 2 && p2.n_blocks != 4) p2.n_blocks = 4;
        p2.tile_m = p13.tile_m;
        p2.k_split = overrides().k_split ? overrides().k_split : 1;
    } else {
        if (p2.k_split < 1) p2.k_split = 1;
        p2.tile_m = 0;
    }
    rc = validate_plan(&p2, what);
    if (rc) return rc;
    // Prefill steps of tiled 16-row blocks run gate_up and down in one launch when the volume of h that down's column
    // tiles read, n_tiles(down) x R x I x 2 bytes, is below 2 GB: an empirical threshold.  Measured, fused step in one
    // launch against two: Qwen3-30B-A3B-shaped steps of 256 .. 4096 tokens 1.2 .. 6% faster (0.1 .. 0.8 GB), of 8192
    // tokens the same (1.6 GB); DeepSeek-V3-shaped steps of 512 and 1024 tokens 0.4% and 0.5% faster (0.9, 1.9 GB),
    // of 2048 and 4096 tokens 0.8% and 0.9% slower (3.8, 7.5 GB); the Kimi-K2 prefill share of 8192 tokens 0.7%
    // slower (R counts every route; about an eighth are local); with y in BF16, DeepSeek-V3-shaped 4096 tokens 1.0%
    // slower and the Kimi-K2 share the same.  The one launch fills the tail of gate_up's last
    // round with down's first workgroups and saves a launch gap, but every gate_up workgroup stores its rows of h
    // device-coherently and waits for them before it counts its tile ready; a step of many gate_up rounds pays that
    // more often than it gains at the one tail.  W4A16_ONE_LAUNCH=0 or 1 forces the choice where the plans allow it.
    if (p13.kernel == W4A16_KERNEL_PREFILL) {
        GemmArgs g13{nullptr, k, nullptr, w13->shape, nullptr, nullptr, T * k, 0, nullptr, kOutAct};
        GemmArgs g2{nullptr, 1, nullptr, w2->shape, nullptr, nullptr, T * k, 0, nullptr, kOutBf16};
        const double reread = (double)prefill_n_tiles(w2->shape, p2) * T * k * I * 2.0;
        const int force = overrides().one_launch;
        const bool want = force >= 0 ? force != 0 : reread < 2.0e9;
        if (want && prefill_fused_supported(g13, p13, g2, p2)) p13.flags |= W4A16_PLAN_ONE_LAUNCH;
    }
    *gate_up = p13;
    *down = p2;
    return ok();
}

int w4a16_fused_moe(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                    const w4a16_weights* w13, const w4a16_weights* w2, uint16_t* out, void* ws, size_t ws_bytes,
                    hipStream_t s) {
    return w4a16_fused_moe_profiled(x, topk_ids, topk_w, T, k, w13, w2, out, ws, ws_bytes, s, nullptr);
}

int w4a16_fused_moe_profiled(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                             const w4a16_weights* w13, const w4a16_weights* w2, uint16_t* out, void* ws,
                             size_t ws_bytes, hipStream_t s, hipEvent_t* ev) {
    w4a16_plan p13, p2;
    int rc = w4a16_fused_moe_plans(T, k, w13, w2, &p13, &p2);
    if (rc) return rc;
    return w4a16_fused_moe_planned(x, topk_ids, topk_w, T, k, w13, w2, &p13, &p2, out, ws, ws_bytes, s, ev);
}

int w4a16_fused_moe_planned(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                            const w4a16_weights* w13, const w4a16_weights* w2, const w4a16_plan* gate_up,
                            const w4a16_plan* down, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s,
                            hipEvent_t* ev) {
    const char* what = "w4a16_fused_moe";
    int rc = check_fused_plans(T, k, w13, w2, gate_up, down, what);
    if (rc) return rc;
    const int E = w13->shape.E, H = w13->shape.K, I = w2->shape.K;
    if (T == 0) return ok();
    if (!x || !topk_ids || !topk_w || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    if (!aligned16(x) || ((uintptr_t)out & 3u)) return fail(W4A16_INVALID_ARG, "%s: x must be 16-byte aligned", what);
    const w4a16_plan p13 = *gate_up, p2 = *down;
    const FusedPlan fp = fused_full_layout(T, k, w13, w2, p13, p2);
    const FusedLayout& f = fp.f;
    if (!ws || ws_bytes < f.total)
        return fail(W4A16_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, needs %zu", what, ws_bytes, f.total);
    if (!aligned16(ws)) return fail(W4A16_INVALID_ARG, "%s: workspace must be 16-byte aligned", what);

    char* base = static_cast<char*>(ws);
    int32_t* sorted_ids = reinterpret_cast<int32_t*>(base + f.off_sorted);
    int32_t* expert_ids = reinterpret_cast<int32_t*>(base + f.off_eids);
    int32_t* ntp = reinterpret_cast<int32_t*>(base + f.off_ntp);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + f.off_offsets);
    int32_t* counts = reinterpret_cast<int32_t*>(base + f.off_counts);
    uint16_t* h = reinterpret_cast<uint16_t*>(base + f.off_h);
    uint16_t* y = reinterpret_cast<uint16_t*>(base + f.off_y);
    const int R = T * k;
    GemmArgs g13{x, k, w13->packed, w13->shape, sorted_ids, expert_ids, R, f.maxB, h, kOutAct};
    g13.ntp = ntp;
    GemmArgs g2{h, 1, w2->packed, w2->shape, sorted_ids, expert_ids, R, f.maxB, y, kOutBf16};
    g2.ntp = ntp;
    rc = check_prefill_shape(what, g13, p13);
    if (!rc) rc = check_prefill_shape(what, g2, p2);
    if (rc) return rc;

#define W4A16_STAGE(i)                                                                     \
    do {                                                                                   \
        if (ev) {                                                                          \
            hipError_t e_ = hipEventRecord(ev[i], s);                                      \
            if (e_ != hipSuccess)                                                          \
                return fail(W4A16_HIP_ERROR, "%s: event record failed: %s", what, hipGetErrorString(e_)); \
        }                                                                                  \
    } while (0)
    const bool self_route = fused_self_route(R, E, g13, p13);
    // prefill plans that gather route blocks into tiles: the routing writes the tile list too (from the per-expert
    // counts), and both GEMMs use it as it is
    TileOut to;
    if (!self_route && tiled_prefill(p13)) {
        to.group = prefill_tile_rows(p13) / p13.block_m;
        to.count = reinterpret_cast<int32_t*>(base + f.off_tiles);
        to.tiles = to.count + 4;
    }
    W4A16_STAGE(0);
    if (self_route) {
        g13.self_route_ids = topk_ids;
    } else {
        rc = check_launch(launch_route_prep_scratch(topk_ids, R, E, p13.block_m, f.maxP, f.maxB, sorted_ids, expert_ids,
                                                    ntp, offsets, counts, reinterpret_cast<int32_t*>(base + f.off_route),
                                                    s, to),
                          "w4a16_fused_moe (route_prep)");
        if (rc) return rc;
    }
    W4A16_STAGE(1);
    const GemmWs w13ws = gemm_ws(w13->shape, p13, f.maxB), w2ws = gemm_ws(w2->shape, p2, f.maxB);
    bind_ws(g13, w13ws, base + f.off_split + fp.off_c13, fp.off_p13 - fp.off_c13, base + f.off_tiles);
    bind_ws(g2, w2ws, base + f.off_split + fp.off_c2, fp.off_p2 - fp.off_c2, base + f.off_tiles);
    // both GEMMs tile the same routing the same way (one area, same route blocks and tile height): the tile list
    // the routing wrote serves both
    g13.tiles_ready = to.tiles != nullptr;
    g2.tiles_ready = to.tiles != nullptr && tiled_prefill(p2) && p13.block_m == p2.block_m &&
                     prefill_tile_rows(p13) == prefill_tile_rows(p2);
    if (fp.one_launch && p13.kernel == W4A16_KERNEL_PREFILL) {
        // gate_up and down in one launch: down's workgroups of a tile start once every gate_up column tile of that
        // tile has stored its rows of h, so down fills the chip while gate_up's last workgroups run (humans& page,
        // "Blackwell hides the conversion work")
        rc = check_launch(launch_gemm_prefill_fused(g13, p13, g2, p2,
                                                    reinterpret_cast<unsigned*>(base + f.off_split + fp.off_sync), s),
                          "w4a16_fused_moe (gate_up + silu_mul + down, one launch)");
        if (rc) return rc;
        W4A16_STAGE(2);
    } else if (fp.one_launch) {
        // gate_up and down in one launch: down's workgroups of a route block start once gate_up has stored that
        // block's rows of h (humans& page, "Blackwell hides the conversion work": the second GEMM's work begins
        // before the first one ends); both route their rows in-kernel, nothing writes the routing tensors
        g2.self_route_ids = topk_ids;
        g13.sorted_ids = g13.expert_ids = g2.sorted_ids = g2.expert_ids = nullptr;
        g13.ntp = g2.ntp = nullptr;
        rc = check_launch(launch_gemm_decode_fused(g13, p13, g2, p2,
                                                   reinterpret_cast<unsigned*>(base + f.off_split + fp.off_sync), s),
                          "w4a16_fused_moe (gate_up + silu_mul + down, one launch)");
        if (rc) return rc;
        W4A16_STAGE(2);
    } else {
        rc = check_launch(run_gemm(g13, p13, s), "w4a16_fused_moe (gate_up + silu_mul)");
        if (rc) return rc;
        W4A16_STAGE(2);
        rc = check_launch(run_gemm(g2, p2, s), "w4a16_fused_moe (down)");
        if (rc) return rc;
    }
    W4A16_STAGE(3);
    rc = check_launch(launch_combine_bf16(y, topk_w, topk_ids, T, k, E, H, out, s), "w4a16_fused_moe (combine)");
    if (rc) return rc;
    W4A16_STAGE(4);
#undef W4A16_STAGE
    return ok();
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation fused call

// The static scratch of w4a16_fused_moe_noalloc.  Each GPU holds its own copy at its own address; in host code the
// name is only a host-side stand-in, so host code uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[W4A16_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of scratch per device, set once

// Address of scratch on the current device, looked up once per device.
int scratch_address(void** out, const char* what) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(W4A16_HIP_ERROR, "%s: hipGetDevice failed: %s", what, hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices) return fail(W4A16_HIP_ERROR, "%s: device %d beyond %d", what, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || p == nullptr)
            return fail(W4A16_HIP_ERROR, "%s: hipGetSymbolAddress of the scratch failed: %s", what,
                        hipGetErrorString(err));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4A16_OK;
}
}  // namespace

extern "C" int w4a16_fused_moe_noalloc(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                                       const w4a16_weights* w13, const w4a16_weights* w2, uint16_t* out,
                                       hipStream_t s) {
    const char* what = "w4a16_fused_moe_noalloc";
    w4a16_plan p13, p2;
    int rc = w4a16_fused_moe_plans(T, k, w13, w2, &p13, &p2);
    if (rc) return rc;
    rc = check_fused_plans(T, k, w13, w2, &p13, &p2, what);
    if (rc) return rc;
    if (T == 0) return ok();
    const FusedPlan fp = fused_full_layout(T, k, w13, w2, p13, p2);
    const FusedLayout& f = fp.f;
    if (f.total > W4A16_NOALLOC_SCRATCH_BYTES)
        return fail(W4A16_WORKSPACE_TOO_SMALL,
                    "%s: T=%d k=%d needs %zu bytes of intermediates, the static scratch holds %zu; use "
                    "w4a16_fused_moe with a workspace",
                    what, T, k, f.total, (size_t)W4A16_NOALLOC_SCRATCH_BYTES);
    if (!x || !topk_ids || !topk_w || !out) return fail(W4A16_INVALID_ARG, "%s: NULL pointer argument", what);
    void* ws = nullptr;
    rc = scratch_address(&ws, what);
    if (rc) return rc;
    // the split-K counters and the one-launch step's sync words start at zero: the scratch keeps whatever the
    // last call left there
    if (fp.zero_bytes) {
        rc = check_launch(launch_zero_words(static_cast<uint32_t*>(ws), fp.zero_bytes / 4, s), what);
        if (rc) return rc;
    }
    return w4a16_fused_moe_planned(x, topk_ids, topk_w, T, k, w13, w2, &p13, &p2, out, ws,
                                   W4A16_NOALLOC_SCRATCH_BYTES, s, nullptr);
}
