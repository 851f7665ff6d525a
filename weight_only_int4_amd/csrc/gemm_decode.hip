// Decode grouped GEMM: few routed rows per expert, bound by the weight stream.
//
// Design (MI355X-first; the operand swap and tiny token tile follow the idea
// of Chord's decode profile, "H200 and Blackwell indexed decode", and the
// split-K program per (expert, N tile, K slice) of the nf4 page, "How it
// works"):
//  * One workgroup per (route block of BM rows, 16*NBW*WN output columns,
//    K slice).  Its WN wavefronts own disjoint columns and walk the same K
//    range in stages of 128 k, so the BM activation rows of a stage are
//    gathered once into LDS (double-buffered, one barrier per stage) and read
//    by every wavefront.
//  * Each wavefront streams its packed superblocks with 16-byte loads (one
//    fully coalesced 1 KiB read per half superblock per n-block) and keeps the
//    next stage's weights in flight in registers while it computes the
//    current one; weights never go through LDS.
//  * Per scale group of 32 k the raw codes enter the MFMA as BF16 values
//    128 + q (one mask/OR per two weights).  The accumulator input of that
//    MFMA is -136 * (group sum of the activations), itself produced by an
//    MFMA against a constant, so the MFMA returns sum x*(q-8) for the group
//    exactly as the products are exact; one FMA per output then applies the
//    group's scale.  That is ~1.5 VALU operations per weight at 16 rows,
//    against ~2.9 for a full per-weight dequantisation.
//  * When few workgroups exist (a handful of active experts), the K range is
//    split across KS workgroups (grid.z).  Each writes its fp32 partial tile
//    to the workspace with device-coherent (write-through) stores, waits for
//    them to complete, and bumps a per-tile counter; the last to arrive adds
//    the KS partials in a fixed order with device-coherent loads and writes
//    the output, so the result does not depend on arrival order, and resets
//    the counter for the next call.  Per-access coherence avoids a
//    device-scope fence, which on this chip writes back the whole L2 of the
//    issuing XCD.
#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int KT = 128;       // k per stage (4 scale groups, half a superblock)
constexpr int LDX = KT + 8;   // padded LDS row in BF16 elements (16 rows of a fragment hit distinct banks)

struct DecodeParams {
    const uint16_t* A;
    int a_row_div;
    const uint8_t* packed;
    Shape sh;
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    int R;
    void* out;
    float* partials;      // [max_blocks][n_tiles][KS][BM][COLS] when KS > 1
    unsigned* counters;   // [max_blocks][n_tiles] when KS > 1, zero between calls
};

constexpr int kDecodeThreads = 256;  // four wavefronts, each owning its own columns

template <int MT, int NBW, bool OUT_F32>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_kernel(DecodeParams p) {
    constexpr int BM = 16 * MT;
    constexpr int CHUNKS = BM * (KT / 8);        // 16-byte pieces of one activation stage
    constexpr int XR = CHUNKS / kDecodeThreads;  // pieces per thread (exact: CHUNKS = 256 * MT)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * LDX];
    __shared__ int srow[BM];
    __shared__ int ssid[BM];
    __shared__ int s_last;

    const int b = blockIdx.x;
    const int e = p.expert_ids[b];
    if (e < 0 || e >= p.sh.E) return;  // unowned block (or ids from a larger expert count)
    const Shape sh = p.sh;
    const int K = sh.K;
    constexpr int WN = kDecodeThreads / 64;
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const int nbw0 = (blockIdx.y * WN + w) * NBW;  // first n-block of this wavefront
    const int KS = gridDim.z, ks = blockIdx.z;
    const int nst = (sh.G + 3) / 4;
    const int st_begin = (int)((long)ks * nst / KS), st_end = (int)((long)(ks + 1) * nst / KS);

    for (int m = threadIdx.x; m < BM; m += blockDim.x) {
        const int sid = p.sorted_ids[b * BM + m];
        ssid[m] = sid < p.R ? sid : -1;
        srow[m] = sid < p.R ? sid / p.a_row_div : -1;
    }
    __syncthreads();

    // per-wavefront packed superblock rows (clamped n-blocks compute discarded columns)
    const uint8_t* wbase[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        const int nb = nbw0 + q < sh.NB ? nbw0 + q : sh.NB - 1;
        wbase[q] = p.packed + ((size_t)e * sh.NB + nb) * sh.KB * SB_BYTES;
    }

    auto load_x = [&](int st, u32x4* regs) {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int x = threadIdx.x + r * kDecodeThreads;
            const int m = x >> 4, ch = x & 15;
            const int k0 = st * KT + ch * 8;
            const int row = srow[m];
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row >= 0 && k0 < K) v = *reinterpret_cast<const u32x4*>(p.A + (size_t)row * K + k0);
            regs[r] = v;
        }
    };
    auto store_x = [&](uint16_t* buf, const u32x4* regs) {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int x = threadIdx.x + r * kDecodeThreads;
            const int m = x >> 4, ch = x & 15;
            *reinterpret_cast<u32x4*>(&buf[m * LDX + ch * 8]) = regs[r];
        }
    };
    auto load_w = [&](int st, u32x4* cw, u32x4* sc) {
        const int kb = st >> 1, h = st & 1;
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const uint8_t* sbp = wbase[q] + (size_t)kb * SB_BYTES;
            cw[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sbp + h * 1024 + L * 16));
            sc[q] = *reinterpret_cast<const u32x4*>(sbp + SB_CODE_BYTES + j * 16);
        }
    };

    f32x4 acc[MT][NBW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q) acc[mt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 m136 = minus136();

    // one scale group: gate the whole group on a uniform predicate only for a ragged last stage
    auto group = [&](const uint16_t* buf, int g, int gs, const u32x4* cw, const u32x4* sc) {
        bf16x8 xf[MT];
        f32x4 xc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            xf[mt] = *reinterpret_cast<const bf16x8*>(&buf[(mt * 16 + j) * LDX + 32 * g + 8 * c]);
            xc[mt] = mfma16(xf[mt], m136, zero);
        }
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const bf16x8 wf = biased_codes(cw[q][g]);
            const float s = group_scale(sc[q], gs);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 d = mfma16(xf[mt], wf, xc[mt]);
                acc[mt][q] += s * d;
            }
        }
    };
    // One stage: start the next stage's loads into the other register set, compute this stage, then publish
    // the next activation tile.  Two named register sets alternate, so no register copy forces the
    // prefetched loads to complete early.
    u32x4 xr[XR];
    auto stage = [&](int st, const u32x4* cw, const u32x4* sc, u32x4* cwn, u32x4* scn) {
        const bool more = st + 1 < st_end;
        if (more) {
            load_x(st + 1, xr);
            load_w(st + 1, cwn, scn);
        }
        const int cur = (st - st_begin) & 1;
        const uint16_t* buf = xs[cur];
        const int g0 = (st & 1) * 4;
        if (st * 4 + 4 <= sh.G) {
#pragma unroll
            for (int g = 0; g < 4; ++g) group(buf, g, g0 + g, cw, sc);
        } else {
            const int ng = sh.G - st * 4;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (g < ng) group(buf, g, g0 + g, cw, sc);
        }
        if (more) store_x(xs[cur ^ 1], xr);
        __syncthreads();
    };

    u32x4 cwA[NBW], scA[NBW], cwB[NBW], scB[NBW];
    if (st_begin < st_end) {
        load_x(st_begin, xr);
        load_w(st_begin, cwA, scA);
        store_x(xs[0], xr);
    }
    __syncthreads();
    for (int st = st_begin; st < st_end; st += 2) {
        stage(st, cwA, scA, cwB, scB);
        if (st + 1 < st_end) stage(st + 1, cwB, scB, cwA, scA);
    }

    const int COLS = NBW * 16 * WN;  // columns of the workgroup
    if (KS == 1) {
        // lane holds rows 4c + r of each 16-row tile, column j of each of its n-blocks
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int sid = ssid[mt * 16 + 4 * c + r];
                if (sid < 0) continue;
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    const int n = (nbw0 + q) * 16 + j;
                    if (nbw0 + q >= sh.NB || n >= sh.N) continue;
                    if (OUT_F32)
                        static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = acc[mt][q][r];
                    else
                        static_cast<uint16_t*>(p.out)[(size_t)sid * sh.N + n] = f32_to_bf16_bits(acc[mt][q][r]);
                }
            }
        return;
    }

    // split K: publish the partial tile, the last workgroup of the tile reduces in ks order
    const size_t tile = (size_t)b * gridDim.y + blockIdx.y;
    float* mine = p.partials + (tile * KS + ks) * (size_t)(BM * COLS);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(&mine[(mt * 16 + 4 * c + r) * COLS + (w * NBW + q) * 16 + j], acc[mt][q][r],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the stores above are device-coherent; wait until they have completed before signalling
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)(KS - 1);
    }
    __syncthreads();
    if (!s_last) return;
    const float* all = p.partials + tile * KS * (size_t)(BM * COLS);
    const int n_base = blockIdx.y * COLS;
    for (int idx = threadIdx.x; idx < BM * COLS; idx += kDecodeThreads) {
        const int m = idx / COLS, col = idx % COLS;
        const int sid = ssid[m];
        const int n = n_base + col;
        if (sid < 0 || n >= sh.N) continue;
        float v = 0.f;
        for (int z = 0; z < KS; ++z)
            v += __hip_atomic_load(&all[(size_t)z * BM * COLS + idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (OUT_F32)
            static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = v;
        else
            static_cast<uint16_t*>(p.out)[(size_t)sid * sh.N + n] = f32_to_bf16_bits(v);
    }
    if (threadIdx.x == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int NBW, bool F32>
hipError_t launch_t(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    DecodeParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                   a.out, a.partials, a.counters};
    const dim3 grid(a.max_blocks, decode_n_tiles(a.sh, pl), pl.k_split);
    hipLaunchKernelGGL((gemm_decode_kernel<MT, NBW, F32>), grid, dim3(kDecodeThreads), 0, s, p);
    return hipGetLastError();
}

template <int MT, bool F32>
hipError_t dispatch_nbw(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    switch (pl.n_blocks) {
        case 1: return launch_t<MT, 1, F32>(a, pl, s);
        case 2: return launch_t<MT, 2, F32>(a, pl, s);
        case 4: return launch_t<MT, 4, F32>(a, pl, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool F32>
hipError_t dispatch_mt(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    switch (pl.block_m / 16) {
        case 1: return dispatch_nbw<1, F32>(a, pl, s);
        case 2: return dispatch_nbw<2, F32>(a, pl, s);
        case 3: return dispatch_nbw<3, F32>(a, pl, s);
        case 4: return dispatch_nbw<4, F32>(a, pl, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int decode_n_tiles(const Shape& sh, const w4a16_plan& p) {
    const int cols = p.n_blocks * p.waves;
    return (sh.NB + cols - 1) / cols;
}

size_t decode_partial_floats(const Shape& sh, const w4a16_plan& p, int max_blocks) {
    if (p.kernel != W4A16_KERNEL_DECODE || p.k_split <= 1) return 0;
    return (size_t)max_blocks * decode_n_tiles(sh, p) * p.k_split * p.block_m * (p.n_blocks * 16 * p.waves);
}

size_t decode_counters(const Shape& sh, const w4a16_plan& p, int max_blocks) {
    if (p.kernel != W4A16_KERNEL_DECODE || p.k_split <= 1) return 0;
    return (size_t)max_blocks * decode_n_tiles(sh, p);
}

hipError_t launch_gemm_decode(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    if (a.max_blocks == 0) return hipSuccess;
    return a.out_f32 ? dispatch_mt<true>(a, p, s) : dispatch_mt<false>(a, p, s);
}

}  // namespace w4a16
