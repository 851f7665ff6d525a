// Decode grouped GEMM: few routed rows per expert, bound by the weight stream.
//
// Design (MI355X-first; the operand swap and tiny token tile follow the idea
// of Chord's decode profile, "H200 and Blackwell indexed decode", and the
// split-K program per (expert, N tile, K slice) of the nf4 page, "How it
// works"):
//  * One workgroup per (route block, group of n-blocks); its WK wavefronts
//    split the superblocks along K and add their partial sums through LDS, so
//    no atomics and the result is deterministic.
//  * Each wavefront streams its packed superblocks with 16-byte loads (one
//    fully coalesced 1 KiB read per half superblock) and never stages weights
//    in LDS.
//  * Per scale group of 32 k the raw codes enter the MFMA as BF16 values
//    128 + q (one mask/OR per two weights).  The accumulator input of that
//    MFMA is -136 * (group sum of the activations), itself produced by an
//    MFMA against a constant, so the MFMA returns sum x*(q-8) for the group;
//    one FMA per output then applies the group's scale.  This costs
//    ~1.5 VALU operations per weight at 16 rows, far below the ~2.9 of a full
//    per-weight dequantisation, which matters because the weight stream
//    runs at HBM speed.
#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

struct DecodeParams {
    const uint16_t* A;
    int a_row_div;
    const uint8_t* packed;
    Shape sh;
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    int R;
    void* out;
};

template <int MT, int NBW, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_decode_kernel(DecodeParams p) {
    constexpr int BM = 16 * MT;
    constexpr int COLS = NBW * 16;
    constexpr int LDR = COLS + 1;  // padded row of the reduction buffer
    extern __shared__ float red[];  // [WK][BM][LDR]

    const int b = blockIdx.x;
    const int e = p.expert_ids[b];
    if (e < 0 || e >= p.sh.E) return;  // unowned block (or ids from a larger expert count)
    const int WK = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const int nb0 = blockIdx.y * NBW;
    const Shape sh = p.sh;
    const int K = sh.K;

    const uint16_t* arow[MT];
    bool avalid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int sid = p.sorted_ids[b * BM + mt * 16 + j];
        avalid[mt] = sid < p.R;
        arow[mt] = p.A + (size_t)(avalid[mt] ? sid / p.a_row_div : 0) * K + 8 * c;
    }

    f32x4 acc[MT][NBW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q) acc[mt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 m136 = minus136();
    const bf16x8 xzero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    const int kb_begin = (w * sh.KB) / WK, kb_end = ((w + 1) * sh.KB) / WK;

    for (int kb = kb_begin; kb < kb_end; ++kb) {
        u32x4 cw0[NBW], cw1[NBW], sc[NBW];
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int nb = nb0 + q < sh.NB ? nb0 + q : sh.NB - 1;  // clamp: result discarded when out of range
            const uint8_t* sbp = p.packed + (((size_t)e * sh.NB + nb) * sh.KB + kb) * SB_BYTES;
            cw0[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sbp + L * 16));
            cw1[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sbp + 1024 + L * 16));
            sc[q] = *reinterpret_cast<const u32x4*>(sbp + SB_CODE_BYTES + j * 16);
        }
        const int ngroups = min(SB_GROUPS, sh.G - kb * SB_GROUPS);
#pragma unroll
        for (int g = 0; g < SB_GROUPS; ++g) {
            if (g < ngroups) {
                bf16x8 xf[MT];
                f32x4 xc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xf[mt] = avalid[mt] ? *reinterpret_cast<const bf16x8*>(arow[mt] + kb * SB_K + 32 * g) : xzero;
                    xc[mt] = mfma16(xf[mt], m136, zero);
                }
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    const uint32_t word = (g < 4) ? cw0[q][g] : cw1[q][g - 4];
                    const bf16x8 wf = biased_codes(word);
                    const float s = group_scale(sc[q], g);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const f32x4 d = mfma16(xf[mt], wf, xc[mt]);
                        acc[mt][q] += s * d;
                    }
                }
            }
        }
    }

    // cross-wavefront reduction through LDS, then coalesced stores
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[((size_t)w * BM + mt * 16 + 4 * c + r) * LDR + q * 16 + j] = acc[mt][q][r];
    __syncthreads();
    const int n_base = nb0 * 16;
    for (int idx = threadIdx.x; idx < BM * COLS; idx += blockDim.x) {
        const int m = idx / COLS, col = idx % COLS;
        const int n = n_base + col;
        if (n >= sh.N) continue;
        const int sid = p.sorted_ids[b * BM + m];
        if (sid >= p.R) continue;
        float v = 0.f;
        for (int ww = 0; ww < WK; ++ww) v += red[((size_t)ww * BM + m) * LDR + col];
        if (OUT_F32)
            static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = v;
        else
            static_cast<uint16_t*>(p.out)[(size_t)sid * sh.N + n] = f32_to_bf16_bits(v);
    }
}

template <int MT, int NBW, bool F32>
hipError_t launch_t(const GemmArgs& a, int WK, hipStream_t s) {
    DecodeParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                   a.out};
    const dim3 grid(a.max_blocks, (a.sh.NB + NBW - 1) / NBW);
    const size_t shmem = sizeof(float) * (size_t)WK * 16 * MT * (NBW * 16 + 1);
    hipLaunchKernelGGL((gemm_decode_kernel<MT, NBW, F32>), grid, dim3(64 * WK), shmem, s, p);
    return hipGetLastError();
}

template <int MT, bool F32>
hipError_t dispatch_nbw(const GemmArgs& a, int nbw, int WK, hipStream_t s) {
    switch (nbw) {
        case 1: return launch_t<MT, 1, F32>(a, WK, s);
        case 2: return launch_t<MT, 2, F32>(a, WK, s);
        case 4: return launch_t<MT, 4, F32>(a, WK, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool F32>
hipError_t dispatch_mt(const GemmArgs& a, int mt, int nbw, int WK, hipStream_t s) {
    switch (mt) {
        case 1: return dispatch_nbw<1, F32>(a, nbw, WK, s);
        case 2: return dispatch_nbw<2, F32>(a, nbw, WK, s);
        case 3: return dispatch_nbw<3, F32>(a, nbw, WK, s);
        case 4: return dispatch_nbw<4, F32>(a, nbw, WK, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    if (a.max_blocks == 0) return hipSuccess;
    const int mt = p.block_m / 16;
    return a.out_f32 ? dispatch_mt<true>(a, mt, p.n_blocks, p.waves, s)
                     : dispatch_mt<false>(a, mt, p.n_blocks, p.waves, s);
}

}  // namespace w4a16
