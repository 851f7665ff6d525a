// Prefill grouped GEMM: many routed rows per expert, bound by the matrix cores.
//
// Design (MI355X-first):
//  * One workgroup per (route block of BM rows of one expert, WN*NBW
//    n-blocks).  The owning expert comes from expert_ids[block] in-kernel, so
//    no host synchronisation is needed (Chord page, "Two kernel families";
//    nf4 page, "How it works", finds tiles in-kernel the same way).
//  * The BM activation rows, gathered through sorted_ids, are staged in LDS
//    128 k at a time (rows padded by 16 bytes so the 16 rows read by one
//    MFMA fragment fall in distinct banks).
//  * The wavefronts split the workgroup's columns, so every weight is loaded
//    from HBM and dequantised exactly once per workgroup, in registers, and
//    fed straight to v_mfma_f32_16x16x32_bf16: dequantisation (about 2.9
//    VALU operations per weight) is amortised over BM rows (Chord page,
//    "Grouped SM90 kernels": a taller M tile amortises the INT4
//    dequantisation).
#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int KT = 128;            // k per LDS stage (half a superblock)
constexpr int LDA = KT + 8;        // padded LDS row, in BF16 elements

struct PrefillParams {
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
__global__ __launch_bounds__(256) void gemm_prefill_kernel(PrefillParams p) {
    constexpr int BM = 16 * MT;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
    __shared__ int srow[BM];

    const int b = blockIdx.x;
    const int e = p.expert_ids[b];
    if (e < 0 || e >= p.sh.E) return;  // unowned block (or ids from a larger expert count)
    const int WN = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const Shape sh = p.sh;
    const int K = sh.K;
    const int nbw0 = (blockIdx.y * WN + w) * NBW;

    for (int m = threadIdx.x; m < BM; m += blockDim.x) {
        const int sid = p.sorted_ids[b * BM + m];
        srow[m] = sid < p.R ? sid / p.a_row_div : -1;
    }

    f32x4 acc[MT][NBW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q) acc[mt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nhalves = (sh.G + 3) / 4;
    for (int hs = 0; hs < nhalves; ++hs) {
        const int kb = hs >> 1, h = hs & 1;
        __syncthreads();  // previous stage fully consumed (and srow ready on the first pass)
        // gather BM rows x 128 k into LDS: 16 chunks of 16 bytes per row
        for (int x = threadIdx.x; x < BM * 16; x += blockDim.x) {
            const int m = x >> 4, ch = x & 15;
            const int k0 = hs * KT + ch * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            const int row = srow[m];
            if (row >= 0 && k0 < K) v = *reinterpret_cast<const u32x4*>(p.A + (size_t)row * K + k0);
            *reinterpret_cast<u32x4*>(&As[m * LDA + ch * 8]) = v;
        }
        // this wavefront's weights for the stage
        u32x4 cw[NBW], sc[NBW];
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const int nb = nbw0 + q < sh.NB ? nbw0 + q : sh.NB - 1;
            const uint8_t* sbp = p.packed + (((size_t)e * sh.NB + nb) * sh.KB + kb) * SB_BYTES;
            cw[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sbp + h * 1024 + L * 16));
            sc[q] = *reinterpret_cast<const u32x4*>(sbp + SB_CODE_BYTES + j * 16);
        }
        __syncthreads();
        const int ngroups = min(4, sh.G - hs * 4);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (g < ngroups) {
                bf16x8 wf[NBW];
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    const float s = group_scale(sc[q], h * 4 + g);
                    wf[q] = dequant8(cw[q][g], s, -8.0f * s);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[(mt * 16 + j) * LDA + 32 * g + 8 * c]);
#pragma unroll
                    for (int q = 0; q < NBW; ++q) acc[mt][q] = mfma16(af, wf[q], acc[mt][q]);
                }
            }
        }
    }

    // epilogue: lane holds rows 4c + r of each 16-row tile, column j of each n-block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mt * 16 + 4 * c + r;
            const int sid = p.sorted_ids[b * BM + m];
            if (sid >= p.R) continue;
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
}

template <int MT, int NBW, bool F32>
hipError_t launch_t(const GemmArgs& a, int WN, hipStream_t s) {
    PrefillParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                    a.out};
    const int cols = WN * NBW;
    const dim3 grid(a.max_blocks, (a.sh.NB + cols - 1) / cols);
    hipLaunchKernelGGL((gemm_prefill_kernel<MT, NBW, F32>), grid, dim3(64 * WN), 0, s, p);
    return hipGetLastError();
}

template <bool F32>
hipError_t dispatch(const GemmArgs& a, int mt, int nbw, int WN, hipStream_t s) {
    if (nbw == 4 && mt == 4) return launch_t<4, 4, F32>(a, WN, s);
    if (nbw == 4 && mt == 8) return launch_t<8, 4, F32>(a, WN, s);
    if (nbw == 2 && mt == 8) return launch_t<8, 2, F32>(a, WN, s);
    if (nbw == 2 && mt == 4) return launch_t<4, 2, F32>(a, WN, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    if (a.max_blocks == 0) return hipSuccess;
    const int mt = p.block_m / 16;
    return a.out_f32 ? dispatch<true>(a, mt, p.n_blocks, p.waves, s) : dispatch<false>(a, mt, p.n_blocks, p.waves, s);
}

}  // namespace w4a16
