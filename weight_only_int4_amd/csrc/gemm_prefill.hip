// Prefill grouped GEMM: many routed rows per expert, bound by the matrix cores.
//
// Design (MI355X-first):
//  * One workgroup per (route block of BM rows of one expert, 4*NBW
//    n-blocks).  The owning expert comes from expert_ids[block] in-kernel, so
//    no host synchronisation is needed (Chord page, "Two kernel families";
//    nf4 page, "How it works", finds tiles in-kernel the same way).
//  * The BM activation rows, gathered through sorted_ids, are staged in LDS
//    128 k at a time, double-buffered: the next stage's rows are loaded while
//    the current stage is multiplied, one barrier per stage.  Rows are padded
//    by 16 bytes so the 16 rows read by one MFMA fragment fall in distinct
//    banks.
//  * The four wavefronts split the workgroup's columns, so every weight is
//    loaded from HBM and dequantised exactly once per workgroup, in
//    registers, and fed straight to v_mfma_f32_16x16x32_bf16; the next
//    stage's packed weights are in flight in a second register set while the
//    current one is used.  Dequantisation (about 2.9 VALU operations per
//    weight) is amortised over BM rows (Chord page, "Grouped SM90 kernels": a
//    taller M tile amortises the INT4 dequantisation) and overlaps the MFMAs
//    of the neighbouring group.
//  * The MFMA operand is bf16((q - 8) * s), the product rounded once.
#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int KT = 128;       // k per stage (4 scale groups, half a superblock)
constexpr int LDA = KT + 8;   // padded LDS row in BF16 elements
constexpr int kThreads = 256; // four wavefronts, each owning its own columns

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

template <int MT, int NBW, int OM>
__global__ __launch_bounds__(kThreads) void gemm_prefill_kernel(PrefillParams p) {
    static_assert(OM != kOutAct || NBW % 2 == 0, "the activation epilogue pairs gate and up n-blocks");
    constexpr int BM = 16 * MT;
    constexpr int XR = BM * (KT / 8) / kThreads;  // 16-byte activation pieces per thread per stage
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];
    __shared__ int srow[BM];
    __shared__ int ssid[BM];

    const int b = blockIdx.x;
    const int e = p.expert_ids[b];
    if (e < 0 || e >= p.sh.E) return;  // unowned block (or ids from a larger expert count)
    const Shape sh = p.sh;
    const int K = sh.K;
    constexpr int WN = kThreads / 64;
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const int wave_global = blockIdx.y * WN + w;  // column group of this wavefront
    const int nst = (sh.G + 3) / 4;

    for (int m = threadIdx.x; m < BM; m += kThreads) {
        const int sid = p.sorted_ids[b * BM + m];
        ssid[m] = sid < p.R ? sid : -1;
        srow[m] = sid < p.R ? sid / p.a_row_div : -1;
    }
    __syncthreads();

    const uint8_t* wbase[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        int nb;
        if (OM == kOutAct) {  // slots [0, NBW/2) read gate rows, the rest the matching up rows
            const int half = sh.NB / 2, o = wave_global * (NBW / 2) + q % (NBW / 2);
            nb = o < half ? (q < NBW / 2 ? o : half + o) : sh.NB - 1;
        } else {
            nb = wave_global * NBW + q < sh.NB ? wave_global * NBW + q : sh.NB - 1;
        }
        // clamped blocks compute discarded columns
        wbase[q] = p.packed + ((size_t)e * sh.NB + nb) * sh.KB * SB_BYTES;
    }

    auto load_x = [&](int st, u32x4* regs) {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int x = threadIdx.x + r * kThreads;
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
            const int x = threadIdx.x + r * kThreads;
            const int m = x >> 4, ch = x & 15;
            *reinterpret_cast<u32x4*>(&buf[m * LDA + ch * 8]) = regs[r];
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

    auto group = [&](const uint16_t* buf, int g, int gs, const u32x4* cw, const u32x4* sc) {
        bf16x8 wf[NBW];
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const float s = group_scale(sc[q], gs);
            wf[q] = dequant8(cw[q][g], s, -8.0f * s);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(&buf[(mt * 16 + j) * LDA + 32 * g + 8 * c]);
#pragma unroll
            for (int q = 0; q < NBW; ++q) acc[mt][q] = mfma16(af, wf[q], acc[mt][q]);
        }
    };
    u32x4 xr[XR];
    auto stage = [&](int st, const u32x4* cw, const u32x4* sc, u32x4* cwn, u32x4* scn) {
        const bool more = st + 1 < nst;
        if (more) {
            load_x(st + 1, xr);
            load_w(st + 1, cwn, scn);
        }
        const uint16_t* buf = As[st & 1];
        const int g0 = (st & 1) * 4;
        // a ragged last stage computes its padding groups too: their codes are 8 and scales 0 in the packed
        // image and their activations are zero in LDS, so they add exactly zero
#pragma unroll
        for (int g = 0; g < 4; ++g) group(buf, g, g0 + g, cw, sc);
        if (more) store_x(As[(st + 1) & 1], xr);
        __syncthreads();
    };

    u32x4 cwA[NBW], scA[NBW], cwB[NBW], scB[NBW];
    load_x(0, xr);
    load_w(0, cwA, scA);
    store_x(As[0], xr);
    __syncthreads();
    // pairs of stages alternate the two register sets (no copies between them)
    for (int st = 0; st < nst; st += 2) {
        stage(st, cwA, scA, cwB, scB);
        if (st + 1 < nst) stage(st + 1, cwB, scB, cwA, scA);
    }

    // epilogue: lane holds rows 4c + r of each 16-row tile, column j of each n-block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int sid = ssid[mt * 16 + 4 * c + r];
            if (sid < 0) continue;
            if (OM == kOutAct) {
                const int NO = sh.N / 2;
#pragma unroll
                for (int q = 0; q < NBW / 2; ++q) {
                    const int n = (wave_global * (NBW / 2) + q) * 16 + j;
                    if (n >= NO) continue;
                    static_cast<uint16_t*>(p.out)[(size_t)sid * NO + n] =
                        f32_to_bf16_bits(silu_mul(acc[mt][q][r], acc[mt][q + NBW / 2][r]));
                }
            } else {
#pragma unroll
                for (int q = 0; q < NBW; ++q) {
                    const int n = (wave_global * NBW + q) * 16 + j;
                    if (n >= sh.N) continue;
                    if (OM == kOutF32)
                        static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = acc[mt][q][r];
                    else
                        static_cast<uint16_t*>(p.out)[(size_t)sid * sh.N + n] = f32_to_bf16_bits(acc[mt][q][r]);
                }
            }
        }
}

template <int MT, int NBW, int OM>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
    PrefillParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                    a.out};
    constexpr int cols = (kThreads / 64) * NBW;
    const dim3 grid(a.max_blocks, (a.sh.NB + cols - 1) / cols);
    hipLaunchKernelGGL((gemm_prefill_kernel<MT, NBW, OM>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int OM>
hipError_t dispatch(const GemmArgs& a, int mt, int nbw, hipStream_t s) {
    if (nbw == 4 && mt == 4) return launch_t<4, 4, OM>(a, s);
    if (nbw == 4 && mt == 8) return launch_t<8, 4, OM>(a, s);
    if (nbw == 2 && mt == 8) return launch_t<8, 2, OM>(a, s);
    if (nbw == 2 && mt == 4) return launch_t<4, 2, OM>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    if (a.max_blocks == 0) return hipSuccess;
    const int mt = p.block_m / 16;
    switch (a.out_mode) {
        case kOutBf16: return dispatch<kOutBf16>(a, mt, p.n_blocks, s);
        case kOutF32: return dispatch<kOutF32>(a, mt, p.n_blocks, s);
        case kOutAct: return dispatch<kOutAct>(a, mt, p.n_blocks, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
