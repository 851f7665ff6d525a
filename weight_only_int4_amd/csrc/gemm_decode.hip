// Decode grouped GEMM: few routed rows per expert, bound by the weight stream.
// This file holds the LDS-staged kernel, used for route blocks of 32 to 64
// rows; one 16-row tile per workgroup goes to the register-streaming kernel
// of gemm_decode_reg.hip.
//
// Design (MI355X-first; the operand swap and tiny token tile follow the idea
// of Chord's decode profile, "H200 and Blackwell indexed decode", and the
// split-K program per (expert, N tile, K slice) of the nf4 page, "How it
// works"):
//  * One workgroup per (route block of BM rows, 64*NBW output columns, K
//    slice); its four wavefronts own disjoint columns and walk the same K range
//    in stages of 128 k.
//  * Both operands stream HBM -> LDS with direct global-to-LDS loads
//    (global_load_lds_dwordx4) into a ring of D stage slots, so D-1 stages are
//    in flight per wavefront without holding a single register.  Each lane
//    reads back exactly the 16 bytes it loaded (weights: the B fragment of its
//    column and k-slot; activations: its own piece of the shared tile), so a
//    wavefront only waits on its own load counter, and one barrier per stage
//    publishes the activation tile and frees the oldest slot.
//  * The activation tile is stored unpadded with the 16-byte chunks of row r
//    XOR-permuted by r mod 16, so the 16 rows of an MFMA fragment hit 16
//    distinct bank groups.
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
#include "decode_common.h"

namespace w4a16 {
using namespace decode;
namespace {


// 16 zero bytes: the source of activation pieces past the end of K
__device__ const u32x4 kZero16 = {0u, 0u, 0u, 0u};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most `later` stages of OPS loads each are still in flight (later <= D - 2 <= 4)
template <int D, int OPS>
__device__ __forceinline__ void wait_stage(int later) {
    switch (later) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<(D - 2 >= 1 ? 1 : 0) * OPS>(); break;
        case 2: wait_vmcnt<(D - 2 >= 2 ? 2 : 0) * OPS>(); break;
        case 3: wait_vmcnt<(D - 2 >= 3 ? 3 : 0) * OPS>(); break;
        default: wait_vmcnt<(D - 2 >= 4 ? 4 : 0) * OPS>(); break;
    }
}

// Barrier between stages.  __syncthreads() would also drain every direct load still in flight (the
// workgroup release fence counts them as pending LDS writes), which would empty the ring; instead each
// wavefront has already waited for its own loads of the stage, and here only its LDS reads of the previous
// stage must be complete before another wavefront refills that slot.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");  // no LDS access moves across the barrier
}

template <int MT, int NBW>
struct DecodeLds {
    static constexpr int BM = 16 * MT;
    static constexpr int X_BYTES = BM * KT * 2;                 // one activation stage
    static constexpr int W_BYTES = NBW * 1024 + 1024;           // one wavefront's codes of one stage + scale rows
    static constexpr int SLOT = X_BYTES + kWaves * W_BYTES;
};

template <int MT, int NBW, int D, int OM>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_kernel(DecodeParams p) {
    static_assert(OM != kOutAct || NBW % 2 == 0, "the activation epilogue pairs gate and up n-blocks");
    using Lay = DecodeLds<MT, NBW>;
    constexpr int BM = Lay::BM;
    constexpr int OPS = MT + NBW + 1;  // direct loads a wavefront issues per stage
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int srow[BM];
    __shared__ int ssid[BM];
    __shared__ int s_last;

    const int b = blockIdx.x;
    const int e = p.expert_ids[b];
    if (e < 0 || e >= p.sh.E) return;  // unowned block (or ids from a larger expert count)
    const Shape sh = p.sh;
    const int K = sh.K;
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const int wave_global = blockIdx.y * kWaves + w;  // column group of this wavefront
    const int KS = gridDim.z, ks = blockIdx.z;
    const int nst = (sh.G + 3) / 4;
    const int st_begin = (int)((long)ks * nst / KS), st_end = (int)((long)(ks + 1) * nst / KS);

    for (int m = threadIdx.x; m < BM; m += kDecodeThreads) {
        const int sid = p.sorted_ids[b * BM + m];
        ssid[m] = sid < p.R ? sid : -1;
        srow[m] = sid < p.R ? sid / p.a_row_div : -1;
    }
    __syncthreads();

    // per-lane sources of the activation pieces: piece r of this wavefront covers row
    // m = 4*(w*MT + r) + L/16 and LDS chunk L%16, which holds global chunk (L%16) ^ (m%16).
    // A sentinel row reads a valid row instead (rows are independent; its results are discarded).
    const int any_row = srow[0] >= 0 ? srow[0] : 0;
    const uint16_t* xsrc[MT];
#pragma unroll
    for (int r = 0; r < MT; ++r) {
        const int m = 4 * (w * MT + r) + (L >> 4);
        const int row = srow[m] >= 0 ? srow[m] : any_row;
        const int ch = (L & 15) ^ (m & 15);
        xsrc[r] = p.A + (size_t)row * K + ch * 8;
    }
    const uint8_t* wbase[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        int o;
        const int nb = slot_nblock<NBW, OM>(sh, wave_global, q, &o);
        wbase[q] = p.packed + ((size_t)e * sh.NB + nb) * sh.KB * SB_BYTES;
    }

    // this lane's scale row for the gathered scale load (see issue())
    const uint8_t* sbase;
    {
        const int ql = (L >> 4) < NBW ? (L >> 4) : NBW - 1;
        int o;
        const int nb = slot_nblock<NBW, OM>(sh, wave_global, ql, &o);
        sbase = p.packed + ((size_t)e * sh.NB + nb) * sh.KB * SB_BYTES + SB_CODE_BYTES + (L & 15) * 16;
    }

    auto slot_of = [&](int st) { return smem + (size_t)((st - st_begin) % D) * Lay::SLOT; };
    // issue this wavefront's direct loads of stage st (OPS instructions, in a fixed order)
    auto issue = [&](int st) {
        uint8_t* sl = slot_of(st);
#pragma unroll
        for (int r = 0; r < MT; ++r) {
            const int k0 = st * KT + ((L & 15) ^ ((4 * (w * MT + r) + (L >> 4)) & 15)) * 8;
            const void* src = k0 < K ? (const void*)(xsrc[r] + st * KT) : (const void*)&kZero16;
            dma16(src, sl + (4 * (w * MT + r)) * (KT * 2));
        }
        const int kb = st >> 1, h = st & 1;
        uint8_t* wsl = sl + Lay::X_BYTES + w * Lay::W_BYTES;
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const uint8_t* sbp = wbase[q] + (size_t)kb * SB_BYTES;
            dma16(sbp + h * 1024 + L * 16, wsl + q * 1024);
        }
        // one full-wavefront load gathers the scale rows of all its n-blocks: lane L takes row L%16 of
        // n-block L/16 (lanes past NBW*16 repeat the last n-block); rows land at (q*16 + j)*16
        dma16(sbase + (size_t)kb * SB_BYTES, wsl + NBW * 1024);
    };

    f32x4 acc[MT][NBW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q) acc[mt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 m136 = minus136();
    const uint32_t kMask = opaque_vgpr(0x000F000Fu), kBias = opaque_vgpr(0x43004300u);

    // prologue: stages st_begin .. st_begin+D-2 in flight
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (st_begin + d < st_end) issue(st_begin + d);

    for (int st = st_begin; st < st_end; ++st) {
        // wait for this wavefront's loads of stage st: the loads of later stages may stay in flight
        wait_stage<D, OPS>(min(D - 2, st_end - 1 - st));
        stage_barrier();  // every wavefront's pieces of the tile have landed; slot of stage st-1 is free
        if (st + D - 1 < st_end) issue(st + D - 1);

        const uint8_t* sl = slot_of(st);
        const uint8_t* wsl = sl + Lay::X_BYTES + w * Lay::W_BYTES;
        u32x4 cw[NBW], sc[NBW];
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            cw[q] = *reinterpret_cast<const u32x4*>(wsl + q * 1024 + L * 16);
            sc[q] = *reinterpret_cast<const u32x4*>(wsl + NBW * 1024 + (q * 16 + j) * 16);
        }
        const int g0 = (st & 1) * 4;
        // a ragged last stage computes its padding groups too: their codes are 8 and scales 0 in the packed
        // image and their activations are zero, so they add exactly zero
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x8 xf[MT];
            f32x4 xc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + j;
                xf[mt] = *reinterpret_cast<const bf16x8*>(sl + row * (KT * 2) + (((4 * g + c) ^ j) * 16));
                xc[mt] = mfma16(xf[mt], m136, zero);
            }
#pragma unroll
            for (int q = 0; q < NBW; ++q) {
                const bf16x8 wf = biased_codes_vop3(cw[q][g], kMask, kBias);
                const float s = group_scale(sc[q], g0 + g);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 d = mfma16(xf[mt], wf, xc[mt]);
                    acc[mt][q] += s * d;
                }
            }
        }
    }

    decode_epilogue<MT, NBW, OM>(p, acc, ssid, &s_last, b, blockIdx.y, gridDim.y, gridDim.z, blockIdx.z, wave_global,
                                 w, c, j);
}


// LDS budget of the ring per workgroup
constexpr int kRingLdsBytes = 32 * 1024;
// ring depth per tile shape: as many stages in flight as the LDS budget holds
template <int MT, int NBW>
constexpr int ring_depth() {
    constexpr int d = kRingLdsBytes / DecodeLds<MT, NBW>::SLOT;
    return d > 6 ? 6 : (d < 2 ? 2 : d);
}

template <int MT, int NBW, int OM>
hipError_t launch_t(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    constexpr int D = ring_depth<MT, NBW>();
    constexpr size_t shmem = (size_t)D * DecodeLds<MT, NBW>::SLOT;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_decode_kernel<MT, NBW, D, OM>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (attr != hipSuccess) return attr;
    DecodeParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                   a.out, a.partials, a.counters};
    const dim3 grid(a.max_blocks, decode_n_tiles(a.sh, pl), pl.k_split);
    hipLaunchKernelGGL((gemm_decode_kernel<MT, NBW, D, OM>), grid, dim3(kDecodeThreads), shmem, s, p);
    return hipGetLastError();
}

template <int MT, int OM>
hipError_t dispatch_nbw(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    switch (pl.n_blocks) {
        case 1:
            if constexpr (OM == kOutAct) return hipErrorInvalidValue;  // gate and up need a slot each
            else return launch_t<MT, 1, OM>(a, pl, s);
        case 2: return launch_t<MT, 2, OM>(a, pl, s);
        case 4: return launch_t<MT, 4, OM>(a, pl, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OM>
hipError_t dispatch_mt(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    switch (pl.block_m / 16) {
        case 1: return dispatch_nbw<1, OM>(a, pl, s);
        case 2: return dispatch_nbw<2, OM>(a, pl, s);
        case 3: return dispatch_nbw<3, OM>(a, pl, s);
        case 4: return dispatch_nbw<4, OM>(a, pl, s);
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
    if (decode_reg_supported(a, p)) return launch_gemm_decode_reg(a, p, s);
    if (a.self_route_ids) return hipErrorInvalidValue;      // in-kernel routing is on the register kernel only
    if (a.sh.fmt != kFmtInt4) return hipErrorInvalidValue;  // the LDS-staged kernel reads INT4 images only
    switch (a.out_mode) {
        case kOutBf16: return dispatch_mt<kOutBf16>(a, p, s);
        case kOutF32: return dispatch_mt<kOutF32>(a, p, s);
        case kOutAct: return dispatch_mt<kOutAct>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
