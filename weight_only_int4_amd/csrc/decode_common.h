// Pieces shared by the two decode GEMM kernels (LDS-staged and register-streaming): launch geometry, kernel
// parameters, the n-block of each wavefront slot, and the epilogue with the split-K fix-up.
#pragma once

#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace decode {

constexpr int KT = 128;              // k per stage (4 scale groups, half a superblock)
constexpr int kDecodeThreads = 256;  // four wavefronts, each owning its own columns
constexpr int kWaves = kDecodeThreads / 64;

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
    const int32_t* ntp = nullptr;  // num_tokens_padded (device) or NULL: bounds the valid route blocks
    int route_blocks = 0;          // route blocks of the grid (grid.x may be rounded up)
    // in-kernel routing (gate_up of the fused decode step): top-k ids [R] in, the routing tensors out
    const int32_t* topk = nullptr;
    int32_t* sorted_out = nullptr;
    int32_t* eids_out = nullptr;
    int32_t* ntp_out = nullptr;
};

// n-block of weight slot q of wavefront w (see kOutAct for the split of slots between gate and up rows);
// `o` receives the output n-block index it feeds and `valid` whether that block exists
template <int NBW, int OM>
__device__ __forceinline__ int slot_nblock(const Shape& sh, int wave_global, int q, int* o) {
    if (OM == kOutAct) {
        constexpr int HB = NBW / 2;
        const int half = sh.NB / 2;
        *o = wave_global * HB + (q % HB);
        const int nb = (q < HB ? 0 : half) + *o;
        return *o < half ? nb : sh.NB - 1;  // clamp: result discarded when out of range
    }
    *o = wave_global * NBW + q;
    return *o < sh.NB ? *o : sh.NB - 1;
}

// A BF16 output element; COH: device-coherent (visible to workgroups on other XCDs once the store completes).
template <bool COH>
__device__ __forceinline__ void store_bf16(uint16_t* dst, uint16_t v) {
    if constexpr (COH) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *dst = v;
}

// Epilogue shared by the decode kernels.  Lane (c, j) of wavefront w holds rows 4c + r of each 16-row tile and
// column j of each of its NBW n-blocks.  With one K slice (KS == 1) the results go straight to the output; with KS
// slices every workgroup publishes its fp32 partial tile with device-coherent stores and bumps the tile's
// counter, and the last to arrive adds the KS partials in slice order, writes the output and resets the counter.
// Returns whether this workgroup wrote the output tile.  COH: BF16 and activation outputs are stored
// device-coherently (read by other workgroups of the same launch).
template <int MT, int NBW, int OM, bool COH = false>
__device__ __forceinline__ bool decode_epilogue(const DecodeParams& p, const f32x4 (&acc)[MT][NBW], const int* ssid,
                                                int* s_last, int b, int nt, int n_tiles, int KS, int ks,
                                                int wave_global, int w, int c, int j) {
    constexpr int BM = 16 * MT;
    constexpr int COLS = NBW * 16 * kWaves;  // weight columns of the workgroup
    const Shape& sh = p.sh;
    if (KS == 1) {
        // lane holds rows 4c + r of each 16-row tile, column j of each of its n-blocks
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
                        store_bf16<COH>(static_cast<uint16_t*>(p.out) + (size_t)sid * NO + n,
                                        f32_to_bf16_bits(silu_mul(acc[mt][q][r], acc[mt][q + NBW / 2][r])));
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < NBW; ++q) {
                        const int n = (wave_global * NBW + q) * 16 + j;
                        if (n >= sh.N) continue;
                        if (OM == kOutF32)
                            static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = acc[mt][q][r];
                        else
                            store_bf16<COH>(static_cast<uint16_t*>(p.out) + (size_t)sid * sh.N + n,
                                            f32_to_bf16_bits(acc[mt][q][r]));
                    }
                }
            }
        return true;
    }

    // split K: publish the partial tile, the last workgroup of the tile reduces in ks order
    const size_t tile = (size_t)b * n_tiles + nt;
    float* mine = p.partials + (tile * KS + ks) * (size_t)(BM * COLS);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(&mine[(mt * 16 + 4 * c + r) * COLS + (w * NBW + q) * 16 + j], acc[mt][q][r],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the stores above are device-coherent: every wavefront waits until its own have completed, then the
    // barrier orders all of them before the arrival below
    wait_own_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = prev == (unsigned)(KS - 1);
    }
    __syncthreads();
    if (!*s_last) return false;
    const float* all = p.partials + tile * KS * (size_t)(BM * COLS);
    auto reduce = [&](int idx) {
        float v = 0.f;
        for (int z = 0; z < KS; ++z)
            v += __hip_atomic_load(&all[(size_t)z * BM * COLS + idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return v;
    };
    if (OM == kOutAct) {
        // output column oc of the tile: wavefront oc / (16*HB), its slot (oc / 16) % HB, lane column oc % 16
        constexpr int HB = NBW / 2, OCOLS = NBW * 16 * kWaves / 2;
        const int NO = sh.N / 2;
        for (int idx = threadIdx.x; idx < BM * OCOLS; idx += kDecodeThreads) {
            const int m = idx / OCOLS, oc = idx % OCOLS;
            const int sid = ssid[m];
            const int ww = oc / (16 * HB), q = (oc / 16) % HB, jj = oc % 16;
            const int n = ((nt * kWaves + ww) * HB + q) * 16 + jj;
            if (sid < 0 || n >= NO) continue;
            const int gcol = (ww * NBW + q) * 16 + jj;
            const float g = reduce(m * COLS + gcol), u = reduce(m * COLS + gcol + HB * 16);
            store_bf16<COH>(static_cast<uint16_t*>(p.out) + (size_t)sid * NO + n, f32_to_bf16_bits(silu_mul(g, u)));
        }
    } else {
        const int n_base = nt * COLS;
        for (int idx = threadIdx.x; idx < BM * COLS; idx += kDecodeThreads) {
            const int m = idx / COLS, col = idx % COLS;
            const int sid = ssid[m];
            const int n = n_base + col;
            if (sid < 0 || n >= sh.N) continue;
            const float v = reduce(idx);
            if (OM == kOutF32)
                static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = v;
            else
                store_bf16<COH>(static_cast<uint16_t*>(p.out) + (size_t)sid * sh.N + n, f32_to_bf16_bits(v));
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

}  // namespace decode
}  // namespace w4a16
