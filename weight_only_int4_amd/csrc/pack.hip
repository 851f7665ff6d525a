// Offline weight re-layout and the verification dequantiser (INT4 and MXFP4 images).
//
// The pack turns codes [E,N,K] (one code per byte) and BF16 scales [E,N,K/32]
// into the superblock image described in w4a16_internal.h; it runs once per
// weight set, before the forward path (Chord page, "Grouped SM90 kernels":
// the packer prepares weights once and the forward path sees only the
// prepared bytes).  The dequantiser reads that image back and writes
// w = (q - 8) * s (Chord page, "H200 and Blackwell indexed decode": subtract
// the zero point, then scale) so tests can compare it with the definition bit
// for bit.
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
    // gfx950 converts with round-to-nearest-even (v_cvt_pk_bf16_f32)
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// One workgroup of 256 threads per superblock: threads 0..127 write the two
// 1 KiB code halves (16 bytes each), threads 128..143 the 16-byte scale rows.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales, Shape sh,
                                                   uint8_t* __restrict__ packed) {
    const long sb = blockIdx.x;  // ((e*NB + nb)*KB + kb)
    const int kb = (int)(sb % sh.KB);
    const int nb = (int)((sb / sh.KB) % sh.NB);
    const int e = (int)(sb / ((long)sh.KB * sh.NB));
    uint8_t* dst = packed + sb * SB_BYTES;
    const int t = threadIdx.x;
    if (t < 128) {
        const int h = t >> 6, L = t & 63, c = L >> 4, j = L & 15;
        const int n = nb * NB_ROWS + j;
        uint32_t words[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int gg = kb * SB_GROUPS + 4 * h + d;
            uint32_t w = 0x88888888u;  // code 8 everywhere: weight 0
            if (n < sh.N && gg < sh.G) {
                const uint8_t* src = codes + ((size_t)e * sh.N + n) * sh.K + 32 * gg + 8 * c;
                const uint64_t v = *reinterpret_cast<const uint64_t*>(src);
                w = 0;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t lo = (uint32_t)(v >> (16 * p)) & 0xFu;       // code u = 2p
                    const uint32_t hi = (uint32_t)(v >> (16 * p + 8)) & 0xFu;   // code u = 2p + 1
                    w |= (lo << (4 * p)) | (hi << (16 + 4 * p));
                }
            }
            words[d] = w;
        }
        *reinterpret_cast<uint4*>(dst + h * 1024 + L * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    } else if (t < 128 + NB_ROWS) {
        const int j = t - 128;
        const int n = nb * NB_ROWS + j;
        uint32_t words[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t pair = 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int gg = kb * SB_GROUPS + 2 * q + half;
                uint32_t sbits = 0;
                if (n < sh.N && gg < sh.G) sbits = scales[((size_t)e * sh.N + n) * sh.G + gg];
                pair |= sbits << (16 * half);
            }
            words[q] = pair;
        }
        *reinterpret_cast<uint4*>(dst + SB_CODE_BYTES + j * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    }
}

// MXFP4 image: the same superblock geometry, codes in natural nibble order, one E8M0 byte per group.
__global__ __launch_bounds__(256) void pack_mxfp4_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, Shape sh,
                                                         uint8_t* __restrict__ packed) {
    const long sb = blockIdx.x;  // ((e*NB + nb)*KB + kb)
    const int kb = (int)(sb % sh.KB);
    const int nb = (int)((sb / sh.KB) % sh.NB);
    const int e = (int)(sb / ((long)sh.KB * sh.NB));
    uint8_t* dst = packed + sb * SB_BYTES_MXFP4;
    const int t = threadIdx.x;
    if (t < 128) {
        const int h = t >> 6, L = t & 63, c = L >> 4, j = L & 15;
        const int n = nb * NB_ROWS + j;
        uint32_t words[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int gg = kb * SB_GROUPS + 4 * h + d;
            uint32_t w = 0;  // code 0 everywhere: weight +0
            if (n < sh.N && gg < sh.G) {
                const uint8_t* src = codes + ((size_t)e * sh.N + n) * sh.K + 32 * gg + 8 * c;
                const uint64_t v = *reinterpret_cast<const uint64_t*>(src);
#pragma unroll
                for (int u = 0; u < 8; ++u) w |= ((uint32_t)(v >> (8 * u)) & 0xFu) << (4 * u);
            }
            words[d] = w;
        }
        *reinterpret_cast<uint4*>(dst + h * 1024 + L * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    } else if (t < 128 + NB_ROWS) {
        const int j = t - 128;
        const int n = nb * NB_ROWS + j;
        uint32_t words[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint32_t four = 0;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int gg = kb * SB_GROUPS + 4 * q + d;
                uint32_t e8 = 127;  // padding: scale 1
                if (n < sh.N && gg < sh.G) e8 = scales[((size_t)e * sh.N + n) * sh.G + gg];
                four |= e8 << (8 * d);
            }
            words[q] = four;
        }
        *reinterpret_cast<uint2*>(dst + SB_CODE_BYTES + j * 8) = make_uint2(words[0], words[1]);
    }
}

// One thread per (row n, group g) of one expert: 32 weights.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ packed, Shape sh, int expert,
                                                      float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)sh.N * sh.G) return;
    const int n = (int)(idx / sh.G), g = (int)(idx % sh.G);
    const int nb = n / NB_ROWS, j = n % NB_ROWS, kb = g / SB_GROUPS, gl = g % SB_GROUPS;
    const int h = gl >> 2, d = gl & 3;
    const uint8_t* sbp = packed + (((size_t)expert * sh.NB + nb) * sh.KB + kb) * sb_bytes(sh.fmt);
    if (sh.fmt == kFmtMxfp4) {
        // E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (bit 3 the sign) times 2^(e - 127)
        const int e8 = sbp[SB_CODE_BYTES + j * 8 + gl];
        const float s = e8 == 0xFF ? __builtin_nanf("") : ldexpf(1.0f, e8 - 127);
        const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(sbp + h * 1024 + (c * 16 + j) * 16 + d * 4);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int code = (int)((w >> (4 * u)) & 0xFu);
                const float v = (code & 8) ? -mag[code & 7] : mag[code & 7];
                const float wq = v * s;  // exact: at most 2 significant bits
                const size_t o = (size_t)n * sh.K + 32 * g + 8 * c + u;
                if (out_f32) out_f32[o] = wq;
                if (out_bf16) out_bf16[o] = float_to_bf16_rne(wq);
            }
        }
        return;
    }
    const uint32_t sbits = *reinterpret_cast<const uint16_t*>(sbp + SB_CODE_BYTES + j * 16 + gl * 2);
    const float s = bf16_bits_to_float(sbits);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(sbp + h * 1024 + (c * 16 + j) * 16 + d * 4);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int shift = (u & 1) ? 16 + 4 * (u >> 1) : 4 * (u >> 1);
            const int q = (int)((w >> shift) & 0xFu);
            const float wq = (float)(q - 8) * s;  // exact: at most 12 significant bits
            const size_t o = (size_t)n * sh.K + 32 * g + 8 * c + u;
            if (out_f32) out_f32[o] = wq;
            if (out_bf16) out_bf16[o] = float_to_bf16_rne(wq);
        }
    }
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, const Shape& sh, void* packed, hipStream_t s) {
    const long blocks = (long)sh.E * sh.NB * sh.KB;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, sh,
                       static_cast<uint8_t*>(packed));
    return hipGetLastError();
}

hipError_t launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, const Shape& sh, void* packed,
                             hipStream_t s) {
    const long blocks = (long)sh.E * sh.NB * sh.KB;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, sh,
                       static_cast<uint8_t*>(packed));
    return hipGetLastError();
}

hipError_t launch_dequant(const void* packed, const Shape& sh, int expert, float* out_f32, uint16_t* out_bf16,
                          hipStream_t s) {
    const long work = (long)sh.N * sh.G;
    if (work == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(packed), sh, expert, out_f32, out_bf16);
    return hipGetLastError();
}

}  // namespace w4a16
