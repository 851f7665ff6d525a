// Register-level helpers shared by the decode and prefill GEMM kernels.
//
// Both kernels use v_mfma_f32_16x16x32_bf16 with the activation rows as the
// A operand (16 rows x 32 k) and the weights as the B operand (32 k x 16
// output columns).  Lane L holds A row L%16 and B column L%16, each with the
// eight k of slot L/16; the 16x16 fp32 result lands as rows 4*(L/16)+r,
// r = 0..3, of column L%16.  Which eight k a slot holds only has to agree
// between A and B, and the packed layout fixes it as k = 8*slot + u.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A 32-bit constant held in a VGPR that the compiler cannot see through.  gfx9
// VOP3 encodings take no literal constants, so (x & mask) | bias with literal
// mask and bias compiles to an AND and an OR with a literal each; with both
// constants in opaque VGPRs it becomes one v_and_or_b32.  The value is made
// once, outside the loops; the inline assembly is a plain move, and every
// instruction that reads its result is ordinary compiled code (so the
// compiler's hazard checks for the MFMA operands built from it still apply).
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
    uint32_t r;
    __asm__ volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Eight codes of one packed word as BF16 values 128 + q (exact), in 7 VALU
// operations when mask and bias are opaque VGPR values (opaque_vgpr of
// 0x000F000F and 0x43004300): code u = 2p sits in bits [4p, 4p+4) and
// u = 2p+1 in [16+4p, 20+4p), so a shift and one AND-OR build two operands.
__device__ __forceinline__ bf16x8 biased_codes_vop3(uint32_t w, uint32_t mask, uint32_t bias) {
    u32x4 v;
    v.x = (w & mask) | bias;
    v.y = ((w >> 4) & mask) | bias;
    v.z = ((w >> 8) & mask) | bias;
    v.w = ((w >> 12) & mask) | bias;
    return __builtin_bit_cast(bf16x8, v);
}

// Eight codes of one packed word as BF16 values 128 + q (exact).  Code u = 2p
// sits in bits [4p, 4p+4) and u = 2p+1 in [16+4p, 20+4p), so one shift, mask
// and OR with the BF16 pattern of 128 (0x4300) builds two operands.
__device__ __forceinline__ bf16x8 biased_codes(uint32_t w) {
    u32x4 v;
    v.x = (w & 0x000F000Fu) | 0x43004300u;
    v.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    v.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    v.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, v);
}

// B operand with every element equal to -136 (BF16 0xC308): multiplying the
// activation fragment by it gives -136 * (sum of the 32 activations of the
// group) in every column, the correction that turns sum x*(128+q) into
// sum x*(q-8).
__device__ __forceinline__ bf16x8 minus136() {
    u32x4 v = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
    return __builtin_bit_cast(bf16x8, v);
}

// BF16 scale of group g (0..7) from the 16-byte scale row of a superblock.
__device__ __forceinline__ float group_scale(u32x4 sc, int g) {
    const uint32_t word = sc[g >> 1];
    return __uint_as_float((g & 1) ? (word & 0xFFFF0000u) : (word << 16));
}

// Two floats to a packed pair of BF16 values, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Eight fully dequantised weights bf16((q - 8) * s) of one packed word, with the
// code-to-float conversion folded into the multiply-add, in 17 VALU operations: one shift and four
// AND-ORs place each code in a binary16 bit pattern whose value is affine in
// the code (0x6400 | q is 1024 + q for a code in bits 0..3 of a half,
// 0x5400 | (q << 4) is 64 + q for a code in bits 4..7), one mixed-precision
// fused multiply-add per weight reads that half as binary32 and forms
// (1024 + q) * s - 1032 s or (64 + q) * s - 72 s, which is (q - 8) * s exactly,
// and each pair is rounded once to BF16 (round to nearest even).  The masks and
// patterns come in as opaque VGPR values (0x000F000F, 0x00F000F0, 0x64006400,
// 0x54005400) so that each AND-OR is one VOP3 instruction; neg1032s = -1032 s,
// neg72s = -72 s.
struct MixConsts {
    uint32_t mask_lo, mask_hi, magic_lo, magic_hi;
};
__device__ __forceinline__ MixConsts mix_consts() {
    return {opaque_vgpr(0x000F000Fu), opaque_vgpr(0x00F000F0u), opaque_vgpr(0x64006400u), opaque_vgpr(0x54005400u)};
}
__device__ __forceinline__ bf16x8 dequant8_mix(uint32_t w, float s, float neg1032s, float neg72s, const MixConsts& k) {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const uint32_t w8 = w >> 8;
    const f16x2_t p0 = __builtin_bit_cast(f16x2_t, (w & k.mask_lo) | k.magic_lo);   // codes 0, 1
    const f16x2_t p1 = __builtin_bit_cast(f16x2_t, (w & k.mask_hi) | k.magic_hi);   // codes 2, 3
    const f16x2_t p2 = __builtin_bit_cast(f16x2_t, (w8 & k.mask_lo) | k.magic_lo);  // codes 4, 5
    const f16x2_t p3 = __builtin_bit_cast(f16x2_t, (w8 & k.mask_hi) | k.magic_hi);  // codes 6, 7
    u32x4 v;
    v.x = pack_bf16x2(__builtin_fmaf((float)p0.x, s, neg1032s), __builtin_fmaf((float)p0.y, s, neg1032s));
    v.y = pack_bf16x2(__builtin_fmaf((float)p1.x, s, neg72s), __builtin_fmaf((float)p1.y, s, neg72s));
    v.z = pack_bf16x2(__builtin_fmaf((float)p2.x, s, neg1032s), __builtin_fmaf((float)p2.y, s, neg1032s));
    v.w = pack_bf16x2(__builtin_fmaf((float)p3.x, s, neg72s), __builtin_fmaf((float)p3.y, s, neg72s));
    return __builtin_bit_cast(bf16x8, v);
}

// MXFP4: eight E2M1 codes of one 32-bit word (code u in bits [4u, 4u+4)) to the BF16 fragment
// e2m1(code) * 2^(e - 127), where e is the exponent field of `scale` (an E8M0 byte shifted into a binary32
// exponent).  The hardware conversion takes one byte -- two neighbouring k -- per instruction and applies the
// scale's power of two; E2M1 times a power of two has at most 2 significant bits, so the result is exact.
__device__ __forceinline__ bf16x8 mxfp4_dequant8(uint32_t w, float scale) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4 v;
    v.x = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    v.y = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    v.z = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    v.w = __builtin_bit_cast(uint32_t, (bf16x2_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return __builtin_bit_cast(bf16x8, v);
}

// The E8M0 scale of group d (0..3) from four scale bytes as a binary32 power of two.
__device__ __forceinline__ float e8m0_scale(uint32_t four_bytes, int d) {
    return __uint_as_float(((four_bytes >> (8 * d)) & 0xFFu) << 23);
}

// Buffer resources (raw, unformatted, unswizzled) on gfx9-family chips: word 3 of the descriptor, the cache
// policy bits of a non-temporal and of a device-coherent load, and an offset no resource reaches (a load from it returns zeros; a direct
// load to LDS from it writes zeros).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNonTemporal = 2;
constexpr int kBufferDeviceCoherent = 16;  // the sc1 bit: the load is coherent at device scope
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_resource(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// s_waitcnt vmcnt(0), the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in 6:4,
// lgkmcnt in 11:8).  On gfx9 the vector memory counter also counts stores, which it releases once the store has
// been acknowledged at the coherence level its cache policy names, so after this wait the wavefront's
// device-coherent stores are visible to every workgroup of the device.  A workgroup-scope release fence does not
// wait for them (the workgroup's wavefronts share the CU's path to memory).
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// silu(g) * u in binary32 from unrounded gate and up accumulators, with the hardware's exponential and reciprocal
// (a few binary32 ulps, far below the BF16 rounding of h that follows; the full-precision expf and division cost
// about 25 VALU instructions per output, which the epilogue of a VALU-bound GEMM pays for)
__device__ __forceinline__ float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

}  // namespace w4a16
