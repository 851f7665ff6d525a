// Activation and weighted top-k combine of the expert MLP (humans& page,
// "Dedicated warps keep the pipeline busy": FC1, FC2 and the top-K merge).
#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// h[r,c] = bf16(silu(g) * u) with g = gu[r,c], u = gu[r,I+c]; two columns per thread.
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gu, int rows, int I,
                                                       uint16_t* __restrict__ h) {
    const int pairs = I >> 1;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)rows * pairs) return;
    const int r = (int)(idx / pairs), c = 2 * (int)(idx % pairs);
    const uint32_t g2 = *reinterpret_cast<const uint32_t*>(gu + (size_t)r * 2 * I + c);
    const uint32_t u2 = *reinterpret_cast<const uint32_t*>(gu + (size_t)r * 2 * I + I + c);
    const float g0 = bf16_to_f32(g2 & 0xFFFFu), g1 = bf16_to_f32(g2 >> 16);
    const float u0 = bf16_to_f32(u2 & 0xFFFFu), u1 = bf16_to_f32(u2 >> 16);
    const float h0 = silu_mul(g0, u0);
    const float h1 = silu_mul(g1, u1);
    const uint32_t packed = (uint32_t)f32_to_bf16_bits(h0) | ((uint32_t)f32_to_bf16_bits(h1) << 16);
    *reinterpret_cast<uint32_t*>(h + (size_t)r * I + c) = packed;
}

// Same activation from binary32 gate/up values (the fused MLP keeps the gate_up
// accumulators unrounded): h[r,c] = bf16(silu(gu[r,c]) * gu[r,I+c]).
__global__ __launch_bounds__(256) void silu_mul_f32_kernel(const float* __restrict__ gu, int rows, int I,
                                                           uint16_t* __restrict__ h) {
    const int pairs = I >> 1;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)rows * pairs) return;
    const int r = (int)(idx / pairs), c = 2 * (int)(idx % pairs);
    const float2 g = *reinterpret_cast<const float2*>(gu + (size_t)r * 2 * I + c);
    const float2 u = *reinterpret_cast<const float2*>(gu + (size_t)r * 2 * I + I + c);
    const float h0 = silu_mul(g.x, u.x);
    const float h1 = silu_mul(g.y, u.y);
    const uint32_t packed = (uint32_t)f32_to_bf16_bits(h0) | ((uint32_t)f32_to_bf16_bits(h1) << 16);
    *reinterpret_cast<uint32_t*>(h + (size_t)r * I + c) = packed;
}

// Loads of y rows: binary32 (the unfused down projection's output) or BF16 bits (the fused step's y).
__device__ __forceinline__ void load_y2(const float* p, float* v) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x;
    v[1] = t.y;
}
__device__ __forceinline__ void load_y2(const uint16_t* p, float* v) {
    const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_to_f32(t & 0xFFFFu);
    v[1] = bf16_to_f32(t >> 16);
}

// Eight consecutive values of a y row, fetched into registers (issue) and widened to binary32 (unpack), so that
// the loads of several routes can be in flight before the first is used.
template <typename Y>
struct Y8;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <>
struct Y8<float> {
    f32x4_t a, b;
    // y is read once: non-temporal loads keep it from displacing other lines in the caches
    __device__ __forceinline__ void issue(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + 1);
    }
    __device__ __forceinline__ void unpack(float* v) const {
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    }
};
template <>
struct Y8<uint16_t> {
    u32x4 a;
    // y is read once: non-temporal loads keep it from displacing other lines in the caches
    __device__ __forceinline__ void issue(const uint16_t* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ void unpack(float* v) const {
        const uint32_t w[4] = {a[0], a[1], a[2], a[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
};

// out[t,n] = bf16(sum_{valid j ascending} tw[t,j] * y[t*k+j, n]); two columns per thread.
template <typename Y>
__global__ __launch_bounds__(256) void combine_kernel(const Y* __restrict__ y, const float* __restrict__ tw,
                                                      const int32_t* __restrict__ ids, int T, int k, int E, int H,
                                                      uint16_t* __restrict__ out) {
    const int pairs = H >> 1;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)T * pairs) return;
    const int t = (int)(idx / pairs), n = 2 * (int)(idx % pairs);
    float a0 = 0.f, a1 = 0.f;
    for (int jj = 0; jj < k; ++jj) {
        const int e = ids[(size_t)t * k + jj];
        if (e < 0 || e >= E) continue;
        const float wt = tw[(size_t)t * k + jj];
        float v[2];
        load_y2(y + ((size_t)t * k + jj) * H + n, v);
        a0 = __builtin_fmaf(wt, v[0], a0);  // one rounding per route, as in every combine of this library
        a1 = __builtin_fmaf(wt, v[1], a1);
    }
    const uint32_t packed = (uint32_t)f32_to_bf16_bits(a0) | ((uint32_t)f32_to_bf16_bits(a1) << 16);
    *reinterpret_cast<uint32_t*>(out + (size_t)t * H + n) = packed;
}

// The same sum, eight columns per lane: one workgroup per (token, 2048 columns).  The token's ids and weights
// are uniform across the workgroup; the y rows of up to eight routes are in flight together (one or two 16-byte
// loads per route and lane) before any is accumulated, in route order as above.  Needs H % 8 == 0.
constexpr int kCombineCols = 8;
constexpr int kCombineUnroll = 8;
constexpr size_t kCombineSpecBytes = (size_t)4 << 20;  // y up to this size is loaded before the ids arrive

// COLS_FAST: the column group is grid.x, so the workgroups of one token run next to each other and read its
// rows of y together (grid.y then holds the tokens, at most 65535).  SPEC: the y rows of all k routes are
// loaded before the ids say which are valid (row t*k + j exists for every j), so the loads do not wait for the
// ids; invalid rows are loaded but not added.  For small y only: a step whose routes are mostly non-local would
// read many rows it does not need.
template <typename Y, bool COLS_FAST, bool SPEC>
__global__ __launch_bounds__(256) void combine8_kernel(const Y* __restrict__ y, const float* __restrict__ tw,
                                                       const int32_t* __restrict__ ids, int T, int k, int E, int H,
                                                       uint16_t* __restrict__ out) {
    const int t = COLS_FAST ? blockIdx.y : blockIdx.x;
    const int n = ((COLS_FAST ? blockIdx.x : blockIdx.y) * 256 + threadIdx.x) * kCombineCols;
    if (n >= H) return;
    const int32_t* tid = ids + (size_t)t * k;
    const float* tww = tw + (size_t)t * k;
    float acc[kCombineCols];
#pragma unroll
    for (int c = 0; c < kCombineCols; ++c) acc[c] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kCombineUnroll) {
        Y8<Y> v[kCombineUnroll];
        float wt[kCombineUnroll];
        bool ok[kCombineUnroll];
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const int j = j0 + u;
            if (SPEC && j < k) v[u].issue(y + ((size_t)t * k + j) * H + n);
            const int e = j < k ? tid[j] : -1;
            ok[u] = e >= 0 && e < E;
            wt[u] = ok[u] ? tww[j] : 0.f;
            if (!SPEC && ok[u]) v[u].issue(y + ((size_t)t * k + j) * H + n);
        }
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            if (!ok[u]) continue;
            float vv[kCombineCols];
            v[u].unpack(vv);
#pragma unroll
            for (int c = 0; c < kCombineCols; ++c) acc[c] = __builtin_fmaf(wt[u], vv[c], acc[c]);
        }
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_bits(acc[4]) | ((uint32_t)f32_to_bf16_bits(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_bits(acc[6]) | ((uint32_t)f32_to_bf16_bits(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + n) = o;
}

// Zero-fills n 32-bit words (used where a caller may capture the call in a graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* gu, int rows, int I, uint16_t* h, hipStream_t s) {
    const long work = (long)rows * (I / 2);
    if (work == 0) return hipSuccess;
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, gu, rows, I, h);
    return hipGetLastError();
}

hipError_t launch_silu_mul_f32(const float* gu, int rows, int I, uint16_t* h, hipStream_t s) {
    const long work = (long)rows * (I / 2);
    if (work == 0) return hipSuccess;
    hipLaunchKernelGGL(silu_mul_f32_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, gu, rows, I, h);
    return hipGetLastError();
}

template <typename Y>
hipError_t launch_combine_t(const Y* y, const float* tw, const int32_t* ids, int T, int k, int E, int H,
                            uint16_t* out, hipStream_t s) {
    const long work = (long)T * (H / 2);
    if (work == 0) return hipSuccess;
    if (H % kCombineCols == 0 && ((uintptr_t)y & 15u) == 0 && ((uintptr_t)out & 15u) == 0) {
        const unsigned col_groups = (unsigned)((H / kCombineCols + 255) / 256);
        if (T <= 65535 && (size_t)T * k * H * sizeof(Y) <= kCombineSpecBytes)
            hipLaunchKernelGGL((combine8_kernel<Y, true, true>), dim3(col_groups, (unsigned)T), dim3(256), 0, s, y, tw,
                               ids, T, k, E, H, out);
        else if (T <= 65535)
            hipLaunchKernelGGL((combine8_kernel<Y, true, false>), dim3(col_groups, (unsigned)T), dim3(256), 0, s, y,
                               tw, ids, T, k, E, H, out);
        else
            hipLaunchKernelGGL((combine8_kernel<Y, false, false>), dim3((unsigned)T, col_groups), dim3(256), 0, s, y,
                               tw, ids, T, k, E, H, out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((combine_kernel<Y>), dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, y, tw, ids, T, k, E,
                       H, out);
    return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* tw, const int32_t* ids, int T, int k, int E, int H,
                          uint16_t* out, hipStream_t s) {
    return launch_combine_t(y, tw, ids, T, k, E, H, out, s);
}

hipError_t launch_combine_bf16(const uint16_t* y, const float* tw, const int32_t* ids, int T, int k, int E, int H,
                               uint16_t* out, hipStream_t s) {
    return launch_combine_t(y, tw, ids, T, k, E, H, out, s);
}

}  // namespace w4a16
