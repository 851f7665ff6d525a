/*
 * Plain CPU oracle for the W4A16 mixture-of-experts grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: it exists so tests, the smoke check and the CPU baseline
 * of the benchmark can compare the HIP library against an independent,
 * obviously correct implementation.  It shares no source with the library.
 *
 * What is computed, and where it is defined:
 *  - Weights are unsigned 4-bit codes q in [0,15] with one BF16 scale per
 *    32 consecutive k of an (expert, output row); the dequantised weight is
 *    w = (q - 8) * s ("vLLM x Novita AI: Chord, Faster INT4 MoE for Kimi
 *    K2.x", sections "Grouped SM90 kernels" -- codes [G,N,K], scales
 *    [G,N,K/32] -- and "H200 and Blackwell indexed decode" -- dequantisation
 *    subtracts the zero point and then applies the scale).  The zero point 8
 *    is the plain reading of "unsigned INT4" with a symmetric range.
 *  - Each routed row is multiplied by its expert's weight matrix transposed:
 *    out[rows of e] = x[rows of e] @ W[e]^T ("LegumMagister/nf4-grouped-gemm",
 *    section "Usage").
 *  - Routing is the indexed form sorted_ids / expert_ids / num_tokens_padded
 *    (Chord page, "Two kernel families" and Figure 3: activations stay
 *    unpadded and padding lives in the index tensors as sentinels), plus
 *    per-expert offsets (nf4 page, "Usage": cumulative rows per expert).
 *  - A second weight format, MXFP4: 4-bit E2M1 codes with one E8M0 scale per
 *    32 consecutive k, w = e2m1(c) * 2^(e - 127).  The b12x page
 *    ("local-inference-lab/b12x pull 479", section "Summary") runs MXFP4
 *    routed experts with E8M0 scales; the humans& page (section "BF16
 *    preserves each local product") dequantises E2M1 values by their block
 *    scale into BF16, where such products are exact.  The value set of E2M1
 *    (sign, two exponent bits with bias 1, one mantissa bit) and of E8M0 (a
 *    bare power of two, 0xFF not a number) are those of the OCP Microscaling
 *    formats the pages name.
 *  - The fused expert MLP (gate_up, SiLU*mul, down, weighted top-k merge) is
 *    the chain the humans& page describes for its persistent kernel
 *    ("humans& Beats FlashInfer's Best MoE Kernel by 25% on Blackwell GPUs",
 *    section "Dedicated warps keep the pipeline busy").
 *
 * Every function is a direct transcription of its definition: loops in the
 * natural index order, fp32 accumulation in ascending k (or fp64 when asked),
 * single round-to-nearest-even conversions to BF16.  Threads split only the
 * independent output rows; each row's arithmetic is sequential.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* BF16 <-> float, from the IEEE-754 binary32 bit layout.              */
/* BF16 is the upper 16 bits of a binary32; conversion from binary32   */
/* rounds the dropped 16 bits to nearest, ties to even.                */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

uint16_t orc_bf16_rne(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
        /* NaN: keep sign, force a quiet NaN so truncation cannot yield inf */
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    /* round half to even on the 16 dropped bits */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;  /* a carry into the exponent is the correct result (incl. overflow to inf) */
}

/* Round a double to BF16 in one step (used where a value is formed in double). */
uint16_t orc_bf16_rne_f64(double d) {
    if (isnan(d)) return (uint16_t)0x7FC0u;
    if (d == 0.0) return signbit(d) ? (uint16_t)0x8000u : (uint16_t)0u;
    /* Exact conversion to binary32 first would double-round; do it directly.
     * BF16 has 8 significant bits; normal exponent range as binary32. */
    int sign = d < 0;
    double a = fabs(d);
    if (isinf(a)) return (uint16_t)(sign ? 0xFF80u : 0x7F80u);
    int e;
    frexp(a, &e);            /* a = m * 2^e, m in [0.5,1) */
    int exp_unbiased = e - 1; /* a in [2^(e-1), 2^e) */
    if (exp_unbiased < -126) exp_unbiased = -126; /* subnormal: fixed quantum */
    double quantum = ldexp(1.0, exp_unbiased - 7);
    double units = a / quantum;          /* exact: power-of-two scaling */
    double fl = floor(units);
    double frac = units - fl;            /* exact */
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    double v = r * quantum;              /* exact, may reach 2^e */
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign ? 0xFF80u : 0x7F80u);
    float fv = (float)v;                 /* exact: v has <= 8 significant bits in range */
    uint16_t h = (uint16_t)(f32_bits(fv) >> 16);
    return (uint16_t)(h | (sign ? 0x8000u : 0u));
}

/* ------------------------------------------------------------------ */
/* Dequantisation: w = (q - 8) * s, q = low nibble of the code byte,    */
/* s = scale of group k/32.  The product has at most 4+8 significant    */
/* bits, so the binary32 result is exact; the BF16 image is one RNE.    */
/* ------------------------------------------------------------------ */

float orc_dequant_one(uint8_t code, uint16_t scale_bf16) {
    int q = (int)(code & 0x0F);
    return (float)(q - 8) * orc_bf16_to_f32(scale_bf16);
}

/* MXFP4: E2M1 code c (low nibble): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0 is
 * subnormal (0 or 0.5).  Positive values in code order: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  E8M0 scale byte e: 2^(e-127),
 * 0xFF not a number.  The product has at most 2 significant bits, so binary32 holds it exactly down to 2^-149. */
float orc_e2m1(uint8_t code) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mag[code & 7];
    return (code & 8) ? -v : v;
}

float orc_e8m0(uint8_t e) { return e == 0xFF ? NAN : ldexpf(1.0f, (int)e - 127); }

float orc_dequant_mxfp4_one(uint8_t code, uint8_t scale_e8m0) {
    return orc_e2m1((uint8_t)(code & 0x0F)) * orc_e8m0(scale_e8m0);
}

/* One expert, MXFP4: codes [N,K], E8M0 scales [N,K/32] -> out_f32 / out_bf16 [N,K] (either may be NULL). */
void orc_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int N, int K, float* out_f32,
                       uint16_t* out_bf16) {
    int G = K / 32;
    for (int n = 0; n < N; ++n) {
        const uint8_t* srow = scales + (size_t)n * G;
        for (int k = 0; k < K; ++k) {
            float w = orc_dequant_mxfp4_one(codes[(size_t)n * K + k], srow[k / 32]);
            if (out_f32) out_f32[(size_t)n * K + k] = w;
            if (out_bf16) out_bf16[(size_t)n * K + k] = orc_bf16_rne(w);
        }
    }
}

/* A weight of either format: fmt 0 = INT4 codes with BF16 scales (uint16 array), 1 = MXFP4 with E8M0 scales
 * (uint8 array); g indexes the scale array. */
static float orc_weight(int fmt, const uint8_t* codes, const void* scales, size_t idx, size_t g) {
    if (fmt == 1) return orc_dequant_mxfp4_one(codes[idx], ((const uint8_t*)scales)[g]);
    return orc_dequant_one(codes[idx], ((const uint16_t*)scales)[g]);
}

/* One expert: codes [N,K], scales [N,K/32] -> out_f32 [N,K], out_bf16 [N,K] (either may be NULL). */
void orc_dequant(const uint8_t* codes, const uint16_t* scales, int N, int K,
                 float* out_f32, uint16_t* out_bf16) {
    int G = K / 32;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k) {
            float w = orc_dequant_one(codes[(size_t)n * K + k], scales[(size_t)n * G + k / 32]);
            if (out_f32) out_f32[(size_t)n * K + k] = w;
            if (out_bf16) out_bf16[(size_t)n * K + k] = orc_bf16_rne(w);
        }
}

/* ------------------------------------------------------------------ */
/* Routing (indexed form).                                             */
/* Route i = t*k + j is valid when 0 <= topk_ids[i] < E.               */
/* Expert e's segment of sorted_ids starts at the sum of the padded    */
/* sizes ceil(c/BM)*BM of all lower experts, lists e's routes in       */
/* ascending i, then sentinels equal to R until the padded size.       */
/* Slots from num_tokens_padded to max_padded hold R as well.          */
/* expert_ids[b] is the owner of block b, or -1 past the padded end.   */
/* ------------------------------------------------------------------ */

void orc_route_bounds(int T, int k, int E, int BM, int* max_padded, int* max_blocks) {
    long R = (long)T * k;
    long act = R < E ? R : E;
    long raw = R + act * (BM - 1);
    long blocks = (raw + BM - 1) / BM;
    *max_padded = (int)(blocks * BM);
    *max_blocks = (int)blocks;
}

int orc_route_prep(const int32_t* topk_ids, int T, int k, int E, int BM,
                   int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_tokens_padded,
                   int32_t* expert_offsets, int32_t* counts) {
    int R = T * k, maxP, maxB;
    orc_route_bounds(T, k, E, BM, &maxP, &maxB);
    int32_t* cnt = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t* pad_off = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    int32_t* fill = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    if (!cnt || !pad_off || !fill) { free(cnt); free(pad_off); free(fill); return -1; }
    for (int i = 0; i < R; ++i) {
        int e = topk_ids[i];
        if (e >= 0 && e < E) cnt[e] += 1;
    }
    expert_offsets[0] = 0;
    pad_off[0] = 0;
    for (int e = 0; e < E; ++e) {
        counts[e] = cnt[e];
        expert_offsets[e + 1] = expert_offsets[e] + cnt[e];
        int padded = (cnt[e] + BM - 1) / BM * BM;
        pad_off[e + 1] = pad_off[e] + padded;
    }
    *num_tokens_padded = pad_off[E];
    for (int p = 0; p < maxP; ++p) sorted_ids[p] = R;
    for (int i = 0; i < R; ++i) {
        int e = topk_ids[i];
        if (e >= 0 && e < E) sorted_ids[pad_off[e] + fill[e]++] = i;
    }
    for (int b = 0; b < maxB; ++b) expert_ids[b] = -1;
    for (int e = 0; e < E; ++e)
        for (int p = pad_off[e]; p < pad_off[e + 1]; p += BM) expert_ids[p / BM] = e;
    free(cnt); free(pad_off); free(fill);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Grouped GEMM by definition, one routed row at a time.               */
/* For each valid route i with expert e = topk_ids[i]:                 */
/*   acc[n] = sum_{k ascending} A[i / a_row_div][k] * w[e][n][k]       */
/* in binary32 (acc64 = 0) or binary64 (acc64 = 1); out = bf16(acc).   */
/* Rows of invalid routes are not touched.                             */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint16_t* A; int a_row_div;
    const uint8_t* codes; const void* scales; int fmt;
    int E, N, K;
    const int32_t* topk_ids; int R; int acc64;
    double* out_acc; uint16_t* out;
    const int32_t* rows; int nrows;   /* optional list of route indices to compute */
    int tid, nthreads;
} gemm_job;

static void gemm_row(const gemm_job* j, int i) {
    int e = j->topk_ids[i];
    if (e < 0 || e >= j->E) return;
    int N = j->N, K = j->K, G = K / 32;
    const uint16_t* a = j->A + (size_t)(i / j->a_row_div) * K;
    const uint8_t* cw = j->codes + (size_t)e * N * K;
    const size_t sw = (size_t)e * N * G;  /* first scale of expert e */
    for (int n = 0; n < N; ++n) {
        if (j->acc64) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)orc_bf16_to_f32(a[k]) *
                       (double)orc_weight(j->fmt, cw, j->scales, (size_t)n * K + k, sw + (size_t)n * G + k / 32);
            if (j->out_acc) j->out_acc[(size_t)i * N + n] = acc;
            if (j->out) j->out[(size_t)i * N + n] = orc_bf16_rne_f64(acc);
        } else {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                float prod = orc_bf16_to_f32(a[k]) *
                             orc_weight(j->fmt, cw, j->scales, (size_t)n * K + k, sw + (size_t)n * G + k / 32);
                acc = acc + prod;
            }
            if (j->out_acc) j->out_acc[(size_t)i * N + n] = (double)acc;
            if (j->out) j->out[(size_t)i * N + n] = orc_bf16_rne(acc);
        }
    }
}

static void* gemm_worker(void* p) {
    gemm_job* j = (gemm_job*)p;
    int total = j->rows ? j->nrows : j->R;
    for (int r = j->tid; r < total; r += j->nthreads) gemm_row(j, j->rows ? j->rows[r] : r);
    return NULL;
}

static void run_threads(void* (*fn)(void*), void* jobs, size_t job_size, int nthreads) {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, fn, (char*)jobs + job_size * t);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
}

/* rows == NULL: all R routes; otherwise only the listed route indices.  fmt: 0 INT4 / BF16 scales, 1 MXFP4. */
void orc_grouped_gemm_fmt(const uint16_t* A, int a_row_div, const uint8_t* codes, const void* scales, int fmt,
                          int E, int N, int K, const int32_t* topk_ids, int R, int acc64,
                          double* out_acc, uint16_t* out, const int32_t* rows, int nrows, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    gemm_job* jobs = (gemm_job*)malloc(sizeof(gemm_job) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        gemm_job j = {A, a_row_div, codes, scales, fmt, E, N, K, topk_ids, R, acc64,
                      out_acc, out, rows, nrows, t, nthreads};
        jobs[t] = j;
    }
    run_threads(gemm_worker, jobs, sizeof(gemm_job), nthreads);
    free(jobs);
}

void orc_grouped_gemm(const uint16_t* A, int a_row_div, const uint8_t* codes, const uint16_t* scales,
                      int E, int N, int K, const int32_t* topk_ids, int R, int acc64,
                      double* out_acc, uint16_t* out, const int32_t* rows, int nrows, int nthreads) {
    orc_grouped_gemm_fmt(A, a_row_div, codes, scales, 0, E, N, K, topk_ids, R, acc64, out_acc, out, rows, nrows,
                         nthreads);
}

/* ------------------------------------------------------------------ */
/* SiLU(g) * u with g = gu[c], u = gu[I + c] ("w13": gate rows first).  */
/* silu(g) = g / (1 + exp(-g)), formed in binary64, rounded once.       */
/* ------------------------------------------------------------------ */

double orc_silu(double g) { return g / (1.0 + exp(-g)); }

uint16_t orc_silu_mul_one(double g, double u) { return orc_bf16_rne_f64(orc_silu(g) * u); }

/* gu: [rows, 2I] values (binary64 holding the pre-rounding accumulators); h: [rows, I] bf16 */
void orc_silu_mul(const double* gu, int rows, int I, uint16_t* h) {
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < I; ++c)
            h[(size_t)r * I + c] = orc_silu_mul_one(gu[(size_t)r * 2 * I + c], gu[(size_t)r * 2 * I + I + c]);
}

/* ------------------------------------------------------------------ */
/* Weighted top-k combine:                                              */
/*   out[t,:] = bf16( sum_{j valid, ascending} tw[t,j] * y[t*k + j,:] ) */
/* accumulated in binary32; a token with no valid route gets zeros.    */
/* ------------------------------------------------------------------ */

void orc_combine(const double* y, const float* tw, const int32_t* topk_ids, int T, int k, int E, int H,
                 uint16_t* out, double* out_acc) {
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < H; ++n) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int e = topk_ids[(size_t)t * k + j];
                if (e < 0 || e >= E) continue;
                acc = acc + tw[(size_t)t * k + j] * (float)y[((size_t)t * k + j) * H + n];
            }
            out[(size_t)t * H + n] = orc_bf16_rne(acc);
            if (out_acc) out_acc[(size_t)t * H + n] = (double)acc;  /* the value before rounding */
        }
}

/* ------------------------------------------------------------------ */
/* Fused expert MLP: gate_up (binary32 accumulators, unrounded) ->       */
/* h = bf16(silu(g) * u) -> down (binary32, unrounded) -> combine.      */
/* w13: codes [E, 2I, H], scales [E, 2I, H/32]; w2: [E, H, I], [E,H,I/32]. */
/* Optional outputs: out_acc [T, H] (combine accumulators before rounding), */
/* h_out [R, I] bf16, y_out [R, H] (binary64 holders of binary32 values).   */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint16_t* x; const int32_t* topk_ids; int T, k, E, H, I;
    const uint8_t* c13; const void* s13; const uint8_t* c2; const void* s2; int fmt;
    double* gu; uint16_t* h; double* y;
    int tid, nthreads;
} moe_job;

static void* moe_worker(void* p) {
    moe_job* j = (moe_job*)p;
    int R = j->T * j->k, H = j->H, I = j->I;
    int G13 = H / 32, G2 = I / 32;
    for (int i = j->tid; i < R; i += j->nthreads) {
        int e = j->topk_ids[i];
        if (e < 0 || e >= j->E) continue;
        const uint16_t* a = j->x + (size_t)(i / j->k) * H;
        double* gu = j->gu + (size_t)i * 2 * I;
        for (int n = 0; n < 2 * I; ++n) {
            const uint8_t* cw = j->c13 + ((size_t)e * 2 * I + n) * H;
            const size_t sw = ((size_t)e * 2 * I + n) * G13;
            float acc = 0.0f;
            for (int kk = 0; kk < H; ++kk)
                acc = acc + orc_bf16_to_f32(a[kk]) * orc_weight(j->fmt, cw, j->s13, (size_t)kk, sw + kk / 32);
            gu[n] = (double)acc;
        }
        uint16_t* h = j->h + (size_t)i * I;
        for (int c = 0; c < I; ++c) h[c] = orc_silu_mul_one(gu[c], gu[I + c]);
        double* y = j->y + (size_t)i * H;
        for (int n = 0; n < H; ++n) {
            const uint8_t* cw = j->c2 + ((size_t)e * H + n) * I;
            const size_t sw = ((size_t)e * H + n) * G2;
            float acc = 0.0f;
            for (int kk = 0; kk < I; ++kk)
                acc = acc + orc_bf16_to_f32(h[kk]) * orc_weight(j->fmt, cw, j->s2, (size_t)kk, sw + kk / 32);
            y[n] = (double)acc;
        }
    }
    return NULL;
}

int orc_fused_moe_fmt(const uint16_t* x, const int32_t* topk_ids, const float* tw, int T, int k,
                      int E, int H, int I,
                      const uint8_t* c13, const void* s13, const uint8_t* c2, const void* s2, int fmt,
                      uint16_t* out, double* out_acc, uint16_t* h_out, double* y_out, int nthreads) {
    size_t R = (size_t)T * k;
    double* gu = (double*)malloc(sizeof(double) * (R ? R : 1) * 2 * (size_t)I);
    uint16_t* h = h_out ? h_out : (uint16_t*)malloc(sizeof(uint16_t) * (R ? R : 1) * (size_t)I);
    double* y = y_out ? y_out : (double*)malloc(sizeof(double) * (R ? R : 1) * (size_t)H);
    if (!gu || !h || !y) return -1;
    if (nthreads < 1) nthreads = 1;
    moe_job* jobs = (moe_job*)malloc(sizeof(moe_job) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        moe_job j = {x, topk_ids, T, k, E, H, I, c13, s13, c2, s2, fmt, gu, h, y, t, nthreads};
        jobs[t] = j;
    }
    run_threads(moe_worker, jobs, sizeof(moe_job), nthreads);
    free(jobs);
    orc_combine(y, tw, topk_ids, T, k, E, H, out, out_acc);
    free(gu);
    if (!h_out) free(h);
    if (!y_out) free(y);
    return 0;
}

int orc_fused_moe(const uint16_t* x, const int32_t* topk_ids, const float* tw, int T, int k,
                  int E, int H, int I,
                  const uint8_t* c13, const uint16_t* s13, const uint8_t* c2, const uint16_t* s2,
                  uint16_t* out, double* out_acc, uint16_t* h_out, double* y_out, int nthreads) {
    return orc_fused_moe_fmt(x, topk_ids, tw, T, k, E, H, I, c13, s13, c2, s2, 0, out, out_acc, h_out, y_out,
                             nthreads);
}
