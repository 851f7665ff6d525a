/*
 * w4a16.h -- C ABI of libw4a16, a W4A16 mixture-of-experts grouped GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are the pages this library was designed from):
 *  - Expert weights are unsigned 4-bit codes q with one BF16 scale per 32
 *    consecutive k of an (expert, output row); the weight is w = (q - 8) * s,
 *    dequantised inside the kernels ("vLLM x Novita AI: Chord, Faster INT4 MoE
 *    for Kimi K2.x", sections "Grouped SM90 kernels" and "H200 and Blackwell
 *    indexed decode").
 *  - Each routed activation row is multiplied by its expert's weight matrix
 *    transposed: out[rows of e] = A[rows of e] @ W[e]^T
 *    ("LegumMagister/nf4-grouped-gemm", section "Usage").
 *  - Routing uses the indexed tensors sorted_ids / expert_ids /
 *    num_tokens_padded, where activations stay unpadded and padding lives in
 *    the indices as sentinels (Chord page, "Two kernel families" and
 *    Figure 3), plus per-expert offsets (nf4 page, "Usage").
 *  - The fused expert MLP chains gate_up, SiLU*mul, down and the weighted
 *    top-k merge (humans& page, "Dedicated warps keep the pipeline busy").
 *
 * Conventions for every call:
 *  - Returns W4A16_OK (0) or a negative status; the message of the last
 *    failure on the calling thread is w4a16_last_error().
 *  - Device buffers are allocated and owned by the caller and passed as raw
 *    device pointers; the library never allocates device memory (its one
 *    static scratch, used by w4a16_fused_moe_noalloc only, is reserved when
 *    its code loads), never synchronises and never reads device memory from
 *    the host.  Work is
 *    enqueued on the given HIP stream (NULL = the null stream) and may be
 *    captured into a HIP graph.
 *  - All checks happen on the host before any launch; a failed check
 *    launches nothing and leaves every output untouched.
 *  - BF16 values are passed as uint16_t bit patterns, ids as int32_t,
 *    router weights as float.  Arrays are row-major and contiguous.
 *  - Routes are numbered i = t * k + j for token t and slot j.  A route is
 *    valid (local) when 0 <= topk_ids[i] < E; other ids are skipped: no output
 *    row is written for them and they contribute nothing to a combine.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    W4A16_OK = 0,
    W4A16_INVALID_ARG = -1,          /* null pointer, negative size, bad enum */
    W4A16_UNSUPPORTED_SHAPE = -2,    /* e.g. K not a multiple of 32, too many experts */
    W4A16_LAYOUT_MISMATCH = -3,      /* weight handle does not match the call */
    W4A16_WORKSPACE_TOO_SMALL = -4,  /* a caller buffer is smaller than required */
    W4A16_HIP_ERROR = -5             /* a kernel launch failed */
};

enum { W4A16_KERNEL_DECODE = 1, W4A16_KERNEL_PREFILL = 2 };

/* Weight formats of a packed weight set. */
enum { W4A16_FORMAT_INT4 = 0, W4A16_FORMAT_MXFP4 = 1 };

/* Largest expert count the routing kernel accepts. */
#define W4A16_MAX_EXPERTS 1024

/* Launch plan for one grouped GEMM, chosen by w4a16_plan_select (or filled
 * by the caller).  block_m must equal the block_m used by w4a16_route_prep
 * for the routing tensors passed with it. */
typedef struct w4a16_plan {
    int32_t kernel;        /* W4A16_KERNEL_DECODE or W4A16_KERNEL_PREFILL */
    int32_t block_m;       /* rows per route block: 16, 32, 48 or 64 (decode); 16, 32, 64 or 128 (prefill) */
    int32_t n_blocks;      /* 16-column blocks per wavefront: 1, 2 or 4 (prefill: 2 or 4; 2 with block_m 16) */
    int32_t waves;         /* wavefronts per workgroup, each owning its own columns: 4 */
    int32_t k_split;       /* workgroups sharing one output tile along K: decode 1..64, prefill 1..16
                              (the planner splits decode K for grids with few workgroups, and prefill
                              K never) */
    int32_t tile_m;        /* prefill: rows per workgroup tile (0: block_m).  With block_m 16 it is 64
                              or 144, with block_m 32 64 or 128, and a workgroup takes up to
                              tile_m / block_m consecutive route blocks of one expert; otherwise
                              tile_m equals block_m (64 or 128).  decode: 0 */
    int32_t flags;         /* 0, or W4A16_PLAN_ONE_LAUNCH on the gate_up plan of a fused call */
    int32_t reserved[1];   /* must be zero */
} w4a16_plan;

/* Plan flag, read on the gate_up plan of w4a16_fused_moe_planned: run the
 * step's gate_up and down GEMMs in one launch, down's workgroups of a route
 * block (decode) or tile (prefill) starting once gate_up has stored those rows
 * of h (humans& page, "Blackwell hides the conversion work").  Applies to
 * decode plans of 16-row blocks on the register-streaming kernel with at most
 * 4096 routes, and to prefill plans of 16-row blocks in tiles of 64 or 144
 * rows with two n-blocks per wavefront and K whole, both weight sets of one
 * format; otherwise ignored.  Outputs are bit-identical either way.  The
 * fused planner (w4a16_fused_moe_plans*) sets it on prefill plans whose down
 * GEMM reads less than 2 GB of h (n_tiles(down) x T*k x I x 2 bytes), where
 * one launch measured faster; W4A16_ONE_LAUNCH=0 or 1 (read once) forces the
 * choice.  It never sets it on decode plans: two launches were faster on the
 * Qwen3-, Kimi-K2- and DeepSeek-V3-shaped decode steps (one kernel's register
 * budget for both GEMMs, and no tail of gate_up for down to fill). */
#define W4A16_PLAN_ONE_LAUNCH 1

/* Host handle describing one packed weight set (E experts of N x K). */
typedef struct w4a16_weights w4a16_weights;

/* Message of the last failure on this thread ("" if none). */
const char* w4a16_last_error(void);

/* Library version string, including the packed-layout version. */
const char* w4a16_version(void);

/* ---------------------------------------------------------------- weights
 * Offline re-layout (Chord page, "Grouped SM90 kernels": codes [G,N,K] and
 * scales [G,N,K/32] are repacked once, before the forward path sees them).
 */

/* Bytes of the packed buffer for E experts of N x K.  K % 32 == 0 required. */
int w4a16_packed_bytes(int E, int N, int K, size_t* bytes);

/* Pack one weight set.
 *   codes   device, uint8 [E,N,K]; the low nibble of each byte is the code q
 *           (the upper nibble is ignored).
 *   scales  device, BF16 bits [E,N,K/32]; scales[e,n,g] applies to
 *           k in [32g, 32g+32).
 *   packed  device, packed_bytes >= w4a16_packed_bytes(E,N,K); written on
 *           stream s.  The caller keeps it alive while the handle is used.
 *   out     receives a host handle (free with w4a16_weights_destroy).
 * Errors: INVALID_ARG (null pointers, E/N < 1), UNSUPPORTED_SHAPE (K < 32 or
 * K % 32 != 0), WORKSPACE_TOO_SMALL (packed_bytes), HIP_ERROR. */
int w4a16_pack_weights(const uint8_t* codes, const uint16_t* scales, int E, int N, int K,
                       void* packed, size_t packed_bytes, hipStream_t s, w4a16_weights** out);

/* MXFP4 weight sets: w = e2m1(c) * 2^(e - 127), with c the E2M1 code in the
 * low nibble of codes[e,n,k] (bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and e the E8M0
 * byte scales[e,n,k/32] (b12x page, "Summary": MXFP4 experts with E8M0
 * scales; humans& page, "BF16 preserves each local product": E2M1 values
 * times their block scale are exact in BF16).  Same kernels, plans and
 * calls as INT4 weights, except decode plans need block_m 16.  Scale bytes
 * 1..252 are supported (0 puts products below the normal range, 255 is not
 * a number, 253 and 254 overflow binary32 for the largest magnitudes).
 *   codes   device, uint8 [E,N,K] (upper nibble ignored)
 *   scales  device, uint8 [E,N,K/32] (E8M0)
 *   packed  device, >= w4a16_packed_bytes_mxfp4(E,N,K) bytes
 * Errors: as w4a16_pack_weights. */
int w4a16_packed_bytes_mxfp4(int E, int N, int K, size_t* bytes);
int w4a16_pack_weights_mxfp4(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                             void* packed, size_t packed_bytes, hipStream_t s, w4a16_weights** out);

/* Format of a handle: W4A16_FORMAT_INT4 or W4A16_FORMAT_MXFP4 (negative: an
 * error code). */
int w4a16_weights_format(const w4a16_weights* w);

/* A second handle for another device buffer that holds a byte-identical copy
 * of w's packed image (for example a copy made with hipMemcpy).  Nothing is
 * launched. */
int w4a16_weights_rebind(const w4a16_weights* w, void* packed, w4a16_weights** out);

/* Shape and packed buffer of a handle (any output pointer may be NULL). */
int w4a16_weights_info(const w4a16_weights* w, int* E, int* N, int* K, void** packed, size_t* bytes);

void w4a16_weights_destroy(w4a16_weights* w);

/* Dequantise one expert from the packed buffer (verification path).
 *   out_f32  device float [N,K] or NULL: (q - 8) * s (MXFP4: e2m1(c) *
 *            2^(e-127)), exact in binary32.
 *   out_bf16 device BF16 bits [N,K] or NULL: that value rounded to nearest
 *            even, the operand the tensor-core path multiplies.
 * Errors: INVALID_ARG (expert out of range, both outputs NULL), HIP_ERROR. */
int w4a16_dequant(const w4a16_weights* w, int expert, float* out_f32, uint16_t* out_bf16, hipStream_t s);

/* ---------------------------------------------------------------- routing
 * Indexed routing (Chord page, "Two kernel families", Figure 3, and "vLLM
 * integration": over-allocated buffers consumed without reading the routed
 * count back to the host).
 */

/* Capacity of the routing tensors for T tokens, top-k, E experts and block
 * size block_m: max_padded = ceil((R + min(E,R)*(block_m-1)) / block_m) *
 * block_m with R = T*k, and max_blocks = max_padded / block_m. */
int w4a16_route_bounds(int T, int k, int E, int block_m, int* max_padded, int* max_blocks);

/* Stable counting sort of the valid routes by expert (one launch).
 *   topk_ids          device int32 [T,k]
 *   sorted_ids        device int32 [max_padded]: expert 0's routes in
 *                     ascending i, padded with the sentinel R = T*k to a
 *                     multiple of block_m, then expert 1's, ...; every slot
 *                     past num_tokens_padded also holds R.
 *   expert_ids        device int32 [max_blocks]: owner of each block_m
 *                     block, -1 past num_tokens_padded.  Experts with no
 *                     routes own no block.
 *   num_tokens_padded device int32 [1]
 *   expert_offsets    device int32 [E+1]: exclusive prefix of counts
 *   counts            device int32 [E]: valid routes per expert
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE (E > W4A16_MAX_EXPERTS, block_m not
 * a positive multiple of 16), HIP_ERROR.  T == 0 is valid. */
int w4a16_route_prep(const int32_t* topk_ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                     int32_t* expert_ids, int32_t* num_tokens_padded, int32_t* expert_offsets,
                     int32_t* counts, hipStream_t s);

/* Same outputs, bit for bit, as w4a16_route_prep, from several workgroups
 * when T*k exceeds 8192 routes (else from one, as above).  The routes are
 * cut into chunks of 4096: each chunk is counted per expert, one workgroup
 * turns the counts into offsets and each chunk's first slot per expert, and
 * each chunk is then scattered from there with the same in-chunk ranking,
 * so the order inside an expert stays ascending route index (Chord page,
 * "Two kernel families": the indexed layout; no host readback).
 *   ws   device scratch of w4a16_route_prep_workspace_bytes(T, k, E) bytes
 *        (ceil(T*k / 4096) * E ints when more than two chunks, else 0; may
 *        then be NULL), 4-byte aligned, owned by the caller, contents on
 *        entry ignored.  Calls sharing ws must not run concurrently.
 * Errors: as w4a16_route_prep, plus WORKSPACE_TOO_SMALL. */
int w4a16_route_prep_workspace_bytes(int T, int k, int E, size_t* bytes);
int w4a16_route_prep_ws(const int32_t* topk_ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                        int32_t* expert_ids, int32_t* num_tokens_padded, int32_t* expert_offsets,
                        int32_t* counts, void* ws, size_t ws_bytes, hipStream_t s);

/* Routing validation, for routing tensors built outside this library (for
 * example a serving engine's over-allocated alignment buffers).  The GEMM
 * calls trust their routing tensors, as the Chord page's indexed fast path
 * does with its routing validation switched off so that it stays
 * graph-capturable ("vLLM integration").  This call checks them on the
 * device, without a host read-back (capturable), and writes a status word:
 * 0 when valid, else a bitmask of
 *   W4A16_ROUTE_BAD_COUNT     num_tokens_padded < 0, > max_padded, or not a
 *                             multiple of block_m
 *   W4A16_ROUTE_BAD_EXPERT    a block below num_tokens_padded whose
 *                             expert_ids entry is outside [0, E)
 *   W4A16_ROUTE_BAD_SLOT      a slot below num_tokens_padded holding an id
 *                             outside [0, R] (R = T*k is the sentinel)
 *   W4A16_ROUTE_WRONG_EXPERT  (topk_ids given) a slot holding route i whose
 *                             topk_ids[i] is not its block's expert
 *   topk_ids  device int32 [R] or NULL (skip the last check)
 *   sorted_ids, expert_ids, num_tokens_padded: device tensors as produced by
 *             w4a16_route_prep for block_m, with max_padded slots
 *   status    device int32 [1], written
 * With the environment variable W4A16_VALIDATE=1 every grouped GEMM call
 * that takes routing tensors runs this check first, synchronises the stream
 * and fails with INVALID_ARG on a non-zero status (a debugging mode: it
 * synchronises, so it cannot be captured).
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, HIP_ERROR. */
enum {
    W4A16_ROUTE_BAD_COUNT = 1,
    W4A16_ROUTE_BAD_EXPERT = 2,
    W4A16_ROUTE_BAD_SLOT = 4,
    W4A16_ROUTE_WRONG_EXPERT = 8
};
int w4a16_validate_routing(const int32_t* topk_ids, int R, int E, int block_m, const int32_t* sorted_ids,
                           const int32_t* expert_ids, const int32_t* num_tokens_padded, int max_padded,
                           int32_t* status, hipStream_t s);

/* ---------------------------------------------------------------- planning */

/* Choose a plan from the routed rows per expert, not the token count (Chord
 * page, "TL;DR" and "Indexed kernels").  expected_rows_per_expert <= 0 means
 * T*k/E.  Host only and memoised; environment overrides W4A16_FORCE_KERNEL
 * (decode|prefill; also read as W4A16_FORCE_SCHEDULE), W4A16_BLOCK_M, W4A16_N_BLOCKS, W4A16_WAVES,
 * W4A16_K_SPLIT and W4A16_TILE_M are read once and are part of the memo
 * key. */
int w4a16_plan_select(int T, int k, int E, int N, int K, float expected_rows_per_expert, w4a16_plan* out);

/* ---------------------------------------------------------------- GEMM */

/* Indexed grouped GEMM:
 *   for every slot p < num_tokens_padded of a block b with expert_ids[b] =
 *   e >= 0 and sorted_ids[p] = i < R:
 *     out[i, n] = bf16( sum_k A[i / a_row_div, k] * w[e, n, k] ),  n < N
 * accumulated in binary32 and rounded to nearest even.
 *   A          device BF16 bits [*, K] (x [T,K] with a_row_div = k, or
 *              h [R,K] with a_row_div = 1)
 *   routing    as produced by w4a16_route_prep with p->block_m for R routes
 *              and the handle's E experts; the kernels read
 *              num_tokens_padded on the device to find the valid route
 *              blocks (NULL: every block up to the bound of
 *              w4a16_route_bounds is visited, and blocks with expert_ids -1
 *              are skipped)
 *   out        device BF16 bits [R, N]; rows of invalid routes untouched
 *   ws         workspace of w4a16_gemm_workspace_bytes (may be NULL if 0).  A
 *              prefill plan with tile_m above block_m builds its tile list
 *              there.  A plan with k_split > 1 (decode or prefill) keeps
 *              partial tiles and per-tile arrival counters in it:
 *              the workspace must be zero-filled once before its first use,
 *              and every call leaves the counters at zero again.  Calls that
 *              share a workspace must not run concurrently.
 * Errors: INVALID_ARG, LAYOUT_MISMATCH (bad handle), UNSUPPORTED_SHAPE (plan
 * values outside the supported set; a prefill plan with one expert's packed
 * weights or the activation matrix of 2 GiB or more), WORKSPACE_TOO_SMALL,
 * HIP_ERROR. */
int w4a16_gemm_workspace_bytes(const w4a16_plan* p, int R, int E, int N, size_t* bytes);
/* The same size for R = T*k routes, in the argument order of the planning
 * calls (T tokens, top-k). */
int w4a16_workspace_bytes(const w4a16_plan* p, int T, int k, int E, int N, size_t* bytes);

int w4a16_grouped_gemm(const uint16_t* A, int a_row_div, const w4a16_weights* w, const int32_t* sorted_ids,
                       const int32_t* expert_ids, const int32_t* num_tokens_padded, int R,
                       const w4a16_plan* p, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s);

/* Same as w4a16_grouped_gemm, but out is device float [R, N] holding the
 * binary32 accumulators unrounded (for a consumer that keeps full precision,
 * such as the down projection feeding the weighted combine). */
int w4a16_grouped_gemm_f32(const uint16_t* A, int a_row_div, const w4a16_weights* w, const int32_t* sorted_ids,
                           const int32_t* expert_ids, const int32_t* num_tokens_padded, int R,
                           const w4a16_plan* p, float* out, void* ws, size_t ws_bytes, hipStream_t s);

/* Gate/up projection with the expert MLP's activation in its epilogue
 * (humans& page, "Dedicated warps keep the pipeline busy": FC1 followed by
 * the activation; SiLU-gated MLP as in the DeepSeek-V3 and Qwen3 MoE layers):
 * w13 holds [E, 2I, K] weights, gate rows [0, I) then up rows [I, 2I), and
 *   h[i, c] = bf16( silu(g) * u ),  silu(g) = g / (1 + exp(-g)),  c < I,
 *   g = sum_k A[i / a_row_div, k] * w13[e, c, k],
 *   u = sum_k A[i / a_row_div, k] * w13[e, I + c, k],
 * g and u accumulated in binary32 and never rounded; the activation is formed
 * in binary32 and rounded once to nearest even.  Exactly
 * w4a16_grouped_gemm_f32 followed by w4a16_silu_mul_f32, without the [R, 2I]
 * intermediate.  h device BF16 bits [R, I]; other arguments and the workspace
 * as for w4a16_grouped_gemm.  Needs 2I a multiple of 32 and
 * p->n_blocks >= 2 (UNSUPPORTED_SHAPE otherwise). */
int w4a16_grouped_gemm_silu(const uint16_t* A, int a_row_div, const w4a16_weights* w13, const int32_t* sorted_ids,
                            const int32_t* expert_ids, const int32_t* num_tokens_padded, int R,
                            const w4a16_plan* p, uint16_t* h, void* ws, size_t ws_bytes, hipStream_t s);

/* Offsets-form grouped GEMM (nf4 page, "Usage": x sorted by expert, offsets =
 * cumulative rows per expert): rows [expert_offsets[e], expert_offsets[e+1])
 * of A_sorted belong to expert e, and
 *   out[r, n] = bf16( sum_k A_sorted[r, k] * w[e(r), n, k] ),  r < expert_offsets[E].
 *   expert_offsets  device int32 [E+1], non-decreasing, expert_offsets[E] <= rows_max
 *   rows_max        host bound on expert_offsets[E] (sizes the launch)
 *   ws              >= w4a16_offsets_workspace_bytes(rows_max, w, p), zero-filled
 *                   once before its first use when p->k_split > 1
 * Rows r >= expert_offsets[E] of out are untouched. */
int w4a16_offsets_workspace_bytes(int rows_max, const w4a16_weights* w, const w4a16_plan* p, size_t* bytes);

int w4a16_grouped_gemm_offsets(const uint16_t* A_sorted, const int32_t* expert_offsets, int rows_max,
                               const w4a16_weights* w, const w4a16_plan* p, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t s);

/* Contiguous-form grouped GEMM (Chord page, "Grouped SM90 kernels": rows
 * concatenated by expert, each expert padded to 128 rows, with m_indices
 * giving each row's expert and -1 on padding rows):
 *   out[r, n] = bf16( sum_k A[r, k] * w[m_indices[r], n, k] )
 * for every r < m with 0 <= m_indices[r] < E; other rows of out are untouched.
 *   A          device BF16 bits [m, K], 16-byte aligned
 *   m_indices  device int32 [m]
 *   out        device BF16 bits [m, N]
 *   ws         >= w4a16_contiguous_workspace_bytes(m, w, p), 16-byte aligned,
 *              zero-filled once before its first use when p->k_split > 1
 * The rows are grouped by expert on the device (the routing of
 * w4a16_route_prep with one route per row), so the 128-row padding and even
 * the grouping itself are accepted but not required.  The same kernels as
 * w4a16_grouped_gemm; p->block_m is the route block of that grouping.
 * Errors: INVALID_ARG, LAYOUT_MISMATCH, UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL,
 * HIP_ERROR. */
int w4a16_contiguous_workspace_bytes(int m, const w4a16_weights* w, const w4a16_plan* p, size_t* bytes);
int w4a16_grouped_gemm_contiguous(const uint16_t* A, const int32_t* m_indices, int m, const w4a16_weights* w,
                                  const w4a16_plan* p, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s);

/* Masked-form grouped GEMM (Chord page, "Grouped SM90 kernels": a fixed
 * per-expert row budget max_m, the valid count per expert in masked_m, a
 * flat output whose rows past each expert's count are to be ignored):
 *   out[e*max_m + r, n] = bf16( sum_k A[e*max_m + r, k] * w[e, n, k] )
 * for r < min(masked_m[e], max_m); the other rows of out are untouched.
 *   A          device BF16 bits [E, max_m, K] (flat [E*max_m, K]), 16-byte aligned
 *   masked_m   device int32 [E] (negative counts as 0, above max_m as max_m)
 *   out        device BF16 bits [E*max_m, N]
 *   ws         >= w4a16_masked_workspace_bytes(max_m, w, p), as above
 * The pages' host-side expected_m is a planning input: pass it to
 * w4a16_plan_select as the expected rows per expert.  E*max_m must fit int32.
 * Errors: as the contiguous form. */
int w4a16_masked_workspace_bytes(int max_m, const w4a16_weights* w, const w4a16_plan* p, size_t* bytes);
int w4a16_grouped_gemm_masked(const uint16_t* A, const int32_t* masked_m, int max_m, const w4a16_weights* w,
                              const w4a16_plan* p, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------- expert MLP */

/* h[r, c] = bf16( silu(gu[r, c]) * gu[r, I + c] ), silu(g) = g / (1 + exp(-g)),
 * for r < rows, c < I.  gu device BF16 bits [rows, 2I] (gate columns first),
 * h device BF16 bits [rows, I]. */
int w4a16_silu_mul(const uint16_t* gu, int rows, int I, uint16_t* h, hipStream_t s);

/* As w4a16_silu_mul with binary32 gate/up values: gu device float [rows, 2I]. */
int w4a16_silu_mul_f32(const float* gu, int rows, int I, uint16_t* h, hipStream_t s);

/* out[t, n] = bf16( sum over valid j ascending of topk_w[t,j] * y[t*k+j, n] ),
 * binary32 accumulation; tokens without a valid route get zeros.
 * y device float [T*k, H]; topk_w device float [T,k]; topk_ids device int32
 * [T,k]; out device BF16 bits [T,H] (every row written). */
int w4a16_moe_combine(const float* y, const float* topk_w, const int32_t* topk_ids, int T, int k, int E,
                      int H, uint16_t* out, hipStream_t s);

/* w4a16_moe_combine over y in BF16 (y device BF16 bits [T*k, H], 4-byte
 * aligned): each y value is widened exactly to binary32, then summed as
 * above.  The fused step's y is BF16: rounding the down projection's output
 * costs at most 2^-9 of each value and halves the bytes that down writes and
 * this combine reads. */
int w4a16_moe_combine_bf16(const uint16_t* y, const float* topk_w, const int32_t* topk_ids, int T, int k, int E,
                           int H, uint16_t* out, hipStream_t s);

/* Fused expert MLP: route_prep -> gate_up GEMM with SiLU*mul -> down GEMM ->
 * weighted top-k combine.  Its output is exactly that of the sequence
 * w4a16_route_prep, w4a16_grouped_gemm_silu (a_row_div = k),
 * w4a16_grouped_gemm (down, a_row_div = 1, BF16 y), w4a16_moe_combine_bf16,
 * with the plans of w4a16_fused_moe_plans and the buffers carved from ws.
 * y is BF16: half the bytes of binary32 for down to write and the combine to
 * read, for one more rounding per route (at most 2^-9 of that route's value).  A decode
 * step (decode plans of 16-row blocks, at most 4096 routes) routes its rows
 * inside the gate_up kernel instead of a separate launch: the same routing
 * tensors and outputs, one launch fewer.
 *   x       device BF16 bits [T,H]
 *   w13     handle of [E, 2I, H] weights, gate rows first then up rows
 *   w2      handle of [E, H, I] weights
 *   out     device BF16 bits [T,H]; every row written (zero rows for
 *           tokens without a valid route)
 *   ws      >= w4a16_fused_moe_workspace_bytes(T, k, w13, w2), zero-filled
 *           once before its first use (split-K counters; each call leaves
 *           them at zero); calls sharing a workspace must not overlap.
 * Errors: INVALID_ARG, LAYOUT_MISMATCH (w13 not [E,2I,H] with w2 [E,H,I]),
 * WORKSPACE_TOO_SMALL, HIP_ERROR. */
int w4a16_fused_moe_workspace_bytes(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                                    size_t* bytes);

/* The two plans w4a16_fused_moe uses (they share block_m, hence one set of
 * routing tensors; the gate_up plan has n_blocks >= 2, and carries
 * W4A16_PLAN_ONE_LAUNCH where the planner runs the two GEMMs in one launch). */
int w4a16_fused_moe_plans(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2, w4a16_plan* gate_up,
                          w4a16_plan* down);

int w4a16_fused_moe(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                    const w4a16_weights* w13, const w4a16_weights* w2, uint16_t* out, void* ws,
                    size_t ws_bytes, hipStream_t s);

/* w4a16_fused_moe that also records caller-created events on the stream
 * between its stages: stage_events[0] before routing, [1] before gate_up
 * (with the activation), [2] before down, [3] before the combine and [4]
 * after it (NULL = no events, identical to w4a16_fused_moe).  When gate_up
 * routes its own rows the routing stage is empty; when gate_up and down run
 * in one launch (W4A16_PLAN_ONE_LAUNCH) the gate_up stage holds both and
 * the down stage is empty.  For per-stage timing of eager calls; nothing
 * else differs. */
int w4a16_fused_moe_profiled(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                             const w4a16_weights* w13, const w4a16_weights* w2, uint16_t* out, void* ws,
                             size_t ws_bytes, hipStream_t s, hipEvent_t* stage_events);

/* The fused plans for an expected number of routed rows per expert (as in
 * w4a16_plan_select; <= 0 means T*k/E).  An expert-parallel share of
 * E local experts out of G receives about T*k/G rows per local expert: the
 * default T*k/E overstates that G/E times and can pick prefill plans where
 * the decode kernel is faster (Chord page, "TL;DR": the schedule follows
 * routed rows per expert). */
int w4a16_fused_moe_plans_hint(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                               float expected_rows_per_expert, w4a16_plan* gate_up, w4a16_plan* down);

/* w4a16_fused_moe with caller-chosen plans (for example from
 * w4a16_fused_moe_plans_hint).  The plans must be valid on their own, share
 * kernel and block_m (one set of routing tensors), the gate_up plan needs
 * n_blocks >= 2, prefill plans share their tile height, and MXFP4 weights
 * take decode plans of block_m 16 only; otherwise INVALID_ARG or
 * UNSUPPORTED_SHAPE before anything is launched.  ws holds at least
 * w4a16_fused_moe_planned_workspace_bytes for the same plans, zero-filled
 * once before its first use.  stage_events: NULL or five events, as in
 * w4a16_fused_moe_profiled. */
int w4a16_fused_moe_planned_workspace_bytes(int T, int k, const w4a16_weights* w13, const w4a16_weights* w2,
                                            const w4a16_plan* gate_up, const w4a16_plan* down, size_t* bytes);
int w4a16_fused_moe_planned(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                            const w4a16_weights* w13, const w4a16_weights* w2, const w4a16_plan* gate_up,
                            const w4a16_plan* down, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s,
                            hipEvent_t* stage_events);

/* Bytes of the library's static device scratch, the only device memory the
 * library itself holds: one copy per GPU the library runs on, reserved when
 * the library's code is loaded there and kept until the process ends. */
#define W4A16_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* w4a16_fused_moe for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plans (w4a16_fused_moe_plans), kernels and results bit for bit,
 * with every intermediate (routing tensors, split-K partials and counters,
 * tile list, h, y) in the library's static scratch of
 * W4A16_NOALLOC_SCRATCH_BYTES instead of a caller workspace.  It calls no
 * allocating routine; the caller still passes inputs and the output.
 *   x, topk_ids, topk_w, T, k, w13, w2, out: as in w4a16_fused_moe.
 * A call whose workspace (w4a16_fused_moe_workspace_bytes) exceeds the
 * scratch fails with WORKSPACE_TOO_SMALL before anything is launched; that
 * covers steps up to about R*(2H + 2I) bytes of intermediates, e.g.
 * 512 tokens of the Kimi-K2 one-GPU share or 2048 of a Qwen3-30B-A3B layer.
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind; the split-K counters are cleared on the stream before use.  Calls
 * that overlap on one GPU (other streams, other threads) race.
 * Errors: as w4a16_fused_moe, plus HIP_ERROR when the scratch's device address
 * cannot be obtained. */
int w4a16_fused_moe_noalloc(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, int T, int k,
                            const w4a16_weights* w13, const w4a16_weights* w2, uint16_t* out, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
