// Internal declarations of libw4a16 (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

namespace w4a16 {

// ---------------------------------------------------------------------------
// Packed weight layout (version 1).
//
// The packed image of one weight set is a sequence of "superblocks", each
// covering 16 output rows (an n-block) and 256 consecutive k (8 scale groups)
// of one expert, stored at
//     ((e * NB + nb) * KB + kb) * SB_BYTES
// with NB = ceil(N/16) and KB = ceil(K/256).  One superblock is 2304 bytes:
//
//   bytes [0, 2048): codes, two halves h = 0, 1 of 1024 bytes.  In half h,
//     the 16 bytes at (c*16 + j)*16 hold four 32-bit words d = 0..3 for
//     output row n = 16*nb + j and scale group g = 4*h + d; word d carries
//     the eight codes of k = 256*kb + 32*g + 8*c + u, u = 0..7, code u = 2p
//     in bits [4p, 4p+4) and code u = 2p+1 in bits [16+4p, 20+4p).
//   bytes [2048, 2304): scales, 16 bytes per row j: BF16 scale of groups
//     g = 0..7 of row 16*nb + j.
//
// Rows n >= N carry code 8 and scale 0 (weight 0); groups past K carry code 8
// and scale 0 and are never read by the GEMM kernels.
//
// MXFP4 weight sets (E2M1 codes, one E8M0 scale byte per 32 k) use the same
// superblock geometry with two differences: word d carries code u in bits
// [4u, 4u+4) (each byte holds two neighbouring k, the pair the hardware
// FP4 -> BF16 conversion takes), and the scales are one byte per group, 8
// bytes per row j at 2048 + 8*j, so a superblock is 2176 bytes.  Padding is
// code 0 (+0) with scale 127 (1.0).
//
// Why this order: one wavefront of 64 lanes loading 16 contiguous bytes per
// lane reads exactly one half (1024 bytes, fully coalesced), and lane
// L = c*16 + j then holds, for each of four groups, the eight codes that the
// 16x16x32 BF16 MFMA expects in its B operand for column j and k-slot c.  The
// scales of a row ride in the same superblock, so the whole weight stream is
// a single sequential read per (expert, n-block).  Decode and prefill kernels
// read the same image.
// ---------------------------------------------------------------------------
constexpr int kLayoutVersion = 1;
constexpr int NB_ROWS = 16;     // output rows per n-block
constexpr int SB_K = 256;       // k per superblock
constexpr int SB_GROUPS = 8;    // scale groups per superblock
constexpr int SB_CODE_BYTES = 2048;
constexpr int SB_SCALE_BYTES = 256;
constexpr int SB_BYTES = SB_CODE_BYTES + SB_SCALE_BYTES;
constexpr int SB_BYTES_MXFP4 = SB_CODE_BYTES + NB_ROWS * SB_GROUPS;
constexpr uint32_t kHandleMagic = 0x34413136u;  // "41A6"

// Weight formats (the value is the public W4A16_FORMAT_* constant).
constexpr int kFmtInt4 = W4A16_FORMAT_INT4;
constexpr int kFmtMxfp4 = W4A16_FORMAT_MXFP4;

// Superblock bytes of a format.
__host__ __device__ constexpr int sb_bytes(int fmt) { return fmt == kFmtMxfp4 ? SB_BYTES_MXFP4 : SB_BYTES; }

struct Shape {
    int E, N, K;
    int NB, KB, G;  // n-blocks, superblocks along K, scale groups (K/32)
    int fmt;        // kFmtInt4 or kFmtMxfp4
};

inline Shape make_shape(int E, int N, int K, int fmt = kFmtInt4) {
    Shape s;
    s.E = E; s.N = N; s.K = K;
    s.NB = (N + NB_ROWS - 1) / NB_ROWS;
    s.KB = (K + SB_K - 1) / SB_K;
    s.G = K / 32;
    s.fmt = fmt;
    return s;
}

inline size_t packed_bytes(const Shape& s) {
    return (size_t)s.E * s.NB * s.KB * sb_bytes(s.fmt);
}

}  // namespace w4a16

// Host handle (opaque to callers).
struct w4a16_weights {
    uint32_t magic;
    uint32_t layout_version;
    w4a16::Shape shape;
    void* packed;
    size_t bytes;
};

namespace w4a16 {

// Output modes of the GEMM kernels.
//   kOutBf16: out[row, n] = bf16(acc)
//   kOutF32:  out[row, n] = acc
//   kOutAct:  the weight rows are [gate (N/2 rows); up (N/2 rows)] and
//             out[row, n] = bf16(silu(acc_gate[n]) * acc_up[n]), n < N/2;
//             each wavefront takes half of its n-blocks from the gate rows and
//             the matching half from the up rows, so both halves of an output
//             column end in the same lane.
constexpr int kOutBf16 = 0, kOutF32 = 1, kOutAct = 2;

// Launchers (return hipError_t of the launch).
hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, const Shape& sh, void* packed, hipStream_t s);
hipError_t launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, const Shape& sh, void* packed,
                             hipStream_t s);
hipError_t launch_dequant(const void* packed, const Shape& sh, int expert, float* out_f32, uint16_t* out_bf16,
                          hipStream_t s);
// Optional output of the routing: the tile list of a prefill GEMM whose tiles gather `group` route blocks (the
// records tile_map_kernel builds), written from the per-expert counts; tiles == nullptr: none.
struct TileOut {
    int group = 0;
    int32_t* tiles = nullptr;
    int32_t* count = nullptr;
};
hipError_t launch_route_prep(const int32_t* topk_ids, int R, int E, int block_m, int max_padded, int max_blocks,
                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp, int32_t* offsets,
                             int32_t* counts, hipStream_t s, TileOut to = TileOut{});
// Ints of scratch the routing of R routes uses when spread over several workgroups (0: one workgroup does it).
size_t route_prep_scratch_ints(int R, int E);
hipError_t launch_route_prep_scratch(const int32_t* topk_ids, int R, int E, int block_m, int max_padded,
                                     int max_blocks, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                                     int32_t* offsets, int32_t* counts, int32_t* scratch, hipStream_t s,
                                     TileOut to = TileOut{});
hipError_t launch_route_validate(const int32_t* topk_ids, int R, int E, int block_m, const int32_t* sorted_ids,
                                 const int32_t* expert_ids, const int32_t* ntp, int max_padded, int32_t* status,
                                 hipStream_t s);
hipError_t launch_tile_map(const int32_t* expert_ids, const int32_t* ntp, int block_m, int max_blocks, int group,
                           int32_t* tiles, int32_t* count, int32_t* scratch, hipStream_t s);
hipError_t launch_masked_to_route(const int32_t* masked_m, int E, int max_m, int block_m, int max_padded,
                                  int max_blocks, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                                  hipStream_t s);
hipError_t launch_offsets_to_route(const int32_t* offsets, int E, int rows_max, int block_m, int max_padded,
                                   int max_blocks, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                                   hipStream_t s);

// Routes up to which a decode gate_up routes its rows in-kernel (the top-k ids are staged in LDS).
constexpr int kSelfRouteMaxRoutes = 4096;
// LDS ints of that routing: per-expert counts [E], first block of each expert [E + 1], wavefront totals of the
// scans, then the top-k ids [R]
constexpr int kSelfRouteLdsInts = 2 * W4A16_MAX_EXPERTS + 8 + kSelfRouteMaxRoutes;

struct GemmArgs {
    const uint16_t* A;
    int a_row_div;
    const void* packed;
    Shape sh;
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    int R;             // sentinel value / number of routes
    int max_blocks;    // route blocks (grid.x)
    void* out;         // BF16 bits [R,N], float [R,N], or BF16 bits [R,N/2] (activation mode)
    int out_mode;      // kOutBf16, kOutF32 or kOutAct
    const int32_t* ntp = nullptr;  // num_tokens_padded (device) when known: bounds the valid route blocks
    int32_t* tiles = nullptr;      // prefill tiles of several route blocks: tile list (first block, blocks) pairs
    int32_t* tile_count = nullptr; // ... and its length (device)
    int32_t* tile_scratch = nullptr; // 2 * max_blocks ints the tile list is built with
    bool tiles_ready = false;        // the tile list already holds this routing's tiles (built by an earlier GEMM)
    float* partials = nullptr;     // split-K partial tiles (decode, k_split > 1)
    unsigned* counters = nullptr;  // split-K arrival counters, zero between calls
    // decode gate_up only: route the rows in-kernel from these top-k ids [R] and write sorted_ids, expert_ids and
    // num_tokens_padded (the buffers above, which must then be writable) for the GEMMs that follow
    const int32_t* self_route_ids = nullptr;
};

int decode_n_tiles(const Shape& sh, const w4a16_plan& p);
size_t decode_partial_floats(const Shape& sh, const w4a16_plan& p, int max_blocks);
size_t decode_counters(const Shape& sh, const w4a16_plan& p, int max_blocks);

hipError_t launch_gemm_decode(const GemmArgs& a, const w4a16_plan& p, hipStream_t s);
bool decode_reg_supported(const GemmArgs& a, const w4a16_plan& p);
hipError_t launch_gemm_decode_reg(const GemmArgs& a, const w4a16_plan& p, hipStream_t s);
// The decode step's gate_up (SiLU*mul into h) and down (BF16 y) in one launch, both on the register-streaming
// kernel with in-kernel routing (self_route_ids set in both), down's workgroups of a route block starting once
// gate_up's column tiles of that block have stored h.  sync: 2 * max_blocks + 1 words, zero at rest; each
// GEMM's split-K area its own.
bool decode_fused_supported(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2);
hipError_t launch_gemm_decode_fused(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2,
                                    const w4a16_plan& p2, unsigned* sync, hipStream_t s);
hipError_t launch_gemm_prefill(const GemmArgs& a, const w4a16_plan& p, hipStream_t s);
// gate_up and down of a fused prefill step in one launch: down's workgroups of a tile wait until gate_up has stored
// that tile's rows of h.  sync: 2 * max_blocks + 1 words, zero at rest (each launch leaves them zero).
bool prefill_fused_supported(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2);
hipError_t launch_gemm_prefill_fused(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2,
                                     const w4a16_plan& p2, unsigned* sync, hipStream_t s);
bool prefill_supported(const GemmArgs& a);
// Rows per prefill workgroup tile (plan.tile_m, else block_m); 16- and 32-row route blocks are gathered into
// taller tiles through a tile list.
int prefill_tile_rows(const w4a16_plan& p);
// Split-K workspace of a prefill plan (k_split > 1): fp32 partial tiles and (tile, column tile) counters.
int prefill_n_tiles(const Shape& sh, const w4a16_plan& p);
size_t prefill_max_tiles(const Shape& sh, const w4a16_plan& p, int max_blocks);
size_t prefill_partial_floats(const Shape& sh, const w4a16_plan& p, int max_blocks);
size_t prefill_counters(const Shape& sh, const w4a16_plan& p, int max_blocks);
hipError_t launch_silu_mul(const uint16_t* gu, int rows, int I, uint16_t* h, hipStream_t s);
hipError_t launch_silu_mul_f32(const float* gu, int rows, int I, uint16_t* h, hipStream_t s);
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t s);
hipError_t launch_combine(const float* y, const float* tw, const int32_t* ids, int T, int k, int E, int H,
                          uint16_t* out, hipStream_t s);
hipError_t launch_combine_bf16(const uint16_t* y, const float* tw, const int32_t* ids, int T, int k, int E, int H,
                               uint16_t* out, hipStream_t s);

}  // namespace w4a16
