// Prefill grouped GEMM: many routed rows per expert, bound by the matrix cores.
//
// Design (MI355X-first):
//  * One workgroup of four wavefronts per (route block of BM = 16*MT rows of
//    one expert, 64*NBW weight columns).  The owning expert comes from
//    expert_ids[block] in-kernel, so no host synchronisation is needed (Chord
//    page, "Two kernel families"; the nf4 page, "How it works", finds its
//    tiles in-kernel the same way).
//  * With route blocks of 16 or 32 rows, a workgroup takes a tile of up to
//    BM/16 or BM/32 consecutive blocks of one expert from a tile list built
//    on the device, and runs a body specialised for the tile's height.
//    Padding then costs less than one route block per expert instead of up
//    to BM-1 rows, while the dequantisation is still shared by all rows of
//    the tile (up to 144 of them).
//  * Tile order is XCD-aware.  Consecutive workgroup ids go to the eight XCDs
//    in turn, so id -> (XCD, position) is remapped to give every XCD runs of
//    consecutive (tile, column tile) pairs, tile major: the ~64 workgroups an
//    XCD runs at a time then cover one or two tiles across all column tiles,
//    sharing those rows of activations and the expert's weight slices in the
//    XCD's L2.  The runs are chunks of the valid pairs only (from the routed
//    row count num_tokens_padded, read on the device), about six per XCD and
//    dealt to the XCDs in turn: with skewed routing the tall tiles of the
//    busiest experts come first, and one contiguous range per XCD would leave
//    the first XCDs with most of the work.
//  * The BM gathered activation rows are streamed HBM -> LDS by direct loads
//    (buffer_load ... lds) into a two-slot ring of 128-k stages, stored
//    unpadded with each row's 16-byte chunks XOR-permuted by the row, so the
//    16 rows of an MFMA fragment hit 16 distinct bank groups.  Sentinel rows
//    and k past K read zeros (an offset past the resource).  No registers hold
//    activations in flight.
//  * Each wavefront owns NBW n-blocks across all BM rows.  Its packed weights
//    for the next stage are in flight in a second register set (buffer loads,
//    scalar stage offsets) while the current stage is multiplied.  Every
//    weight is dequantised once per workgroup, to bf16((q - 8) * s) (one
//    mixed-precision FMA on a binary16 pattern of the code, exact, then one
//    rounding; 17 operations per 8 weights and 3 per scale group), and feeds
//    MT MFMAs (v_mfma_f32_16x16x32_bf16):
//    a taller M tile amortises the INT4 conversion (Chord page, "Grouped SM90
//    kernels").  The dequantisation of group g+1 is independent of the MFMAs
//    of group g, so the two interleave.
//  * MXFP4 weights (FMT = kFmtMxfp4) convert in hardware: two E2M1 codes and
//    their E8M0 scale to exact BF16 per instruction, 4 instructions per 8
//    weights instead of about 20.
//  * At most 256 registers per lane for the 128x32 and 64x64 wavefront tiles,
//    so two wavefronts share each SIMD: one issues VALU dequantisation while
//    the other's MFMAs run.
#include <type_traits>

#include "frag.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int KT = 128;        // k per stage (4 scale groups, half a superblock)
constexpr int kThreads = 256;  // four wavefronts, each owning its own columns
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;       // XCDs of the chip; workgroup i runs on XCD i % 8
// XCD order: the valid (tile, column tile) pairs are cut into chunks of consecutive pairs, at least kChunkMin long
// and about kChunkRounds per XCD, and chunk j runs on XCD j % 8
constexpr int kChunkMin = 32;
constexpr int kChunkRounds = 6;

struct PrefillParams {
    const uint16_t* A;
    int a_row_div;
    const uint8_t* packed;
    Shape sh;
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    const int32_t* ntp;  // num_tokens_padded (device) or NULL: every block of the grid may be valid
    int R;
    int max_blocks;
    int n_tiles;
    void* out;
    const int32_t* tiles;       // tile list (first route block, blocks), or NULL: one route block of BM rows per tile
    const int32_t* tile_count;  // its length (device)
    // split K (grid.y slices): fp32 partial tiles [tile][n_tiles][KS][BM][COLS] and one arrival counter per
    // (tile, column tile), zero between calls
    float* partials;
    unsigned* counters;
};

// gate_up and down of a fused step in one launch (gate_up workgroups first, then down workgroups): a tile's down
// workgroups wait until every gate_up column tile of that tile has stored its rows of h.
struct PrefillSync {
    unsigned* ready;     // [tiles]: gate_up column tiles whose rows of h are stored; zero at rest
    unsigned* done;      // [tiles]: down workgroups finished; the last one resets both; zero at rest
    unsigned* timeouts;  // counts down workgroups that stopped waiting (never in a correct launch)
    unsigned ready_target, done_target;
};
constexpr int kRolePlain = 0, kRoleGateUp = 1, kRoleDown = 2;
// bounded wait of a down workgroup: about a second of polling (the gate_up workgroups it waits for were dispatched
// before it and wait on nothing, so this bound is never reached in a correct launch; it only guarantees an end)
constexpr unsigned kMaxPolls = 1u << 24;

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier between stages that leaves direct loads in flight (__syncthreads would drain them): each wavefront has
// waited for its own loads of the stage; its LDS reads of the previous stage complete before the barrier.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

template <int NBW>
struct WStage {
    u32x4 cw[NBW];        // codes of half h of the superblock, per n-block
    uint32_t sc[NBW][2];  // scales of groups 4h .. 4h+3 of row j, per n-block
};

// Wavefronts per SIMD a tile shape is built for: two, except the 128 x 64 wavefront tile, whose 128 accumulators
// plus operands need more than half the register file.
template <int MT, int NBW>
constexpr int prefill_waves_per_simd() {
    return MT * NBW >= 32 ? 1 : 2;
}

// Split K: every slice publishes its fp32 partial tile with device-coherent stores and bumps the (tile, column
// tile) counter; the last to arrive adds the KS partials in slice order, writes the output in its mode and resets
// the counter.  Partial tiles are BM = 16*MT rows (the kernel's tallest tile) by COLS columns; a tile of MTA < MT
// row groups uses the first 16*MTA rows.
template <int MTA, int NBW, int OM, int MT>
__device__ __forceinline__ void prefill_split_epilogue(const PrefillParams& p, const f32x4 (&acc)[MTA][NBW],
                                                       const int* ssid, int* s_last, int nt, int t, int ks, int KS,
                                                       int w, int c, int j) {
    constexpr int BM = 16 * MT, ROWS = 16 * MTA;
    constexpr int COLS = NBW * 16 * kWaves;
    const Shape& sh = p.sh;
    const size_t tile = (size_t)t * p.n_tiles + nt;
    float* mine = p.partials + (tile * KS + ks) * (size_t)(BM * COLS);
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
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
    if (!*s_last) return;
    const float* all = p.partials + tile * KS * (size_t)(BM * COLS);
    auto reduce = [&](int idx) {
        float v = 0.f;
        for (int z = 0; z < KS; ++z)
            v += __hip_atomic_load(&all[(size_t)z * BM * COLS + idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return v;
    };
    if (OM == kOutAct) {
        // output column oc of the tile: wavefront oc / (16*HB), its slot (oc / 16) % HB, lane column oc % 16
        constexpr int HB = NBW / 2, OCOLS = COLS / 2;
        const int NO = sh.N / 2;
        for (int idx = threadIdx.x; idx < ROWS * OCOLS; idx += kThreads) {
            const int m = idx / OCOLS, oc = idx % OCOLS;
            const int sid = ssid[m];
            const int ww = oc / (16 * HB), q = (oc / 16) % HB, jj = oc % 16;
            const int n = ((nt * kWaves + ww) * HB + q) * 16 + jj;
            if (sid < 0 || n >= NO) continue;
            const int gcol = (ww * NBW + q) * 16 + jj;
            const float g = reduce(m * COLS + gcol), u = reduce(m * COLS + gcol + HB * 16);
            static_cast<uint16_t*>(p.out)[(size_t)sid * NO + n] = f32_to_bf16_bits(silu_mul(g, u));
        }
    } else {
        const int n_base = nt * COLS;
        for (int idx = threadIdx.x; idx < ROWS * COLS; idx += kThreads) {
            const int m = idx / COLS, col = idx % COLS;
            const int sid = ssid[m];
            const int n = n_base + col;
            if (sid < 0 || n >= sh.N) continue;
            const float v = reduce(idx);
            if (OM == kOutF32)
                static_cast<float*>(p.out)[(size_t)sid * sh.N + n] = v;
            else
                static_cast<uint16_t*>(p.out)[(size_t)sid * sh.N + n] = f32_to_bf16_bits(v);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One tile: 16*MTA rows starting at route slot row0, all of them of expert e, times the column tile nt.  The
// LDS ring and the row table are the kernel's (sized for its largest tile).
template <int MTA, int NBW, int OM, int FMT, int MT, int ROLE = kRolePlain>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, uint8_t* slot0, uint8_t* slot1, int* ssid,
                                             int* s_last, int row0, int e, int nt, int t, const PrefillSync* fs) {
    constexpr int BM = 16 * MTA;                // rows of this tile
    constexpr int ROWS_PER_WAVE = BM / kWaves;  // activation rows each wavefront streams
    constexpr int DMA = ROWS_PER_WAVE / 4;      // direct loads per wavefront per stage (4 rows of 256 B each)
    static_assert(ROWS_PER_WAVE % 4 == 0, "a direct load fills four rows");
    const Shape sh = p.sh;
    const int K = sh.K;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const int wave_global = nt * kWaves + w;
    const int nst = (sh.G + 3) / 4;
    // this workgroup's K slice: stages [st_begin, st_end) of nst (all of them without split K)
    const int KS = gridDim.y, ks = blockIdx.y;
    const int st_begin = (int)((long)ks * nst / KS), st_end = (int)((long)(ks + 1) * nst / KS);

    for (int m = threadIdx.x; m < BM; m += kThreads) {
        const int sid = p.sorted_ids[row0 + m];
        ssid[m] = sid < p.R ? sid : -1;
    }

    // ---- activation stream: wavefront w fills rows [w*RPW, (w+1)*RPW) of each slot, 4 rows per direct load;
    // lane L of load r writes row w*RPW + 4r + L/16, physical chunk L%16, which holds chunk (L%16) ^ (row%16)
    const uint32_t a_bytes = (uint32_t)(p.R / p.a_row_div) * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t ares = buffer_resource(p.A, a_bytes);
    uint32_t a_off[DMA];
#pragma unroll
    for (int r = 0; r < DMA; ++r) {
        const int row = w * ROWS_PER_WAVE + 4 * r + (L >> 4);
        const int sid = p.sorted_ids[row0 + row];
        const int ch = (L & 15) ^ (row & 15);
        a_off[r] = sid < p.R ? (uint32_t)(sid / p.a_row_div) * (uint32_t)K * 2u + (uint32_t)ch * 16u : kOutOfRange;
    }
    // RAGGED: the stage may reach past K (only the last stage of K can); its chunks past K read zeros, with the
    // whole offset going through the resource's range check
    auto issue_a = [&](int st, uint8_t* slot_base, auto ragged) {
        uint8_t* slot = slot_base + w * ROWS_PER_WAVE * KT * 2;
#pragma unroll
        for (int r = 0; r < DMA; ++r) {
            uint32_t off = a_off[r];
            int soff = st * KT * 2;
            if constexpr (decltype(ragged)::value) {
                const int ch = (L & 15) ^ ((w * ROWS_PER_WAVE + 4 * r + (L >> 4)) & 15);
                off = (st * KT + ch * 8 < K && off != kOutOfRange) ? off + (uint32_t)soff : kOutOfRange;
                soff = 0;
            }
            // the down role reads h that gate_up workgroups of the same launch stored: device-coherent loads
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_void*)(slot + r * 4 * KT * 2), 16, off, soff, 0,
                                                     ROLE == kRoleDown ? kBufferDeviceCoherent : 0);
        }
    };
    auto issue_a_last = [&](int st, uint8_t* slot_base) {  // the last stage of K: ragged or not
        if ((st + 1) * KT > K) issue_a(st, slot_base, std::true_type{});
        else issue_a(st, slot_base, std::false_type{});
    };

    // ---- weight stream: one expert's packed image, per-lane offsets fixed for the whole K loop
    constexpr int SB = sb_bytes(FMT);
    constexpr bool MX = FMT == kFmtMxfp4;
    const uint32_t expert_bytes = (uint32_t)sh.NB * sh.KB * SB;
    const __amdgpu_buffer_rsrc_t wres = buffer_resource(p.packed + (size_t)e * expert_bytes, expert_bytes);
    uint32_t cw_off[NBW], sc_off[NBW];
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
        cw_off[q] = (uint32_t)nb * sh.KB * SB + (uint32_t)L * 16u;
        sc_off[q] = (uint32_t)nb * sh.KB * SB + SB_CODE_BYTES + (uint32_t)j * (MX ? 8u : 16u);
    }
    auto load_w = [&](int st, WStage<NBW>& W) {
        const int kb = st >> 1, h = st & 1;
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            W.cw[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    wres, cw_off[q], kb * SB + h * 1024, kBufferNonTemporal));
            if constexpr (MX) {
                W.sc[q][0] = __builtin_amdgcn_raw_buffer_load_b32(wres, sc_off[q], kb * SB + h * 4, 0);
            } else {
                const auto sv = __builtin_amdgcn_raw_buffer_load_b64(wres, sc_off[q], kb * SB + h * 8, 0);
                W.sc[q][0] = sv[0];
                W.sc[q][1] = sv[1];
            }
        }
    };

    f32x4 acc[MTA][NBW];
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int q = 0; q < NBW; ++q) acc[mt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const MixConsts mixk = mix_consts();
    auto dequant_group = [&](const WStage<NBW>& W, int g, bf16x8* wf) {
        if constexpr (MX) {
#pragma unroll
            for (int q = 0; q < NBW; ++q) wf[q] = mxfp4_dequant8(W.cw[q][g], e8m0_scale(W.sc[q][0], g));
            return;
        }
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            const uint32_t word = W.sc[q][g >> 1];
            const float s = __uint_as_float((g & 1) ? (word & 0xFFFF0000u) : (word << 16));
            wf[q] = dequant8_mix(W.cw[q][g], s, -1032.0f * s, -72.0f * s, mixk);
        }
    };
    // multiply the stage in LDS slot `slot` with the weights W.  A ragged last stage computes its padding groups
    // too: their codes are 8 and scales 0 in the packed image (weight 0) and their activations are zero.
    // Software-pipelined by scale group: while the MFMAs of group g run, the activation fragments of group g+1
    // are read from LDS and its weights dequantised, so neither the LDS latency nor the conversion stalls them.
    auto compute = [&](const uint8_t* slot, const WStage<NBW>& W) {
        bf16x8 af[2][MTA];
        bf16x8 wf[2][NBW];
        auto read_a = [&](int g, bf16x8* out) {
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt)
                out[mt] = *reinterpret_cast<const bf16x8*>(slot + (mt * 16 + j) * (KT * 2) + (((4 * g + c) ^ j) * 16));
        };
        read_a(0, af[0]);
        dequant_group(W, 0, wf[0]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (g < 3) {
                read_a(g + 1, af[(g + 1) & 1]);
                dequant_group(W, g + 1, wf[(g + 1) & 1]);
            }
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
                for (int q = 0; q < NBW; ++q) acc[mt][q] = mfma16(af[g & 1][mt], wf[g & 1][q], acc[mt][q]);
        }
    };
    // one stage: wait for this wavefront's activation loads of stage st, barrier (all pieces landed; the other
    // slot is no longer read), start stage st+1's loads into the other slot and register set, multiply stage st
    // NEXT: 0 = stage st is the last, 1 = stage st+1 is a full stage, 2 = stage st+1 is the last stage of K
    auto stage = [&](int st, const uint8_t* cur, uint8_t* next, const WStage<NBW>& W, WStage<NBW>& Wn, auto next_kind) {
        constexpr int NEXT = decltype(next_kind)::value;
        // The wait counts on the issue order pinned below: a stage's activation loads, then its 2*NBW weight
        // loads, so once at most 2*NBW loads are pending the activation loads of stage st have landed.
        wait_vmcnt<2 * NBW>();
        stage_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NEXT == 1) issue_a(st + 1, next, std::false_type{});
        if constexpr (NEXT == 2) issue_a_last(st + 1, next);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NEXT != 0) load_w(st + 1, Wn);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur, W);
    };
    using none = std::integral_constant<int, 0>;
    using full = std::integral_constant<int, 1>;
    using last = std::integral_constant<int, 2>;

    // Pairs of stages alternate the two slots and the two weight register sets (no copies between them).  The
    // loop's loads are never for the last stage, so it has no branches (a branch around loads would make the
    // compiler assume the worst count of loads in flight and drain them); the last one to three stages are peeled.
    // (the last stage of a slice goes through issue_a_last, which reads a ragged stage only at the end of K)
    WStage<NBW> WA, WB;
    if constexpr (ROLE == kRoleDown) {
        // every gate_up column tile of tile t has stored its rows of h
        if (threadIdx.x == 0) {
            unsigned polls = 0;
            while (__hip_atomic_load(&fs->ready[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < fs->ready_target) {
                __builtin_amdgcn_s_sleep(2);
                if (++polls == kMaxPolls) {
                    __hip_atomic_fetch_add(fs->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
    }
    if (st_end > st_begin) {
        if (st_end - st_begin == 1) issue_a_last(st_begin, slot0);
        else issue_a(st_begin, slot0, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        load_w(st_begin, WA);
        __builtin_amdgcn_sched_barrier(0);
        int st = st_begin;
        for (; st + 3 < st_end; st += 2) {
            stage(st, slot0, slot1, WA, WB, full{});
            stage(st + 1, slot1, slot0, WB, WA, full{});
        }
        if (st + 3 == st_end) {
            stage(st, slot0, slot1, WA, WB, full{});
            stage(st + 1, slot1, slot0, WB, WA, last{});
            stage(st + 2, slot0, slot1, WA, WB, none{});
        } else if (st + 2 == st_end) {
            stage(st, slot0, slot1, WA, WB, last{});
            stage(st + 1, slot1, slot0, WB, WA, none{});
        } else {
            stage(st, slot0, slot1, WA, WB, none{});
        }
    }

    if (KS > 1) {
        prefill_split_epilogue<MTA, NBW, OM, MT>(p, acc, ssid, s_last, nt, t, ks, KS, w, c, j);
        return;
    }

    // ---- epilogue: lane holds rows 4c + r of each 16-row tile, column j of each n-block.  The activation output
    // goes through LDS when the staged tile fits one ring slot and rows are whole 16-byte chunks: each wavefront
    // writes its h values to the staged tile, then the workgroup stores whole rows with 16-byte stores (8 lanes
    // cover a row's 128 bytes), not 2-byte stores four rows at a time.
    constexpr int OC = kWaves * 16 * (NBW / 2);  // activation columns of the tile
    constexpr int RS = OC * 2;                   // bytes of a staged row
    constexpr bool kStageFits = OM == kOutAct && 16 * MTA * RS <= 16 * MT * KT * 2;
    bool staged = false;
    if constexpr (kStageFits) {
        const int NO = sh.N / 2;
        staged = (NO & 7) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
        if (staged) {
            uint8_t* stg = slot0;
            __syncthreads();  // every wavefront has finished reading the ring
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int q = 0; q < NBW / 2; ++q)
                    {
                        // the four row quads of an instruction XOR-swizzled by 32 bytes each: all banks, no conflict
                        const int row = mt * 16 + 4 * c + r, byte = ((w * (NBW / 2) + q) * 16 + j) * 2;
                        const int pch = (byte >> 4) ^ (((row >> 2) & 3) << 1);
                        *reinterpret_cast<uint16_t*>(stg + row * RS + pch * 16 + (byte & 15)) =
                            f32_to_bf16_bits(silu_mul(acc[mt][q][r], acc[mt][q + NBW / 2][r]));
                    }
            __syncthreads();
            constexpr int CPR = OC / 8;  // 16-byte chunks per row
            // gate_up role: h is read by down workgroups of the same launch, so it is stored device-coherently
            // (the fused launch only runs where h is below 2 GiB, so buffer offsets reach every row)
            const __amdgpu_buffer_rsrc_t hres = buffer_resource(p.out, (uint32_t)p.R * (uint32_t)NO * 2u);
            for (int idx = threadIdx.x; idx < BM * CPR; idx += kThreads) {
                const int row = idx / CPR, ch = idx % CPR;
                const int sid = ssid[row], n = nt * OC + ch * 8;
                if (sid < 0 || n >= NO) continue;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * RS + ((ch ^ (((row >> 2) & 3) << 1)) * 16));
                if constexpr (ROLE == kRoleGateUp)
                    __builtin_amdgcn_raw_buffer_store_b128(v, hres, (int)(((uint32_t)sid * (uint32_t)NO + (uint32_t)n) * 2u), 0,
                                                          kBufferDeviceCoherent);
                else
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + (size_t)sid * NO + n) = v;
            }
        }
    }
    // The binary32 output goes through the ring slots too, GP row groups of 16 rows per pass, alternating slots
    // (a pass writes one slot while nothing reads it: every thread finished the previous pass on that slot before
    // it reached the last barrier).  Staged chunks of odd quads of rows are XOR-swizzled by 64 bytes, so the four
    // rows a wavefront writes per instruction fall on two halves of the banks, not one.
    constexpr int COLS = kWaves * NBW * 16;   // binary32 columns of the tile
    constexpr int RB = COLS * 4;              // bytes of a staged binary32 row
    constexpr int GP = (16 * MT * KT * 2) / (16 * RB);
    if constexpr (OM == kOutF32 && GP >= 1 && NBW == 2) {
        staged = (sh.N & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
        if (staged) {
            constexpr int NPASS = (MTA + GP - 1) / GP;
            constexpr int CPR = RB / 16;  // 16-byte chunks per row
            __syncthreads();  // every wavefront has finished reading the ring
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass) {
                uint8_t* stg = (pass & 1) ? slot1 : slot0;
#pragma unroll
                for (int gi = 0; gi < GP; ++gi) {
                    const int mt = pass * GP + gi;
                    if (mt < MTA) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
#pragma unroll
                            for (int q = 0; q < NBW; ++q) {
                                const int row = gi * 16 + 4 * c + r, byte = ((w * NBW + q) * 16 + j) * 4;
                                const int pch = (byte >> 4) ^ (((row >> 2) & 1) << 2);
                                *reinterpret_cast<float*>(stg + row * RB + pch * 16 + (byte & 15)) = acc[mt][q][r];
                            }
                    }
                }
                __syncthreads();
                const int rows = (MTA - pass * GP < GP ? MTA - pass * GP : GP) * 16;
                for (int idx = threadIdx.x; idx < rows * CPR; idx += kThreads) {
                    const int row = idx / CPR, ch = idx % CPR;
                    const int sid = ssid[pass * GP * 16 + row], n = nt * COLS + ch * 4;
                    if (sid < 0 || n >= sh.N) continue;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * RB + ((ch ^ (((row >> 2) & 1) << 2)) * 16));
                    *reinterpret_cast<u32x4*>(static_cast<float*>(p.out) + (size_t)sid * sh.N + n) = v;
                }
            }
        }
    }
    // The BF16 output likewise, in one pass for tiles of up to 144 rows (256-byte rows with two n-blocks per
    // wavefront); the four row quads of an instruction are XOR-swizzled by 32 bytes each, which spreads them over
    // all the banks.
    constexpr int RB2 = COLS * 2;  // bytes of a staged BF16 row
    constexpr int GP2 = (16 * MT * KT * 2) / (16 * RB2);
    if constexpr (OM == kOutBf16 && GP2 >= MTA && NBW == 2) {
        staged = (sh.N & 7) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
        if (staged) {
            constexpr int CPR = RB2 / 16;  // 16-byte chunks per row
            uint8_t* stg = slot0;
            __syncthreads();  // every wavefront has finished reading the ring
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int q = 0; q < NBW; ++q) {
                        const int row = mt * 16 + 4 * c + r, byte = ((w * NBW + q) * 16 + j) * 2;
                        const int pch = (byte >> 4) ^ (((row >> 2) & 3) << 1);
                        *reinterpret_cast<uint16_t*>(stg + row * RB2 + pch * 16 + (byte & 15)) =
                            f32_to_bf16_bits(acc[mt][q][r]);
                    }
            __syncthreads();
            for (int idx = threadIdx.x; idx < BM * CPR; idx += kThreads) {
                const int row = idx / CPR, ch = idx % CPR;
                const int sid = ssid[row], n = nt * COLS + ch * 8;
                if (sid < 0 || n >= sh.N) continue;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * RB2 + ((ch ^ (((row >> 2) & 3) << 1)) * 16));
                *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + (size_t)sid * sh.N + n) = v;
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (staged) break;
            const int sid = ssid[mt * 16 + 4 * c + r];
            if (sid < 0) continue;
            if (OM == kOutAct) {
                const int NO = sh.N / 2;
#pragma unroll
                for (int q = 0; q < NBW / 2; ++q) {
                    const int n = (wave_global * (NBW / 2) + q) * 16 + j;
                    if (n >= NO) continue;
                    uint16_t* dst = static_cast<uint16_t*>(p.out) + (size_t)sid * NO + n;
                    const uint16_t v = f32_to_bf16_bits(silu_mul(acc[mt][q][r], acc[mt][q + NBW / 2][r]));
                    // gate_up role: h is read by down workgroups of the same launch, so it is stored
                    // device-coherently
                    if constexpr (ROLE == kRoleGateUp) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else *dst = v;
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
    if constexpr (ROLE == kRoleGateUp) {
        // this workgroup's rows of h are stored device-coherently: once every wavefront's stores have completed,
        // count the column tile as ready for the tile's down workgroups
        wait_own_stores();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(&fs->ready[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (ROLE == kRoleDown) {
        // the last down workgroup of the tile resets both counters: every other one has passed its wait
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(&fs->done[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (prev == fs->done_target - 1) {
                __hip_atomic_store(&fs->ready[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&fs->done[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Tiles of c route blocks of RB16 * 16 rows: the body for height c * RB16 (c <= MT / RB16)
template <int MT, int NBW, int OM, int RB16, int FMT, int ROLE, int C = 1>
__device__ __forceinline__ void run_tile(int c, const PrefillParams& p, uint8_t* slot0, uint8_t* slot1, int* ssid,
                                         int* s_last, int row0, int e, int nt, int t, const PrefillSync* fs) {
    if constexpr (C * RB16 <= MT) {
        if (c == C) prefill_tile<C * RB16, NBW, OM, FMT, MT, ROLE>(p, slot0, slot1, ssid, s_last, row0, e, nt, t, fs);
        else run_tile<MT, NBW, OM, RB16, FMT, ROLE, C + 1>(c, p, slot0, slot1, ssid, s_last, row0, e, nt, t, fs);
    }
}

// One workgroup of the GEMM: (tile, column tile) pair of position id among the launch's positions (XCD-aware order
// over the valid tiles only; id % 8 is the workgroup's XCD).
template <int MT, int NBW, int OM, int RB16, int FMT, int ROLE>
__device__ __forceinline__ void prefill_body(const PrefillParams& p, int id, uint8_t* slot0, uint8_t* slot1, int* ssid,
                                             int* s_last, const PrefillSync* fs) {
    constexpr bool TILED = RB16 < MT;
    constexpr int BM = 16 * MT;
    int ntl;
    if constexpr (TILED) ntl = __builtin_amdgcn_readfirstlane(*p.tile_count);
    else ntl = p.ntp ? min(__builtin_amdgcn_readfirstlane(*p.ntp) / BM, p.max_blocks) : p.max_blocks;
    const int V = ntl * p.n_tiles;
    const int chunk = max(kChunkMin, (V + kXcds * kChunkRounds - 1) / (kXcds * kChunkRounds));
    const int pos = id / kXcds;
    const int pair = ((pos / chunk) * kXcds + id % kXcds) * chunk + pos % chunk;
    if (pair >= V) return;
    const int t = pair / p.n_tiles, nt = pair % p.n_tiles;
    if constexpr (TILED) {
        const int b0 = p.tiles[2 * t], c = p.tiles[2 * t + 1];
        const int e = p.expert_ids[b0];
        if (e < 0 || e >= p.sh.E) return;
        run_tile<MT, NBW, OM, RB16, FMT, ROLE>(c, p, slot0, slot1, ssid, s_last, b0 * RB16 * 16, e, nt, t, fs);
    } else {
        const int e = p.expert_ids[t];
        if (e < 0 || e >= p.sh.E) return;
        prefill_tile<MT, NBW, OM, FMT, MT, ROLE>(p, slot0, slot1, ssid, s_last, t * BM, e, nt, t, fs);
    }
}

// RB16: route block height in 16-row units; MT (= the tile's largest height) when every route block is a tile.
template <int MT, int NBW, int OM, int RB16, int FMT>
__global__ __launch_bounds__(kThreads, (prefill_waves_per_simd<MT, NBW>())) void gemm_prefill_kernel(PrefillParams p) {
    static_assert(OM != kOutAct || NBW % 2 == 0, "the activation epilogue pairs gate and up n-blocks");
    static_assert(MT % RB16 == 0, "a tile is a whole number of route blocks");
    if constexpr (prefill_waves_per_simd<MT, NBW>() == 1) {
        // at one wavefront per SIMD the accumulators go to AGPRs (VGPRs alone stop at 256); naming an AGPR tells
        // the compiler they may be used
        __asm__ __volatile__("" ::: "a0");
    }
    constexpr int SLOT = 16 * MT * KT * 2;  // bytes of one activation stage
    // the two ring slots are separate arrays, so the compiler can tell the reads of one from the direct loads
    // into the other (with one array it would wait for every direct load before any read of the ring)
    __shared__ __attribute__((aligned(16))) uint8_t slot0[SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[SLOT];
    __shared__ int ssid[16 * MT];
    __shared__ int s_last;
    prefill_body<MT, NBW, OM, RB16, FMT, kRolePlain>(p, (int)blockIdx.x, slot0, slot1, ssid, &s_last, nullptr);
}

// gate_up (SiLU*mul into h) and down (BF16 y) of a fused step in one launch: workgroups [0, ng) are gate_up's,
// the rest down's.  Every gate_up workgroup of an XCD is dispatched before that XCD's first down workgroup and
// waits on nothing, so a down workgroup's wait for its tile always ends.  ng is a multiple of 8, so the XCD of a
// workgroup is the XCD its role's position maps to.
template <int MT, int NBW, int RB16, int FMT>
__global__ __launch_bounds__(kThreads, (prefill_waves_per_simd<MT, NBW>())) void gemm_prefill_fused_kernel(
    PrefillParams gu, PrefillParams dn, PrefillSync fs, int ng) {
    static_assert(NBW % 2 == 0 && MT % RB16 == 0, "prefill tile shape");
    static_assert(prefill_waves_per_simd<MT, NBW>() == 2, "two wavefronts per SIMD");
    constexpr int SLOT = 16 * MT * KT * 2;
    __shared__ __attribute__((aligned(16))) uint8_t slot0[SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[SLOT];
    __shared__ int ssid[16 * MT];
    __shared__ int s_last;
    const int id = (int)blockIdx.x;
    if (id < ng) prefill_body<MT, NBW, kOutAct, RB16, FMT, kRoleGateUp>(gu, id, slot0, slot1, ssid, &s_last, &fs);
    else prefill_body<MT, NBW, kOutBf16, RB16, FMT, kRoleDown>(dn, id - ng, slot0, slot1, ssid, &s_last, &fs);
}

template <int MT, int NBW, int OM, int RB16>
hipError_t launch_t(const GemmArgs& a, int ks, hipStream_t s) {
    constexpr int cols = kWaves * NBW;  // n-blocks of weight columns per workgroup
    const int n_tiles = (a.sh.NB + cols - 1) / cols;
    if (ks > 1 && (a.partials == nullptr || a.counters == nullptr)) return hipErrorInvalidValue;
    PrefillParams p{a.A,          a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids,
                    a.expert_ids, a.ntp,       a.R,  a.max_blocks, n_tiles, a.out, a.tiles, a.tile_count,
                    a.partials,   a.counters};
    // V <= tiles: a tile list of G-block tiles holds at most ceil(max_blocks / G) + min(E, max_blocks) tiles (each
    // expert's run of L blocks is cut into ceil(L / G) <= L / G + 1), plain route blocks are one tile each.  The
    // bound is every route landing on these experts; the grid's workgroups past V exit at once but still cost
    // their dispatch (about 0.3 us per thousand, measured), which matters where only a share of the routes is
    // local.  XCD x takes chunks x, x + 8, ... of c pairs each, so it needs ceil(ceil(V / c) / 8) * c workgroups:
    // at most V/8 + kChunkRounds when c is ceil(V / (8 * kChunkRounds)), and at most V/8 + kChunkMin when c is
    // kChunkMin.  grid.y: the K slices.
    constexpr int G = MT / RB16;
    const unsigned max_tiles = G > 1 ? (unsigned)((a.max_blocks + G - 1) / G + (a.sh.E < a.max_blocks ? a.sh.E : a.max_blocks))
                                     : (unsigned)a.max_blocks;
    const unsigned tiles = max_tiles * (unsigned)n_tiles;
    constexpr unsigned kSlack = kChunkMin > kChunkRounds ? kChunkMin : kChunkRounds;
    const dim3 grid(((tiles + kXcds - 1) / kXcds + kSlack) * kXcds, (unsigned)ks);
    if (a.sh.fmt == kFmtMxfp4)
        hipLaunchKernelGGL((gemm_prefill_kernel<MT, NBW, OM, RB16, kFmtMxfp4>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_prefill_kernel<MT, NBW, OM, RB16, kFmtInt4>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// Workgroups a role needs for its (tile, column tile) pairs (see launch_t).
unsigned prefill_role_workgroups(const GemmArgs& a, int G, int n_tiles) {
    const unsigned max_tiles = G > 1 ? (unsigned)((a.max_blocks + G - 1) / G + (a.sh.E < a.max_blocks ? a.sh.E : a.max_blocks))
                                     : (unsigned)a.max_blocks;
    const unsigned tiles = max_tiles * (unsigned)n_tiles;
    constexpr unsigned kSlack = kChunkMin > kChunkRounds ? kChunkMin : kChunkRounds;
    return ((tiles + kXcds - 1) / kXcds + kSlack) * kXcds;
}

template <int MT, int NBW, int RB16>
hipError_t launch_fused_t(const GemmArgs& a13, const GemmArgs& a2, unsigned* sync, hipStream_t s) {
    constexpr int cols = kWaves * NBW;
    const int nt13 = (a13.sh.NB + cols - 1) / cols, nt2 = (a2.sh.NB + cols - 1) / cols;
    auto params = [](const GemmArgs& a, int n_tiles) {
        return PrefillParams{a.A,      a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids,
                             a.expert_ids, a.ntp,   a.R, a.max_blocks, n_tiles, a.out, a.tiles, a.tile_count,
                             nullptr,  nullptr};
    };
    const PrefillParams gu = params(a13, nt13), dn = params(a2, nt2);
    constexpr int G = MT / RB16;
    const unsigned ng = prefill_role_workgroups(a13, G, nt13), nd = prefill_role_workgroups(a2, G, nt2);
    const PrefillSync fs{sync, sync + a13.max_blocks, sync + 2 * (size_t)a13.max_blocks, (unsigned)nt13,
                         (unsigned)nt2};
    if (a13.sh.fmt == kFmtMxfp4)
        hipLaunchKernelGGL((gemm_prefill_fused_kernel<MT, NBW, RB16, kFmtMxfp4>), dim3(ng + nd), dim3(kThreads), 0, s,
                           gu, dn, fs, (int)ng);
    else
        hipLaunchKernelGGL((gemm_prefill_fused_kernel<MT, NBW, RB16, kFmtInt4>), dim3(ng + nd), dim3(kThreads), 0, s,
                           gu, dn, fs, (int)ng);
    return hipGetLastError();
}

// route blocks of 16*mt rows are tiles; 16- and 32-row route blocks (rb16 = 1, 2) are gathered into tiles of up to
// 16*mt rows
template <int OM>
hipError_t dispatch(const GemmArgs& a, int mt, int nbw, int rb16, int ks, hipStream_t s) {
    if (rb16 < mt) {
        if (a.tiles == nullptr || a.tile_count == nullptr || a.tile_scratch == nullptr) return hipErrorInvalidValue;
        if (rb16 == 2) {
            if (nbw == 2 && mt == 8) return launch_t<8, 2, OM, 2>(a, ks, s);
            if (nbw == 4 && mt == 8) return launch_t<8, 4, OM, 2>(a, ks, s);
            if (nbw == 2 && mt == 4) return launch_t<4, 2, OM, 2>(a, ks, s);
            if (nbw == 4 && mt == 4) return launch_t<4, 4, OM, 2>(a, ks, s);
        }
        if (rb16 == 1 && nbw == 2) {
            if (mt == 9) return launch_t<9, 2, OM, 1>(a, ks, s);
            if (mt == 4) return launch_t<4, 2, OM, 1>(a, ks, s);
        }
        return hipErrorInvalidValue;
    }
    if (rb16 != mt) return hipErrorInvalidValue;
    if (nbw == 4 && mt == 4) return launch_t<4, 4, OM, 4>(a, ks, s);
    if (nbw == 4 && mt == 8) return launch_t<8, 4, OM, 8>(a, ks, s);
    if (nbw == 2 && mt == 8) return launch_t<8, 2, OM, 8>(a, ks, s);
    if (nbw == 2 && mt == 4) return launch_t<4, 2, OM, 4>(a, ks, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(const GemmArgs& a) {
    // the buffer resources address below 2 GiB: one expert's packed weights, and the activation matrix
    return (size_t)a.sh.NB * a.sh.KB * sb_bytes(a.sh.fmt) < (1u << 31) &&
           (size_t)(a.R / a.a_row_div) * a.sh.K * 2 < (1u << 31);
}

int prefill_tile_rows(const w4a16_plan& p) { return p.tile_m ? p.tile_m : p.block_m; }

int prefill_n_tiles(const Shape& sh, const w4a16_plan& p) {
    const int cols = kWaves * p.n_blocks;
    return (sh.NB + cols - 1) / cols;
}

// Tiles a grid can hold: one per route block, or with G route blocks per tile at most ceil(L/G) per expert run
// of L blocks, which sums to at most ceil(max_blocks / G) + (experts owning a block).
size_t prefill_max_tiles(const Shape& sh, const w4a16_plan& p, int max_blocks) {
    const int G = prefill_tile_rows(p) / p.block_m;
    if (G <= 1) return (size_t)max_blocks;
    const int owners = sh.E < max_blocks ? sh.E : max_blocks;
    return (size_t)((max_blocks + G - 1) / G) + (size_t)owners;
}

size_t prefill_partial_floats(const Shape& sh, const w4a16_plan& p, int max_blocks) {
    if (p.kernel != W4A16_KERNEL_PREFILL || p.k_split <= 1) return 0;
    return prefill_max_tiles(sh, p, max_blocks) * prefill_n_tiles(sh, p) * p.k_split * prefill_tile_rows(p) *
           (size_t)(p.n_blocks * 16 * kWaves);
}

size_t prefill_counters(const Shape& sh, const w4a16_plan& p, int max_blocks) {
    if (p.kernel != W4A16_KERNEL_PREFILL || p.k_split <= 1) return 0;
    return prefill_max_tiles(sh, p, max_blocks) * prefill_n_tiles(sh, p);
}

bool prefill_fused_supported(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2) {
    // tiles of 16-row route blocks, two n-blocks per wavefront, K whole, one tile height and one weight format
    const int t13 = prefill_tile_rows(p13), t2 = prefill_tile_rows(p2);
    return p13.kernel == W4A16_KERNEL_PREFILL && p2.kernel == W4A16_KERNEL_PREFILL && p13.block_m == 16 &&
           p2.block_m == 16 && t13 == t2 && (t13 == 144 || t13 == 64) && p13.n_blocks == 2 && p2.n_blocks == 2 &&
           p13.k_split == 1 && p2.k_split == 1 && a13.sh.fmt == a2.sh.fmt && prefill_supported(a13) &&
           prefill_supported(a2);
}

hipError_t launch_gemm_prefill_fused(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2,
                                     const w4a16_plan& p2, unsigned* sync, hipStream_t s) {
    if (a13.max_blocks == 0) return hipSuccess;
    if (!prefill_fused_supported(a13, p13, a2, p2) || a13.out_mode != kOutAct || a2.out_mode != kOutBf16 ||
        sync == nullptr || a13.tiles == nullptr || a13.tile_count == nullptr || a13.tiles != a2.tiles ||
        a13.max_blocks != a2.max_blocks)
        return hipErrorInvalidValue;
    const int mt = prefill_tile_rows(p13) / 16;
    if (!a13.tiles_ready) {
        if (a13.tile_scratch == nullptr) return hipErrorInvalidValue;
        hipError_t err = launch_tile_map(a13.expert_ids, a13.ntp, p13.block_m, a13.max_blocks, mt, a13.tiles,
                                         a13.tile_count, a13.tile_scratch, s);
        if (err != hipSuccess) return err;
    }
    return mt == 9 ? launch_fused_t<9, 2, 1>(a13, a2, sync, s) : launch_fused_t<4, 2, 1>(a13, a2, sync, s);
}

hipError_t launch_gemm_prefill(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    if (a.max_blocks == 0) return hipSuccess;
    const int mt = prefill_tile_rows(p) / 16, rb16 = p.block_m / 16;
    if (rb16 < mt && !a.tiles_ready) {
        hipError_t err = launch_tile_map(a.expert_ids, a.ntp, p.block_m, a.max_blocks, mt / rb16, a.tiles,
                                         a.tile_count, a.tile_scratch, s);
        if (err != hipSuccess) return err;
    }
    switch (a.out_mode) {
        case kOutBf16: return dispatch<kOutBf16>(a, mt, p.n_blocks, rb16, p.k_split, s);
        case kOutF32: return dispatch<kOutF32>(a, mt, p.n_blocks, rb16, p.k_split, s);
        case kOutAct: return dispatch<kOutAct>(a, mt, p.n_blocks, rb16, p.k_split, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
