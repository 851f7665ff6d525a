// Decode grouped GEMM for one 16-row tile per workgroup (a few routed rows per
// expert: the common decode case), with every operand streamed straight into
// registers.
//
// Design (MI355X-first):
//  * Grid, dequantisation and epilogue as in the LDS-staged decode kernel
//    (gemm_decode.hip): one workgroup per (route block, 64*NBW columns, K
//    slice), the (route block, column tile) pairs laid over the XCDs in
//    contiguous runs so that each XCD's L2 holds only its own route blocks'
//    activation rows (Kimi-K2 share at 256 tokens: 76% of HBM instead of
//    65%), four independent wavefronts with disjoint columns, the raw codes
//    fed to the MFMA as BF16 128 + q with a -136 * sum(x) correction, one FMA
//    per output and group for the scale.
//  * Each wavefront keeps a ring of D register sets; per stage of 128 k a set
//    holds its NBW 1 KiB code halves, 8 bytes of scales per row, and its
//    16-byte activation fragments of the four scale groups (lane (c, j): row j,
//    k-slot c).  D-1 stages are in flight per wavefront, with no LDS and no
//    barrier.  The register file (512 KiB per CU) holds more bytes in flight
//    than an LDS ring can at this tile height, and every ring slot being its
//    own registers lets the compiler wait for exactly the loads a stage uses.
//  * Loads are buffer loads: a scalar resource, a per-lane offset fixed for the
//    whole K loop and the stage offset as a scalar, so issuing a load costs no
//    vector instruction.  Sentinel rows, and groups past K in a ragged last
//    stage, read past the resource's extent and get zeros.
//  * The instruction stream is held to about 12 vector operations per 8
//    weights per lane (7 to build the BF16 operands with AND-OR, 4 scale FMAs,
//    1 scale extraction): at 16 lanes per SIMD that is the work that has to
//    hide under the weight stream.  MFMA results go to VGPRs (compiled with
//    the VGPR MFMA form, see build.py), saving a register move per element.
//  * MXFP4 weights (FMT = kFmtMxfp4) need none of that: the hardware converts
//    two E2M1 codes with their E8M0 scale to exact BF16 per instruction (at
//    the full VALU rate), so each group is 4 conversions per n-block and its
//    MFMAs accumulate directly.  That leaves registers for a ring of three
//    stages instead of two: two stages in flight per wavefront, which the
//    smaller per-stage compute needs to keep the weight stream busy.
#include <type_traits>

#include "decode_common.h"

namespace w4a16 {
using namespace decode;
namespace {


template <int NBW>
struct RegStage {
    u32x4 cw[NBW];  // codes of half h of the superblock, per n-block
    uint32_t sc[NBW][2];  // scales of groups 4h .. 4h+3 of row j, per n-block
    u32x4 xa[4];    // activation fragment of each of the 4 groups
};

constexpr int kXcds = 8;  // XCDs of the chip; workgroup i runs on XCD i % 8

// Exclusive prefix sum of v over the workgroup's threads (uniform call site); *total receives the sum.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wt, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wt[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int x = wt[w];
        if (w < wave) before += x;
        tot += x;
    }
    __syncthreads();  // wt is rewritten by the next call
    *total = tot;
    return before + incl - v;
}

// SR: in-kernel routing (gate_up of the fused decode step).  Instead of reading the routing tensors, every
// workgroup copies the top-k ids to LDS and counts them per expert, lays the experts' 16-row blocks out in expert
// order (the order the counting sort of the routing preparation gives), finds the expert of its own block, issues
// the first stages' weight loads (they depend only on the expert and the column tile), and meanwhile ranks that
// expert's routes by route index to pick its 16 rows, exactly the rows the routing preparation would put there.
// The workgroups of column tile 0 (first K slice) write their block's sorted_ids and expert_ids, and workgroup 0
// num_tokens_padded, for the GEMMs that follow; decode rows are independent of their slot, so the outputs are
// those of the routed path bit for bit.
// The two GEMMs of the fused decode step in one launch (gate_up workgroups first, then down workgroups): a route
// block's down workgroups wait until every gate_up column tile of that block has stored its rows of h, so down's
// work starts while gate_up's last workgroups still run, with no launch boundary between them.
struct FusedSync {
    unsigned* ready;     // [route blocks]: gate_up column tiles whose rows of h are stored; zero at rest
    unsigned* done;      // [route blocks]: down workgroups finished; the last one resets both; zero at rest
    unsigned* timeouts;  // counts down workgroups that stopped waiting (never in a correct launch)
    unsigned ready_target, done_target;
};
constexpr int kRolePlain = 0, kRoleGateUp = 1, kRoleDown = 2;
// bounded wait of a down workgroup: about a second of polling (the gate_up workgroups it waits for were dispatched
// before it and wait on nothing, so this bound is never reached in a correct launch; it only guarantees an end)
constexpr unsigned kMaxPolls = 1u << 24;

// One workgroup of the kernel: route block x column tile x K slice (ks of KS), from the workgroup's index id
// among the n_tiles * route-block positions of its slice.
template <int NBW, int D, int OM, int FMT, bool SR, int ROLE>
__device__ __forceinline__ void decode_reg_body(const DecodeParams& p, const int id, const int n_tiles, const int KS,
                                                const int ks, int* ssid, int* s_last, int* sr_lds,
                                                const FusedSync& fs) {
    constexpr int SB = sb_bytes(FMT);
    constexpr bool MX = FMT == kFmtMxfp4;
    static_assert(OM != kOutAct || NBW % 2 == 0, "the activation epilogue pairs gate and up n-blocks");
    static_assert(D >= 2 && D <= 6, "ring depth");
    // activation loads of the down role read h that other workgroups of this launch stored: device-coherent
    constexpr int kActAux = ROLE == kRoleDown ? kBufferDeviceCoherent : 0;
    int* const cnt = sr_lds;
    int* const boff = sr_lds + W4A16_MAX_EXPERTS;
    int* const wt = sr_lds + 2 * W4A16_MAX_EXPERTS + 2;
    int* const ids = sr_lds + 2 * W4A16_MAX_EXPERTS + 8;  // the top-k ids, R <= kSelfRouteMaxRoutes

    // (route block, column tile) of this workgroup.  XCD-aware: consecutive workgroup ids go to the eight XCDs
    // in turn, so id -> (XCD, position) is remapped to give every XCD a contiguous run of the valid (route
    // block, column tile) pairs, route block major; an XCD then gathers the activation rows of its own route
    // blocks only, and its L2 holds them while its weight streams pass through.
    int valid;
    if constexpr (SR) {
        const int E = p.sh.E, tid = threadIdx.x;
        for (int x = tid; x < E; x += kDecodeThreads) cnt[x] = 0;
        __syncthreads();
        for (int i = tid; i < p.R; i += kDecodeThreads) {
            const int ee = p.topk[i];
            ids[i] = ee;
            if (ee >= 0 && ee < E) atomicAdd(&cnt[ee], 1);
        }
        __syncthreads();
        const int per = (E + kDecodeThreads - 1) / kDecodeThreads;
        int local = 0;
        for (int q = 0; q < per; ++q) {
            const int x = tid * per + q;
            if (x < E) local += (cnt[x] + 15) >> 4;
        }
        int tot;
        int run = wg_exclusive_scan(local, wt, &tot);
        for (int q = 0; q < per; ++q) {
            const int x = tid * per + q;
            if (x < E) {
                boff[x] = run;
                run += (cnt[x] + 15) >> 4;
            }
        }
        if (tid == 0) boff[E] = tot;
        __syncthreads();
        tot = __builtin_amdgcn_readfirstlane(tot);
        if (p.ntp_out && id == 0 && ks == 0 && tid == 0) *p.ntp_out = tot * 16;
        valid = min(tot, p.route_blocks);
    } else {
        valid = p.ntp ? min(__builtin_amdgcn_readfirstlane(*p.ntp) / 16, p.route_blocks) : p.route_blocks;
    }
    const int V = valid * n_tiles;
    // id: the number of positions per slice is a multiple of 8, so id % 8 is the workgroup's XCD
    const int per_xcd = (V + kXcds - 1) / kXcds;
    const int pos = id / kXcds, slot = (id % kXcds) * per_xcd + pos;
    if (pos >= per_xcd || slot >= V) return;
    const int b = slot / n_tiles, nt = slot % n_tiles;
    int e, first = 0;
    if constexpr (SR) {
        // owner: the last expert whose first block is at or before b (empty experts share their successor's)
        int lo = 0, hi = p.sh.E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (boff[mid] <= b) lo = mid;
            else hi = mid - 1;
        }
        e = __builtin_amdgcn_readfirstlane(lo);
        first = 16 * (b - __builtin_amdgcn_readfirstlane(boff[e]));  // rank of the block's first row
    } else {
        e = p.expert_ids[b];
        if (e < 0 || e >= p.sh.E) return;  // unowned block (or ids from a larger expert count)
    }
    const Shape sh = p.sh;
    const int K = sh.K;
    // the wavefront index is uniform: as a scalar it keeps every per-stage offset in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), L = threadIdx.x & 63;
    const int c = L >> 4, j = L & 15;
    const int wave_global = nt * kWaves + w;
    const int nst = (sh.G + 3) / 4;
    const int st_begin = (int)((long)ks * nst / KS), st_end = (int)((long)(ks + 1) * nst / KS);

    if (!SR && threadIdx.x < 16) {
        const int sid = p.sorted_ids[b * 16 + threadIdx.x];
        ssid[threadIdx.x] = sid < p.R ? sid : -1;
    }

    // Buffer loads: a scalar resource, a per-lane offset fixed for the whole K loop, and the stage's offset as a
    // scalar, so a load costs no vector arithmetic.  Offsets at or past a resource's extent read zeros.
    const uint32_t expert_bytes = (uint32_t)sh.NB * sh.KB * SB;
    const __amdgpu_buffer_rsrc_t wres = buffer_resource(p.packed + (size_t)e * expert_bytes, expert_bytes);
    uint32_t cw_off[NBW], sc_off[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
        int o;
        const uint32_t nb = (uint32_t)slot_nblock<NBW, OM>(sh, wave_global, q, &o);
        cw_off[q] = nb * sh.KB * SB + (uint32_t)L * 16u;
        sc_off[q] = nb * sh.KB * SB + SB_CODE_BYTES + (uint32_t)j * (MX ? 8u : 16u);
    }
    // weight half of a stage's loads (the other half, the activations, needs the block's rows)
    auto load_w = [&](int st, RegStage<NBW>& S) {
        const int kb = st >> 1, h = st & 1;
        const int soff_code = kb * SB + h * 1024, soff_scale = kb * SB + h * (MX ? 4 : 8);
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
            S.cw[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, cw_off[q], soff_code,
                                                                                      kBufferNonTemporal));
            if constexpr (MX) {
                S.sc[q][0] = __builtin_amdgcn_raw_buffer_load_b32(wres, sc_off[q], soff_scale, 0);
            } else {
                const auto sv = __builtin_amdgcn_raw_buffer_load_b64(wres, sc_off[q], soff_scale, 0);
                S.sc[q][0] = sv[0];
                S.sc[q][1] = sv[1];
            }
        }
    };
    RegStage<NBW> ring[D];
    if constexpr (SR) {
        // the first stages' weights depend only on the expert and the column tile: they are in flight while the
        // workgroup ranks the expert's routes to find its rows
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (st_begin + d < st_end) load_w(st_begin + d, ring[d]);
        if (threadIdx.x < 16) ssid[threadIdx.x] = -1;
        __syncthreads();
        int carry = 0;
        for (int ch = 0; ch < p.R; ch += kDecodeThreads) {
            const int i = ch + threadIdx.x;
            const bool m = i < p.R && ids[i] == e;
            int n;
            const int r = carry + wg_exclusive_scan(m ? 1 : 0, wt, &n);
            if (m && r >= first && r < first + 16) ssid[r - first] = i;
            carry += __builtin_amdgcn_readfirstlane(n);
            if (carry >= first + 16) break;  // uniform: every later route of e ranks past this block
        }
        __syncthreads();
        if (p.sorted_out && nt == 0 && ks == 0) {
            if (threadIdx.x < 16) p.sorted_out[b * 16 + threadIdx.x] = ssid[threadIdx.x] >= 0 ? ssid[threadIdx.x] : p.R;
            if (threadIdx.x == 0) p.eids_out[b] = e;
        }
    }
    if constexpr (ROLE == kRoleDown) {
        // every gate_up column tile of route block b has stored its rows of h
        if (threadIdx.x == 0) {
            unsigned polls = 0;
            while (__hip_atomic_load(&fs.ready[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < fs.ready_target) {
                __builtin_amdgcn_s_sleep(2);
                if (++polls == kMaxPolls) {
                    __hip_atomic_fetch_add(fs.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
    }
    // activations: lane (c, j) reads row j of the tile at k-slot c; sentinel rows read past the end (zeros)
    const uint32_t a_bytes = (uint32_t)(p.R / p.a_row_div) * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t xres = buffer_resource(p.A, a_bytes);
    const int sid_j = SR ? (ssid[j] >= 0 ? ssid[j] : p.R) : p.sorted_ids[b * 16 + j];
    const uint32_t x_off = sid_j < p.R ? (uint32_t)(sid_j / p.a_row_div) * (uint32_t)K * 2u + (uint32_t)c * 16u
                                       : kOutOfRange;

    // RAGGED: the stage may reach past K (only the last stage of K can); its groups past K are skipped by
    // reading zeros (the test is uniform per group since K is a multiple of 32)
    auto load_a = [&](int st, RegStage<NBW>& S, auto ragged) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t off = x_off + (uint32_t)g * 64u;
            int soff = st * KT * 2;
            if constexpr (decltype(ragged)::value) {
                if (st * KT + g * 32 >= K) off = kOutOfRange;
            }
            S.xa[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, soff, kActAux));
        }
    };
    auto load = [&](int st, RegStage<NBW>& S, auto ragged) {
        load_w(st, S);
        load_a(st, S, ragged);
    };
    const std::false_type full{};
    const std::true_type ragged{};

    f32x4 acc[1][NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) acc[0][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 m136 = minus136();

    const uint32_t kMask = opaque_vgpr(0x000F000Fu), kBias = opaque_vgpr(0x43004300u);
    auto compute = [&](const RegStage<NBW>& S) {
        if constexpr (MX) {
            // exact BF16 weights from the hardware conversion, accumulated directly
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const bf16x8 xf = __builtin_bit_cast(bf16x8, S.xa[g]);
#pragma unroll
                for (int q = 0; q < NBW; ++q)
                    acc[0][q] = mfma16(xf, mxfp4_dequant8(S.cw[q][g], e8m0_scale(S.sc[q][0], g)), acc[0][q]);
            }
            return;
        }
        // a ragged last stage computes its padding groups too: their codes are 8 and scales 0 in the packed
        // image and their activations are zero, so they add exactly zero
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const bf16x8 xf = __builtin_bit_cast(bf16x8, S.xa[g]);
            const f32x4 xc = mfma16(xf, m136, zero);
            // all MFMAs of the group first (distinct results), then the scale FMAs: the FMAs of one n-block then
            // never wait on the MFMA that produced them while the others are still to be issued
            f32x4 d[NBW];
#pragma unroll
            for (int q = 0; q < NBW; ++q) d[q] = mfma16(xf, biased_codes_vop3(S.cw[q][g], kMask, kBias), xc);
            __builtin_amdgcn_sched_group_barrier(0x008, NBW + 1, 0);  // the group's MFMAs ...
            __builtin_amdgcn_sched_group_barrier(0x002, 1000, 0);     // ... before its VALU work
#pragma unroll
            for (int q = 0; q < NBW; ++q) {
                const uint32_t word = S.sc[q][g >> 1];
                const float sc = __uint_as_float((g & 1) ? (word & 0xFFFF0000u) : (word << 16));
                acc[0][q] += sc * d[q];
            }
        }
    };

    // The ring slot of stage st is (st - st_begin) % D; unrolling by D keeps every slot index static.  The steady
    // state (every stage issues the load D-1 stages ahead, none of them ragged) has no branches; the last stages
    // drain with guarded issues.
    const int full_end = min(st_end, K / KT);  // stages below this one lie entirely inside K
    int st = st_begin;
    if (full_end - st_begin >= 2 * D - 1) {
        // the prologue issues its stages in order too, so that at the loop head every slot's loads are as old
        // on entry as on the back edge (else the compiler's wait counts take the younger, stricter view)
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (SR) load_a(st_begin + d, ring[d], full);
            else load(st_begin + d, ring[d], full);
        }
        __builtin_amdgcn_sched_barrier(0);
        for (; st + 2 * D - 2 < full_end; st += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                // keep the issue order: the loads of stage st+d+D-1 go out before stage st+d is computed (the
                // scheduler would otherwise gather all loads of the unrolled body in one place)
                __builtin_amdgcn_sched_barrier(0);
                load(st + d + D - 1, ring[(d + D - 1) % D], full);
                __builtin_amdgcn_sched_barrier(0);
                compute(ring[d]);
            }
        }
    } else {
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (st_begin + d < st_end) {
                if constexpr (SR) load_a(st_begin + d, ring[d], ragged);
                else load(st_begin + d, ring[d], ragged);
            }
    }
    // drain: at most 2D-1 stages are left; their loads for stages past st_begin + D - 2 are issued here
#pragma unroll
    for (int d = 0; d < 2 * D - 1; ++d) {
        const int sd = st + d;
        if (sd < st_end) {
            __builtin_amdgcn_sched_barrier(0);
            if (sd + D - 1 < st_end) load(sd + D - 1, ring[(d + D - 1) % D], ragged);
            __builtin_amdgcn_sched_barrier(0);
            compute(ring[d % D]);
        }
    }

    __syncthreads();  // ssid is complete
    const bool wrote = decode_epilogue<1, NBW, OM, ROLE == kRoleGateUp>(p, acc, ssid, s_last, b, nt, n_tiles, KS, ks,
                                                                        wave_global, w, c, j);
    if constexpr (ROLE == kRoleGateUp) {
        // this workgroup's rows of h are stored device-coherently: once every wavefront's stores have completed,
        // count the column tile as ready for the block's down workgroups
        if (wrote) {
            wait_own_stores();
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_fetch_add(&fs.ready[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if constexpr (ROLE == kRoleDown) {
        // the last down workgroup of the block resets both counters: every other one has passed its wait
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(&fs.done[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (prev == fs.done_target - 1) {
                __hip_atomic_store(&fs.ready[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&fs.done[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <int NBW, int D, int OM, int FMT, bool SR = false>
__global__ __launch_bounds__(kDecodeThreads, 1) void gemm_decode_reg_kernel(DecodeParams p) {
    __shared__ int ssid[16];
    __shared__ int s_last;
    // SR: per-expert counts [E], first block of each expert [E + 1], wavefront totals of the scans
    __shared__ int sr_lds[SR ? kSelfRouteLdsInts : 1];
    // gridDim.x * gridDim.y is a multiple of 8
    decode_reg_body<NBW, D, OM, FMT, SR, kRolePlain>(p, blockIdx.x + gridDim.x * blockIdx.y, gridDim.y, gridDim.z,
                                                     blockIdx.z, ssid, &s_last, sr_lds, FusedSync{});
}

// gate_up (SiLU*mul into h) and down (BF16 y) of one decode step in one launch; both route their rows in-kernel.
// Workgroups [0, ng) are gate_up's (pos_gu positions per K slice), the rest down's.
template <int NBW1, int NBW2, int D, int FMT>
__global__ __launch_bounds__(kDecodeThreads, 1) void gemm_decode_fused_kernel(DecodeParams gu, DecodeParams dn,
                                                                              FusedSync fs, int ng, int pos_gu,
                                                                              int nt_gu, int ks_gu, int pos_dn,
                                                                              int nt_dn, int ks_dn) {
    __shared__ int ssid[16];
    __shared__ int s_last;
    __shared__ int sr_lds[kSelfRouteLdsInts];
    const int x = blockIdx.x;
    if (x < ng)
        decode_reg_body<NBW1, D, kOutAct, FMT, true, kRoleGateUp>(gu, x % pos_gu, nt_gu, ks_gu, x / pos_gu, ssid, &s_last,
                                                                  sr_lds, fs);
    else
        decode_reg_body<NBW2, D, kOutBf16, FMT, true, kRoleDown>(dn, (x - ng) % pos_dn, nt_dn, ks_dn, (x - ng) / pos_dn,
                                                                ssid, &s_last, sr_lds, fs);
}

// ring depths: two stages of INT4 weights (three wavefronts per SIMD fit), three of MXFP4 (its conversion leaves the
// registers for a third stage at the same occupancy)
constexpr int kRingDepth = 2;
constexpr int kRingDepthMx = 3;

template <int NBW, int OM>
hipError_t launch_reg(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    DecodeParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                   a.out, a.partials, a.counters};
    p.ntp = a.ntp;
    p.route_blocks = a.max_blocks;
    // grid.x a multiple of the XCD count, so that the remap above is onto the valid pairs
    const unsigned gx = (unsigned)(a.max_blocks + kXcds - 1) / kXcds * kXcds;
    const dim3 grid(gx, decode_n_tiles(a.sh, pl), pl.k_split);
    constexpr int D = kRingDepth, DMX = kRingDepthMx;
    if constexpr (OM == kOutAct) {
        if (a.self_route_ids) {
            // the routing stages the ids and per-expert tables in LDS
            if (a.sh.E > W4A16_MAX_EXPERTS || a.R > kSelfRouteMaxRoutes || a.ntp == nullptr) return hipErrorInvalidValue;
            p.topk = a.self_route_ids;
            p.sorted_out = const_cast<int32_t*>(a.sorted_ids);
            p.eids_out = const_cast<int32_t*>(a.expert_ids);
            p.ntp_out = const_cast<int32_t*>(a.ntp);
            if (a.sh.fmt == kFmtMxfp4)
                hipLaunchKernelGGL((gemm_decode_reg_kernel<NBW, DMX, OM, kFmtMxfp4, true>), grid, dim3(kDecodeThreads),
                                   0, s, p);
            else
                hipLaunchKernelGGL((gemm_decode_reg_kernel<NBW, D, OM, kFmtInt4, true>), grid, dim3(kDecodeThreads), 0,
                                   s, p);
            return hipGetLastError();
        }
    }
    if (a.self_route_ids) return hipErrorInvalidValue;  // in-kernel routing is for the gate_up GEMM only
    if (a.sh.fmt == kFmtMxfp4)
        hipLaunchKernelGGL((gemm_decode_reg_kernel<NBW, DMX, OM, kFmtMxfp4>), grid, dim3(kDecodeThreads), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_decode_reg_kernel<NBW, D, OM, kFmtInt4>), grid, dim3(kDecodeThreads), 0, s, p);
    return hipGetLastError();
}

template <int OM>
hipError_t dispatch_reg(const GemmArgs& a, const w4a16_plan& pl, hipStream_t s) {
    switch (pl.n_blocks) {
        case 1:
            if constexpr (OM == kOutAct) return hipErrorInvalidValue;  // gate and up need a slot each
            else return launch_reg<1, OM>(a, pl, s);
        case 2: return launch_reg<2, OM>(a, pl, s);
        case 4: return launch_reg<4, OM>(a, pl, s);
        default: return hipErrorInvalidValue;
    }
}

template <int NBW1, int NBW2, int FMT>
hipError_t launch_fused_t(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2,
                          unsigned* sync, hipStream_t s) {
    constexpr int D = FMT == kFmtMxfp4 ? kRingDepthMx : kRingDepth;
    auto params = [](const GemmArgs& a) {
        DecodeParams p{a.A, a.a_row_div, static_cast<const uint8_t*>(a.packed), a.sh, a.sorted_ids, a.expert_ids, a.R,
                       a.out, a.partials, a.counters};
        p.route_blocks = a.max_blocks;
        p.topk = a.self_route_ids;  // both GEMMs route their rows in-kernel; nothing writes the routing tensors
        return p;
    };
    const int gx = (a13.max_blocks + kXcds - 1) / kXcds * kXcds;
    const int nt_gu = decode_n_tiles(a13.sh, p13), nt_dn = decode_n_tiles(a2.sh, p2);
    const int pos_gu = gx * nt_gu, pos_dn = gx * nt_dn;
    const int ng = pos_gu * p13.k_split;
    FusedSync fs{sync, sync + a13.max_blocks, sync + 2 * a13.max_blocks, (unsigned)nt_gu, (unsigned)(nt_dn * p2.k_split)};
    const unsigned grid = (unsigned)(ng + pos_dn * p2.k_split);
    hipLaunchKernelGGL((gemm_decode_fused_kernel<NBW1, NBW2, D, FMT>), dim3(grid), dim3(kDecodeThreads), 0, s,
                       params(a13), params(a2), fs, ng, pos_gu, nt_gu, p13.k_split, pos_dn, nt_dn, p2.k_split);
    return hipGetLastError();
}

template <int NBW1, int FMT>
hipError_t launch_fused_n2(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2,
                           unsigned* sync, hipStream_t s) {
    switch (p2.n_blocks) {
        case 2: return launch_fused_t<NBW1, 2, FMT>(a13, p13, a2, p2, sync, s);
        case 4: return launch_fused_t<NBW1, 4, FMT>(a13, p13, a2, p2, sync, s);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT>
hipError_t launch_fused_fmt(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2,
                            unsigned* sync, hipStream_t s) {
    switch (p13.n_blocks) {
        case 2: return launch_fused_n2<2, FMT>(a13, p13, a2, p2, sync, s);
        case 4: return launch_fused_n2<4, FMT>(a13, p13, a2, p2, sync, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_fused_supported(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2, const w4a16_plan& p2) {
    return p13.kernel == W4A16_KERNEL_DECODE && p2.kernel == W4A16_KERNEL_DECODE && decode_reg_supported(a13, p13) &&
           decode_reg_supported(a2, p2) && a13.sh.fmt == a2.sh.fmt && a13.max_blocks == a2.max_blocks &&
           (p13.n_blocks == 2 || p13.n_blocks == 4) && (p2.n_blocks == 2 || p2.n_blocks == 4) &&
           a13.sh.E <= W4A16_MAX_EXPERTS;
}

hipError_t launch_gemm_decode_fused(const GemmArgs& a13, const w4a16_plan& p13, const GemmArgs& a2,
                                    const w4a16_plan& p2, unsigned* sync, hipStream_t s) {
    if (a13.max_blocks == 0) return hipSuccess;
    if (!decode_fused_supported(a13, p13, a2, p2) || a13.self_route_ids == nullptr || a2.self_route_ids == nullptr ||
        a13.out_mode != kOutAct || a2.out_mode != kOutBf16 || sync == nullptr || a13.R > kSelfRouteMaxRoutes ||
        a2.R > kSelfRouteMaxRoutes || a13.sh.E > W4A16_MAX_EXPERTS)
        return hipErrorInvalidValue;
    if ((p13.k_split > 1 && (a13.partials == nullptr || a13.counters == nullptr)) ||
        (p2.k_split > 1 && (a2.partials == nullptr || a2.counters == nullptr)))
        return hipErrorInvalidValue;
    return a13.sh.fmt == kFmtMxfp4 ? launch_fused_fmt<kFmtMxfp4>(a13, p13, a2, p2, sync, s)
                                   : launch_fused_fmt<kFmtInt4>(a13, p13, a2, p2, sync, s);
}

bool decode_reg_supported(const GemmArgs& a, const w4a16_plan& p) {
    // one 16-row tile; the buffer resources address below 2 GiB (one expert's packed weights, the activations)
    return p.block_m == 16 &&
           (size_t)a.sh.NB * a.sh.KB * sb_bytes(a.sh.fmt) < (1u << 31) &&
           (size_t)(a.R / a.a_row_div) * a.sh.K * 2 < (1u << 31);
}

hipError_t launch_gemm_decode_reg(const GemmArgs& a, const w4a16_plan& p, hipStream_t s) {
    if (a.max_blocks == 0) return hipSuccess;
    switch (a.out_mode) {
        case kOutBf16: return dispatch_reg<kOutBf16>(a, p, s);
        case kOutF32: return dispatch_reg<kOutF32>(a, p, s);
        case kOutAct: return dispatch_reg<kOutAct>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
