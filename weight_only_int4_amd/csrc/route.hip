// Routing preparation: stable counting sort of valid routes by expert.
//
// Produces the indexed routing tensors (Chord page, "Two kernel families" and
// Figure 3: activations stay unpadded, padding lives in the index tensors as
// sentinels) and per-expert offsets (nf4 page, "Usage").  Up to 8192 routes
// everything runs in one workgroup, beyond that in three launches; there is
// no host readback, so the routed count never leaves the device (Chord page,
// "vLLM integration").
//
// Order inside an expert is ascending route index.  The routes are cut into
// super-chunks of kRegChunks * (workgroup size) routes, and each wavefront
// takes a contiguous run of kRegChunks * 64 routes of a super-chunk, 64 at a
// time.  A route's rank is (earlier super-chunks) + (earlier wavefronts of
// its super-chunk) + (the wavefront's earlier routes of that expert) + (lower
// lanes of the same 64 with the same expert).  The last term comes from a
// per-expert lane mask that the wavefront's lanes build in LDS with one atomic
// OR each; the third from a per-wavefront running count, so the wavefronts
// rank their runs without a barrier between the groups of 64.
#include <climits>

#include "w4a16_internal.h"

namespace w4a16 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kSmallThreads = 512;  // workgroup of the routing of few routes and experts
constexpr int kRegChunks = 4;       // routes per lane held in registers: a super-chunk is kRegChunks x workgroup

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The ranking pass of scatter_super_chunk, wavefront by wavefront with no barrier: rank[u] is the rank of the
// lane's u-th route among its wavefront's routes of the same expert, and afterwards the wavefront's count of e
// is run[wave][e] + mrow[wave][e].
__device__ __forceinline__ void rank_super_chunk(const int (&e_reg)[kRegChunks], int E, uint64_t* mrow, uint8_t* run,
                                                 int (&rank)[kRegChunks]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t* mw = mrow + (size_t)wave * E;
    uint8_t* rw = run + (size_t)wave * E;
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) {
        const int e = e_reg[u];
        const bool valid = e >= 0 && e < E;
        if (valid) __hip_atomic_fetch_or(&mw[e], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint64_t m = valid ? __hip_atomic_load(&mw[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0ull;
        const int prev = valid ? (int)rw[e] : 0;
        const int r = __popcll(m & lower);
        rank[u] = prev + r;
        if (valid && r == 0) {
            if (u + 1 < kRegChunks) {
                rw[e] = (uint8_t)(prev + __popcll(m));
                __hip_atomic_store(&mw[e], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                __hip_atomic_store(&mw[e], (uint64_t)__popcll(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
}

// Scatter of one super-chunk of routes into sorted_ids.  Lane `lane` of wavefront `wave` holds in e_reg[u] the
// expert of route first + (wave * kRegChunks + u) * 64 + lane (-1 when past the routes or when the caller has no
// route there).  base[e] is the slot of expert e's next route and is advanced by the super-chunk's routes of e.
// mrow: per wavefront and expert a 64-bit word, run: per wavefront and expert a byte, both zero at rest and left
// zero.  Every thread of the workgroup calls this (it has barriers).
//
// Ranking inside a wavefront, for the u-th group of 64: every valid lane sets its bit in mrow[wave][e] with one
// atomic OR and reads the mask back (a wavefront's LDS operations complete in issue order, so the read sees every
// lane's OR); its rank among the wavefront's routes of e so far is run[wave][e] (the earlier groups) plus the set
// bits below its own.  The lowest lane of each expert (rank 0 within the group) then adds the group's count to
// run (at most 64 per group, so it holds at most 192 before the last group) and clears the mask, or in the last
// group leaves the group's count in the mask.  The wavefront's count of e is then run + mask.
template <int NT>
__device__ void scatter_super_chunk(const int (&e_reg)[kRegChunks], int first, int E, uint64_t* mrow, uint8_t* run,
                                   int* base, int32_t* __restrict__ sorted_ids) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint64_t* mw = mrow + (size_t)wave * E;
    int rank[kRegChunks];
    rank_super_chunk(e_reg, E, mrow, run, rank);
    __syncthreads();
    // per expert: the first slot of each wavefront's routes of e (earlier wavefronts first), kept in the mask word
    for (int e = tid; e < E; e += NT) {
        int slot = base[e];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = (int)run[(size_t)w * E + e] + (int)mrow[(size_t)w * E + e];
            mrow[(size_t)w * E + e] = (uint64_t)slot;
            run[(size_t)w * E + e] = 0;
            slot += c;
        }
        base[e] = slot;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) {
        const int e = e_reg[u];
        if (e >= 0 && e < E) sorted_ids[(int)mw[e] + rank[u]] = first + (wave * kRegChunks + u) * 64 + lane;
    }
    __syncthreads();
    for (int x = tid; x < NW * E; x += NT) mrow[x] = 0ull;
    __syncthreads();
}

// Experts of one super-chunk in the layout scatter_super_chunk takes: lane `lane` of wavefront `wave` loads route
// first + (wave * kRegChunks + u) * 64 + lane, for routes below `end` (64 consecutive ids per load).
template <int NT>
__device__ __forceinline__ void load_super_chunk(const int32_t* __restrict__ ids, int first, int end,
                                                 int (&e_reg)[kRegChunks]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < kRegChunks; ++u) {
        const int i = first + (wave * kRegChunks + u) * 64 + lane;
        e_reg[u] = i < end ? ids[i] : -1;
    }
}

// Exclusive scan of one int per thread across the workgroup; returns the
// thread's exclusive prefix and writes the total to *total (all threads).
template <int NT = kThreads>
__device__ int block_exclusive_scan(int v, int* wave_tot, int* total) {
    constexpr int kW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        // the wavefront totals, scanned across the lanes of the first wavefront (no serial chain of LDS accesses)
        const int t = lane < kW ? wave_tot[lane] : 0;
        int run = t;
#pragma unroll
        for (int off = 1; off < kW; off <<= 1) {
            const int o = __shfl_up(run, off, 64);
            if (lane >= off) run += o;
        }
        if (lane < kW) wave_tot[lane] = run - t;
        if (lane == kW - 1) wave_tot[kW] = run;
    }
    __syncthreads();
    const int excl = wave_tot[wave] + incl - v;
    *total = wave_tot[kW];
    __syncthreads();
    return excl;
}

// The tile list of the prefill GEMMs (the same records as tile_map_kernel builds from expert_ids), written by the
// routing itself when the caller asks for it: thread e owns expert e, whose L route blocks start at block b0e, and
// cuts them into ceil(L / group) tiles of as equal a size as possible (the first L % n one block larger).  The
// scan is uniform: every thread of the workgroup calls this.
template <int NT>
__device__ void emit_tiles(const TileOut& to, int L, int b0e, int* wave_tot) {
    const int n = L > 0 ? (L + to.group - 1) / to.group : 0;
    int total;
    const int t0 = block_exclusive_scan<NT>(n, wave_tot, &total);
    if (n > 0) {
        const int base = L / n, rem = L % n;
        for (int i = 0; i < n; ++i) {
            to.tiles[2 * (t0 + i)] = b0e + (i < rem ? i * (base + 1) : rem * (base + 1) + (i - rem) * base);
            to.tiles[2 * (t0 + i) + 1] = i < rem ? base + 1 : base;
        }
    }
    if (threadIdx.x == 0) *to.count = total;
}

// Shared memory layout: wave_cnt[(NT / 64)][E] (64-bit lane masks, then counts) | ints cnt[E] | pad_off[E+1] |
// base[E] | wave_tot[(NT / 64)+1] | bytes run[(NT / 64)][E]
template <int NT>
__global__ __launch_bounds__(NT) void route_prep_kernel(const int32_t* __restrict__ ids, int R, int E, int BM,
                                                              int max_padded, int max_blocks,
                                                              int32_t* __restrict__ sorted_ids,
                                                              int32_t* __restrict__ expert_ids,
                                                              int32_t* __restrict__ ntp_out,
                                                              int32_t* __restrict__ offsets_out,
                                                              int32_t* __restrict__ counts_out, TileOut to) {
    extern __shared__ uint64_t smem64[];
    uint64_t* wave_cnt = smem64;
    int* cnt = reinterpret_cast<int*>(wave_cnt + (NT / 64) * E);
    int* pad_off = cnt + E;
    int* base = pad_off + E + 1;
    int* wave_tot = base + E;
    uint8_t* run = reinterpret_cast<uint8_t*>(wave_tot + (NT / 64) + 1);
    const int tid = threadIdx.x;

    for (int e = tid; e < E; e += NT) cnt[e] = 0;
    for (int x = tid; x < (NT / 64) * E; x += NT) {
        wave_cnt[x] = 0ull;
        run[x] = 0;
    }
    __syncthreads();
    // the ids of the first super-chunk are loaded together and stay in registers for the scatter below, so neither
    // pass waits on a load per group (later super-chunks, past kRegChunks * NT routes, are read again)
    constexpr int kSuper = kRegChunks * NT;
    constexpr int NW = NT / 64;
    int e_reg[kRegChunks];
    load_super_chunk<NT>(ids, 0, R, e_reg);
    // One super-chunk (uniform): the ranking pass runs first and its per-wavefront counts give the totals, so
    // there is no separate counting pass; thread e keeps its expert's wavefront counts in wc.  Otherwise the
    // routes are counted with LDS atomics and every super-chunk is scattered after the scans.
    const bool one = R <= kSuper;
    int rank[kRegChunks];
    int wc[NW];
    int c = 0;
    if (one) {
        rank_super_chunk(e_reg, E, wave_cnt, run, rank);
        __syncthreads();
        if (tid < E) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                wc[w] = (int)run[(size_t)w * E + tid] + (int)wave_cnt[(size_t)w * E + tid];
                c += wc[w];
            }
        }
    } else {
#pragma unroll
        for (int ci = 0; ci < kRegChunks; ++ci)
            if (e_reg[ci] >= 0 && e_reg[ci] < E) atomicAdd(&cnt[e_reg[ci]], 1);
        for (int i = tid + kSuper; i < R; i += NT) {
            const int e = ids[i];
            if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        }
        __syncthreads();
        c = tid < E ? cnt[tid] : 0;
    }

    // scans of counts (unpadded offsets) and padded sizes, E <= NT; one scan of both packed into 16-bit halves
    // when every partial sum stays below 2^15 (uniform; no sum then reaches the sign bit)
    const int padded = tid < E ? ceil_div(c, BM) * BM : 0;
    int tot_c, tot_p, off_c, off_p;
    if (R + E * (BM - 1) < 32768) {
        int tot;
        const int off = block_exclusive_scan<NT>((padded << 16) | c, wave_tot, &tot);
        off_c = off & 0xFFFF;
        off_p = off >> 16;
        tot_c = tot & 0xFFFF;
        tot_p = tot >> 16;
    } else {
        off_c = block_exclusive_scan<NT>(c, wave_tot, &tot_c);
        off_p = block_exclusive_scan<NT>(padded, wave_tot, &tot_p);
    }
    if (one && tid < E) {
        // the first slot of each wavefront's routes of this expert, in the mask word (read by the stores below)
        int slot = off_p;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            wave_cnt[(size_t)w * E + tid] = (uint64_t)slot;
            slot += wc[w];
        }
    }
    if (tid < E) {
        counts_out[tid] = c;
        offsets_out[tid] = off_c;
        pad_off[tid] = off_p;
        base[tid] = off_p;
    }
    if (tid == 0) {
        offsets_out[E] = tot_c;
        pad_off[E] = tot_p;
        *ntp_out = tot_p;
    }
    if (to.tiles) emit_tiles<NT>(to, padded / BM, off_p / BM, wave_tot);
    __syncthreads();

    // the sentinel in every slot the scatter below leaves alone: each expert's padding [off_p + c, off_p + padded)
    // and everything from tot_p on (the scatter writes exactly the slots [off_p, off_p + c) of each expert)
    if (tid < E)
        for (int p = off_p + c; p < off_p + padded; ++p) sorted_ids[p] = R;
    for (int p = tot_p + tid; p < max_padded; p += NT) sorted_ids[p] = R;
    for (int b = tid; b < max_blocks; b += NT) {
        const int p = b * BM;
        int owner = -1;
        if (p < tot_p) {
            int lo = 0, hi = E - 1;  // last e with pad_off[e] <= p
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pad_off[mid] <= p) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        expert_ids[b] = owner;
    }

    if (one) {
        // the slots were written before the barrier that follows the tile list
        const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int u = 0; u < kRegChunks; ++u) {
            const int e = e_reg[u];
            if (e >= 0 && e < E)
                sorted_ids[(int)wave_cnt[(size_t)wave * E + e] + rank[u]] = (wave * kRegChunks + u) * 64 + lane;
        }
        return;
    }
    // super-chunks in route order, each ranked from base (the routes of earlier super-chunks)
    scatter_super_chunk<NT>(e_reg, 0, E, wave_cnt, run, base, sorted_ids);
    for (int first = kSuper; first < R; first += kSuper) {  // uniform
        load_super_chunk<NT>(ids, first, R, e_reg);
        scatter_super_chunk<NT>(e_reg, first, E, wave_cnt, run, base, sorted_ids);
    }
}

// ---- the same routing tensors from several workgroups, for many routes (needs scratch)
//
// Routes are cut into chunks of kChunk (one super-chunk).  (1) Each chunk's workgroup counts its routes per
// expert.  (2) One workgroup turns the counts into per-expert totals, offsets and padded offsets (as above), and
// each chunk's first slot per expert: the expert's padded offset plus the routes of that expert in earlier
// chunks; it also writes the sentinels of the padding slots and expert_ids.  (3) Each chunk's workgroup scatters
// its routes from those bases with the same ranking as above, so the order inside an expert is again ascending
// route index.
constexpr int kChunk = 4 * kThreads;
constexpr int kScanRegChunks = 16;  // chunk counts per expert the scan holds in registers (65536 routes)

__global__ __launch_bounds__(kThreads) void route_count_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                               int32_t* __restrict__ chunk_counts) {
    extern __shared__ int cnt[];
    const int tid = threadIdx.x, c = blockIdx.x;
    const int end = min(R, (c + 1) * kChunk);
    int e_reg[kChunk / kThreads];  // the chunk's ids, loaded together before the counter is cleared
#pragma unroll
    for (int u = 0; u < kChunk / kThreads; ++u) {
        const int i = c * kChunk + u * kThreads + tid;
        e_reg[u] = i < end ? ids[i] : -1;
    }
    for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kChunk / kThreads; ++u)
        if (e_reg[u] >= 0 && e_reg[u] < E) atomicAdd(&cnt[e_reg[u]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) chunk_counts[(size_t)c * E + e] = cnt[e];
}

// Shared memory (ints): pad_off[E+1] | wave_tot[kWaves+1]
__global__ __launch_bounds__(kThreads) void route_scan_kernel(int R, int E, int BM, int max_padded, int max_blocks,
                                                              int nchunks, int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ sorted_ids,
                                                              int32_t* __restrict__ expert_ids,
                                                              int32_t* __restrict__ ntp_out,
                                                              int32_t* __restrict__ offsets_out,
                                                              int32_t* __restrict__ counts_out, TileOut to) {
    extern __shared__ int smem[];
    int* pad_off = smem;
    int* wave_tot = pad_off + E + 1;
    const int tid = threadIdx.x;
    // E <= kThreads: thread e owns expert e.  The first kScanRegChunks chunk counts are loaded together (no load
    // waits behind the previous chunk's store), then replaced by the routes of expert e in earlier chunks.
    int c = 0;
    if (tid < E) {
        int v[kScanRegChunks];
#pragma unroll
        for (int ch = 0; ch < kScanRegChunks; ++ch) v[ch] = ch < nchunks ? chunk_base[(size_t)ch * E + tid] : 0;
#pragma unroll
        for (int ch = 0; ch < kScanRegChunks; ++ch) {
            if (ch < nchunks) chunk_base[(size_t)ch * E + tid] = c;
            c += v[ch];
        }
        for (int ch = kScanRegChunks; ch < nchunks; ++ch) {
            const int x = chunk_base[(size_t)ch * E + tid];
            chunk_base[(size_t)ch * E + tid] = c;
            c += x;
        }
    }
    const int padded = tid < E ? ceil_div(c, BM) * BM : 0;
    int tot_c, tot_p;
    const int off_c = block_exclusive_scan(c, wave_tot, &tot_c);
    const int off_p = block_exclusive_scan(padded, wave_tot, &tot_p);
    if (tid < E) {
        counts_out[tid] = c;
        offsets_out[tid] = off_c;
        pad_off[tid] = off_p;
        for (int ch = 0; ch < nchunks; ++ch) chunk_base[(size_t)ch * E + tid] += off_p;
    }
    if (tid == 0) {
        offsets_out[E] = tot_c;
        pad_off[E] = tot_p;
        *ntp_out = tot_p;
    }
    if (to.tiles) emit_tiles<kThreads>(to, padded / BM, off_p / BM, wave_tot);
    __syncthreads();
    // the sentinel in the slots the scatter kernel leaves alone (as in route_prep_kernel)
    if (tid < E)
        for (int p = off_p + c; p < off_p + padded; ++p) sorted_ids[p] = R;
    for (int p = tot_p + tid; p < max_padded; p += kThreads) sorted_ids[p] = R;
    for (int b = tid; b < max_blocks; b += kThreads) {
        const int p = b * BM;
        int owner = -1;
        if (p < tot_p) {
            int lo = 0, hi = E - 1;  // last e with pad_off[e] <= p
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pad_off[mid] <= p) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        expert_ids[b] = owner;
    }
}

// Shared memory: wave_cnt[kWaves][E] (64-bit lane masks, then first slots) | ints base[E] | bytes run[kWaves][E]
__global__ __launch_bounds__(kThreads) void route_scatter_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                 const int32_t* __restrict__ chunk_base,
                                                                 int32_t* __restrict__ sorted_ids) {
    static_assert(kChunk == kRegChunks * kThreads, "a chunk is one super-chunk");
    extern __shared__ uint64_t smem64[];
    uint64_t* wave_cnt = smem64;
    int* base = reinterpret_cast<int*>(wave_cnt + kWaves * E);
    uint8_t* run = reinterpret_cast<uint8_t*>(base + E);
    const int tid = threadIdx.x, c = blockIdx.x;
    const int end = min(R, (c + 1) * kChunk);
    // the chunk's ids, loaded together up front
    int e_reg[kRegChunks];
    load_super_chunk<kThreads>(ids, c * kChunk, end, e_reg);
    for (int e = tid; e < E; e += kThreads) base[e] = chunk_base[(size_t)c * E + e];
    for (int x = tid; x < kWaves * E; x += kThreads) {
        wave_cnt[x] = 0ull;
        run[x] = 0;
    }
    __syncthreads();
    scatter_super_chunk<kThreads>(e_reg, c * kChunk, E, wave_cnt, run, base, sorted_ids);
}

// Inclusive max-scan of one int per thread across the workgroup.
__device__ int block_inclusive_max(int v, int* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off && o > incl) incl = o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        // exclusive max over the earlier wavefronts' totals, across the lanes of the first wavefront
        const int t = lane < kWaves ? wave_tot[lane] : INT_MIN;
        int run = t;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const int o = __shfl_up(run, off, 64);
            if (lane >= off && o > run) run = o;
        }
        const int prev = __shfl_up(run, 1, 64);
        if (lane < kWaves) wave_tot[lane] = lane == 0 ? INT_MIN : prev;
    }
    __syncthreads();
    const int r = wave_tot[wave] > incl ? wave_tot[wave] : incl;
    __syncthreads();
    return r;
}

// Inclusive min-scan from the right (suffix minimum) of one int per thread across the workgroup.
__device__ int block_suffix_min(int v, int* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(incl, off, 64);
        if (lane + off < 64 && o < incl) incl = o;
    }
    if (lane == 0) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        // exclusive min over the later wavefronts' totals, across the lanes of the first wavefront
        const int t = lane < kWaves ? wave_tot[lane] : INT_MAX;
        int run = t;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const int o = __shfl_down(run, off, 64);
            if (lane + off < kWaves && o < run) run = o;
        }
        const int next = __shfl_down(run, 1, 64);
        if (lane < kWaves) wave_tot[lane] = lane == kWaves - 1 ? INT_MAX : next;
    }
    __syncthreads();
    const int r = wave_tot[wave] < incl ? wave_tot[wave] : incl;
    __syncthreads();
    return r;
}

// Exclusive max-scan of one int per thread across a workgroup of NT threads (INT_MIN for thread 0).
template <int NT>
__device__ int block_exclusive_max(int v, int* wave_tot) {
    constexpr int kW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off && o > incl) incl = o;
    }
    int excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = INT_MIN;
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int t = lane < kW ? wave_tot[lane] : INT_MIN;
        int run = t;
#pragma unroll
        for (int off = 1; off < kW; off <<= 1) {
            const int o = __shfl_up(run, off, 64);
            if (lane >= off && o > run) run = o;
        }
        const int prev = __shfl_up(run, 1, 64);
        if (lane < kW) wave_tot[lane] = lane == 0 ? INT_MIN : prev;
    }
    __syncthreads();
    const int r = wave_tot[wave] > excl ? wave_tot[wave] : excl;
    __syncthreads();
    return r;
}

// Exclusive min-scan from the right of one int per thread across a workgroup of NT threads (INT_MAX for the last
// thread).
template <int NT>
__device__ int block_exclusive_suffix_min(int v, int* wave_tot) {
    constexpr int kW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(incl, off, 64);
        if (lane + off < 64 && o < incl) incl = o;
    }
    int excl = __shfl_down(incl, 1, 64);
    if (lane == 63) excl = INT_MAX;
    if (lane == 0) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int t = lane < kW ? wave_tot[lane] : INT_MAX;
        int run = t;
#pragma unroll
        for (int off = 1; off < kW; off <<= 1) {
            const int o = __shfl_down(run, off, 64);
            if (lane + off < kW && o < run) run = o;
        }
        const int next = __shfl_down(run, 1, 64);
        if (lane < kW) wave_tot[lane] = lane == kW - 1 ? INT_MAX : next;
    }
    __syncthreads();
    const int r = wave_tot[wave] < excl ? wave_tot[wave] : excl;
    __syncthreads();
    return r;
}

// Tiles of consecutive route blocks of one expert, for GEMM kernels whose workgroup covers more rows than a
// route block: routing keeps fine blocks (little padding) while the kernel amortises the weight dequantisation
// over the tile's rows.  A run of L equal expert_ids is cut into n = ceil(L / group) tiles of as equal a size as
// possible (the first L % n take one block more): a kernel whose cost per tile is mostly the dequantisation
// gains nothing from a full tile beside a one-block one.  Run starts come from a max-scan of start flags and run
// ends from a suffix min-scan of end flags, both kept per block in `scratch` (2 * max_blocks ints), so no thread
// walks a run.  tiles[2t] = first block, tiles[2t+1] = blocks; *count = tiles, at most the number of valid
// blocks.  Blocks with a negative expert id get no tile.
__global__ __launch_bounds__(kThreads) void tile_map_kernel(const int32_t* __restrict__ expert_ids,
                                                            const int32_t* __restrict__ ntp, int BM, int max_blocks,
                                                            int group, int32_t* __restrict__ tiles,
                                                            int32_t* __restrict__ count,
                                                            int32_t* __restrict__ scratch) {
    __shared__ int wave_tot[kWaves + 1];
    __shared__ int carry[2];
    const int tid = threadIdx.x;
    int nvalid = ntp ? *ntp / BM : max_blocks;
    if (nvalid > max_blocks) nvalid = max_blocks;
    int32_t* run_first = scratch;
    int32_t* run_last = scratch + max_blocks;
    const int nchunks = (nvalid + kThreads - 1) / kThreads;

    // run starts, first chunk to last (the start of a run open at a chunk's end is carried into the next)
    if (tid == 0) carry[0] = 0;
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
        const int b = ch * kThreads + tid;
        const bool in = b < nvalid;
        const bool start = in && (b == 0 || expert_ids[b - 1] != expert_ids[b]);
        int r0 = block_inclusive_max(start ? b : -1, wave_tot);
        if (r0 < carry[0]) r0 = carry[0];
        if (in) run_first[b] = r0;
        __syncthreads();
        if (tid == kThreads - 1) carry[0] = r0;
        __syncthreads();
    }
    // run ends, last chunk to first
    if (tid == 0) carry[0] = INT_MAX;
    __syncthreads();
    for (int ch = nchunks - 1; ch >= 0; --ch) {
        const int b = ch * kThreads + tid;
        const bool in = b < nvalid;
        const bool end = in && (b == nvalid - 1 || expert_ids[b + 1] != expert_ids[b]);
        int r1 = block_suffix_min(end ? b : INT_MAX, wave_tot);
        if (r1 > carry[0]) r1 = carry[0];
        if (in) run_last[b] = r1;
        __syncthreads();
        if (tid == 0) carry[0] = r1;
        __syncthreads();
    }
    __threadfence_block();
    // tile starts, compacted in block order
    if (tid == 0) carry[1] = 0;
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
        const int b = ch * kThreads + tid;
        bool anchor = false;
        int n = 0;
        if (b < nvalid && expert_ids[b] >= 0) {
            const int r0 = run_first[b], L = run_last[b] - r0 + 1, pos = b - r0;
            const int nt = (L + group - 1) / group, base = L / nt, rem = L % nt;
            const int big = rem * (base + 1);  // blocks in the first rem tiles, of base + 1 blocks each
            if (pos < big) {
                anchor = pos % (base + 1) == 0;
                n = base + 1;
            } else {
                anchor = (pos - big) % base == 0;
                n = base;
            }
        }
        int total;
        const int excl = block_exclusive_scan(anchor ? 1 : 0, wave_tot, &total);
        if (anchor) {
            tiles[2 * (carry[1] + excl)] = b;
            tiles[2 * (carry[1] + excl) + 1] = n;
        }
        __syncthreads();
        if (tid == 0) carry[1] += total;
        __syncthreads();
    }
    if (tid == 0) *count = carry[1];
}

// The same tile list for up to NT * CH route blocks with the blocks in registers: thread t owns blocks
// t*CH .. t*CH + CH - 1, so run starts, run ends and tile positions each take one workgroup scan of a per-thread
// value (the thread's own blocks are scanned in registers), and nothing goes through scratch memory.  The expert
// ids are loaded up to max_blocks, together with num_tokens_padded rather than behind it.
template <int NT, int CH>
__global__ __launch_bounds__(NT) void tile_map_reg_kernel(const int32_t* __restrict__ expert_ids,
                                                          const int32_t* __restrict__ ntp, int BM, int max_blocks,
                                                          int group, int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ count) {
    __shared__ int wave_tot[NT / 64 + 1];
    const int tid = threadIdx.x, b0 = tid * CH;
    // e[j + 1]: expert of block b0 + j, with the neighbours e[0] and e[CH + 1]; INT_MIN outside [0, nvalid)
    int e[CH + 2];
#pragma unroll
    for (int j = 0; j < CH + 2; ++j) {
        const int b = b0 + j - 1;
        e[j] = (b >= 0 && b < max_blocks) ? expert_ids[b] : INT_MIN;
    }
    int nvalid = ntp ? *ntp / BM : max_blocks;
    if (nvalid > max_blocks) nvalid = max_blocks;
#pragma unroll
    for (int j = 0; j < CH + 2; ++j)
        if (b0 + j - 1 >= nvalid) e[j] = INT_MIN;
    // run starts: the last start at or before each block
    int first[CH];
    int m = -1;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int b = b0 + j;
        if (b < nvalid && e[j] != e[j + 1]) m = b;
        first[j] = m;
    }
    const int carry_first = block_exclusive_max<NT>(m, wave_tot);
    // run ends: the first end at or after each block
    int last[CH];
    int mn = INT_MAX;
#pragma unroll
    for (int j = CH - 1; j >= 0; --j) {
        const int b = b0 + j;
        if (b < nvalid && e[j + 2] != e[j + 1]) mn = b;
        last[j] = mn;
    }
    const int carry_last = block_exclusive_suffix_min<NT>(mn, wave_tot);
    // tile anchors in block order
    int nanchor = 0;
    int tsize[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int b = b0 + j;
        tsize[j] = 0;
        if (b < nvalid && e[j + 1] >= 0) {
            const int r0 = first[j] > carry_first ? first[j] : carry_first;
            const int r1 = last[j] < carry_last ? last[j] : carry_last;
            const int L = r1 - r0 + 1, pos = b - r0;
            const int nt = (L + group - 1) / group, base = L / nt, rem = L % nt;
            const int big = rem * (base + 1);  // blocks in the first rem tiles, of base + 1 blocks each
            const bool anchor = pos < big ? pos % (base + 1) == 0 : (pos - big) % base == 0;
            if (anchor) {
                tsize[j] = pos < big ? base + 1 : base;
                ++nanchor;
            }
        }
    }
    int total;
    int at = block_exclusive_scan<NT>(nanchor, wave_tot, &total);
#pragma unroll
    for (int j = 0; j < CH; ++j)
        if (tsize[j] > 0) {
            tiles[2 * at] = b0 + j;
            tiles[2 * at + 1] = tsize[j];
            ++at;
        }
    if (tid == 0) *count = total;
}

// Row ranges -> indexed form: rows [start(e), start(e) + count(e)) of expert e become slots of e's padded
// segment; the sentinel is rows_max.  Offsets form: start(e) = off[e], count(e) = off[e+1] - off[e].  Masked
// form (off == NULL): start(e) = e * max_m, count(e) = masked_m[e] clamped to [0, max_m].
__global__ __launch_bounds__(kThreads) void offsets_to_route_kernel(const int32_t* __restrict__ off,
                                                                    const int32_t* __restrict__ masked_m, int max_m,
                                                                    int E, int rows_max, int BM, int max_padded,
                                                                    int max_blocks, int32_t* __restrict__ sorted_ids,
                                                                    int32_t* __restrict__ expert_ids,
                                                                    int32_t* __restrict__ ntp) {
    extern __shared__ int smem[];
    int* pad_off = smem;                  // E+1
    int* start = pad_off + E + 1;         // E
    int* count = start + E;               // E
    int* wave_tot = count + E;            // kWaves+1
    const int tid = threadIdx.x;
    int c = 0;
    if (tid < E) {
        if (off) {
            c = off[tid + 1] - off[tid];
            start[tid] = off[tid];
        } else {
            c = masked_m[tid] < max_m ? masked_m[tid] : max_m;
            start[tid] = tid * max_m;
        }
        if (c < 0) c = 0;
        count[tid] = c;
    }
    const int padded = ceil_div(c, BM) * BM;
    int tot_p;
    const int off_p = block_exclusive_scan(padded, wave_tot, &tot_p);
    if (tid < E) pad_off[tid] = off_p;
    if (tid == 0) {
        pad_off[E] = tot_p;
        *ntp = tot_p < max_padded ? tot_p : max_padded;
    }
    __syncthreads();
    for (int p = tid; p < max_padded; p += kThreads) {
        int v = rows_max;
        if (p < tot_p) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pad_off[mid] <= p) lo = mid; else hi = mid - 1;
            }
            const int r = p - pad_off[lo];
            const int row = start[lo] + r;
            if (r < count[lo] && row >= 0 && row < rows_max) v = row;
        }
        sorted_ids[p] = v;
    }
    for (int b = tid; b < max_blocks; b += kThreads) {
        const int p = b * BM;
        int owner = -1;
        if (p < tot_p) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pad_off[mid] <= p) lo = mid; else hi = mid - 1;
            }
            owner = lo;
        }
        expert_ids[b] = owner;
    }
}

}  // namespace

hipError_t launch_route_prep(const int32_t* topk_ids, int R, int E, int block_m, int max_padded, int max_blocks,
                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp, int32_t* offsets,
                             int32_t* counts, hipStream_t s, TileOut to) {
    if (E <= kSmallThreads && R <= kRegChunks * kSmallThreads) {
        // few routes and experts: half the workgroup, half the barrier cost and LDS to clear, all routes in one
        // super-chunk; thread e still owns expert e (measured with 128 and 48 experts: 2048 routes 5.3 us against
        // 5.9, 4096 routes 8.2 against 7.3 on 1024 threads)
        constexpr int NT = kSmallThreads, NW = NT / 64;
        const size_t shmem = sizeof(uint64_t) * (size_t)NW * E + sizeof(int) * ((size_t)E + (E + 1) + E + (NW + 1)) +
                             (size_t)NW * E;
        hipLaunchKernelGGL(route_prep_kernel<NT>, dim3(1), dim3(NT), shmem, s, topk_ids, R, E, block_m,
                           max_padded, max_blocks, sorted_ids, expert_ids, ntp, offsets, counts, to);
        return hipGetLastError();
    }
    const size_t shmem = sizeof(uint64_t) * (size_t)kWaves * E + sizeof(int) * ((size_t)E + (E + 1) + E + (kWaves + 1)) +
                         (size_t)kWaves * E;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(route_prep_kernel<kThreads>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (shmem > 65536 && attr != hipSuccess) return attr;
    hipLaunchKernelGGL(route_prep_kernel<kThreads>, dim3(1), dim3(kThreads), shmem, s, topk_ids, R, E, block_m,
                       max_padded, max_blocks, sorted_ids, expert_ids, ntp, offsets, counts, to);
    return hipGetLastError();
}

size_t route_prep_scratch_ints(int R, int E) {
    const int nchunks = (R + kChunk - 1) / kChunk;
    return nchunks > 2 ? (size_t)nchunks * E : 0;
}

hipError_t launch_route_prep_scratch(const int32_t* topk_ids, int R, int E, int block_m, int max_padded,
                                     int max_blocks, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                                     int32_t* offsets, int32_t* counts, int32_t* scratch, hipStream_t s, TileOut to) {
    const int nchunks = (R + kChunk - 1) / kChunk;
    if (nchunks <= 2 || scratch == nullptr)
        return launch_route_prep(topk_ids, R, E, block_m, max_padded, max_blocks, sorted_ids, expert_ids, ntp,
                                 offsets, counts, s, to);
    hipLaunchKernelGGL(route_count_kernel, dim3(nchunks), dim3(kThreads), sizeof(int) * (size_t)E, s, topk_ids, R,
                       E, scratch);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kThreads), sizeof(int) * ((size_t)E + 1 + kWaves + 1), s, R, E,
                       block_m, max_padded, max_blocks, nchunks, scratch, sorted_ids, expert_ids, ntp, offsets,
                       counts, to);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t scatter_lds = sizeof(uint64_t) * (size_t)kWaves * E + sizeof(int) * (size_t)E + (size_t)kWaves * E;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(route_scatter_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (scatter_lds > 65536 && attr != hipSuccess) return attr;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunks), dim3(kThreads), scatter_lds, s, topk_ids, R, E, scratch,
                       sorted_ids);
    return hipGetLastError();
}

hipError_t launch_offsets_to_route(const int32_t* offsets, int E, int rows_max, int block_m, int max_padded,
                                   int max_blocks, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                                   hipStream_t s) {
    const size_t shmem = sizeof(int) * ((size_t)E + 1 + 2 * (size_t)E + kWaves + 1);
    hipLaunchKernelGGL(offsets_to_route_kernel, dim3(1), dim3(kThreads), shmem, s, offsets, nullptr, 0, E, rows_max,
                       block_m, max_padded, max_blocks, sorted_ids, expert_ids, ntp);
    return hipGetLastError();
}

hipError_t launch_masked_to_route(const int32_t* masked_m, int E, int max_m, int block_m, int max_padded,
                                  int max_blocks, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntp,
                                  hipStream_t s) {
    const size_t shmem = sizeof(int) * ((size_t)E + 1 + 2 * (size_t)E + kWaves + 1);
    hipLaunchKernelGGL(offsets_to_route_kernel, dim3(1), dim3(kThreads), shmem, s, nullptr, masked_m, max_m, E,
                       E * max_m, block_m, max_padded, max_blocks, sorted_ids, expert_ids, ntp);
    return hipGetLastError();
}

hipError_t launch_tile_map(const int32_t* expert_ids, const int32_t* ntp, int block_m, int max_blocks, int group,
                           int32_t* tiles, int32_t* count, int32_t* scratch, hipStream_t s) {
    // the register form, 8 route blocks per thread: 256 threads up to 2048 blocks (four wavefronts keep the scans'
    // barriers cheap), 1024 threads up to 8192 (measured: 32 blocks per thread on 256 threads took twice as long,
    // its loads strided 128 bytes apart across the lanes)
    if (max_blocks <= 256 * 8) {
        hipLaunchKernelGGL((tile_map_reg_kernel<256, 8>), dim3(1), dim3(256), 0, s, expert_ids, ntp, block_m,
                           max_blocks, group, tiles, count);
        return hipGetLastError();
    }
    if (max_blocks <= kThreads * 8) {
        hipLaunchKernelGGL((tile_map_reg_kernel<kThreads, 8>), dim3(1), dim3(kThreads), 0, s, expert_ids, ntp,
                           block_m, max_blocks, group, tiles, count);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(kThreads), 0, s, expert_ids, ntp, block_m, max_blocks, group,
                       tiles, count, scratch);
    return hipGetLastError();
}

// Checks caller-provided routing tensors on the device (one workgroup, no host read-back) and writes a status
// bitmask: kRouteBadCount (num_tokens_padded negative, above max_padded or not a multiple of block_m),
// kRouteBadExpert (a block below num_tokens_padded owned by no expert in [0, E)), kRouteBadSlot (a slot below
// num_tokens_padded holding an id outside [0, R]; R is the sentinel), kRouteWrongExpert (with topk_ids: a slot
// holding route i of another expert than its block's).
__global__ __launch_bounds__(1024) void route_validate_kernel(const int32_t* __restrict__ topk, int R, int E,
                                                               int block_m, const int32_t* __restrict__ sorted_ids,
                                                               const int32_t* __restrict__ expert_ids,
                                                               const int32_t* __restrict__ ntp, int max_padded,
                                                               int32_t* __restrict__ status) {
    __shared__ int flags;
    if (threadIdx.x == 0) flags = 0;
    __syncthreads();
    const int n = *ntp;
    int f = 0;
    if (n < 0 || n > max_padded || n % block_m) f |= W4A16_ROUTE_BAD_COUNT;
    const int used = (n < 0 ? 0 : (n > max_padded ? max_padded : n));
    for (int slot = threadIdx.x; slot < used; slot += blockDim.x) {
        const int e = expert_ids[slot / block_m];
        const int sid = sorted_ids[slot];
        if (e < 0 || e >= E) f |= W4A16_ROUTE_BAD_EXPERT;
        if (sid < 0 || sid > R) f |= W4A16_ROUTE_BAD_SLOT;
        else if (topk && sid < R && topk[sid] != e) f |= W4A16_ROUTE_WRONG_EXPERT;
    }
    if (f) atomicOr(&flags, f);
    __syncthreads();
    if (threadIdx.x == 0) *status = flags;
}

hipError_t launch_route_validate(const int32_t* topk_ids, int R, int E, int block_m, const int32_t* sorted_ids,
                                 const int32_t* expert_ids, const int32_t* ntp, int max_padded, int32_t* status,
                                 hipStream_t s) {
    hipLaunchKernelGGL(route_validate_kernel, dim3(1), dim3(1024), 0, s, topk_ids, R, E, block_m, sorted_ids,
                       expert_ids, ntp, max_padded, status);
    return hipGetLastError();
}

}  // namespace w4a16
