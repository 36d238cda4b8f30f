// Count-first token dispatch (afdEP count-first validation record: count the
// routes per expert first, then compute the prefix sums, then stream every
// row to its known offset in an expert-contiguous buffer of capacity C rows
// per expert).
//
// Kernel 1, count_rank: blocks of 2048 routes (4 waves x 8 routes per lane,
// each wave a contiguous run).  For every 64-route step a wave finds the
// lanes holding the same expert by ballots over the bits of the expert id;
// a lane's stable rank is its wave's running LDS count for that expert plus
// the number of lower lanes in its group, and the group's lowest lane adds
// the group size.  Per-wave counts are then prefix-summed over the block's
// waves (giving the rank of a route among the block's routes of its expert)
// and the block totals are published (write-through stores).  The last
// block to arrive (atomic ticket) turns the per-block totals into per-block
// bases, writes the raw counts, the exclusive scan of min(count, C) and the
// m-tile table of the grouped GEMM, and resets the ticket.  A launch of one
// block (at most 2048 routes) keeps its totals in registers and takes no
// ticket.
//
// Kernel 2, scatter: one block per token.  Each route's final rank is
// base[block][e] + its in-block rank; a rank below C places the route at row
// offsets[e] + rank.  The token's row is read once and stored to each of its
// kept rows with 16-byte vector stores.  When no row copy is asked for, a
// metadata-only variant takes one thread per route; when the per-block
// totals are few (blocks x experts <= kLocalScanMax), that variant's blocks
// each scan the totals themselves and the count blocks hand nothing over.
//
// Batches of at most 4096 routes skip the hand-off altogether: one
// 1024-thread workgroup counts, ranks, scans and places every route
// (count_place), and copy_rows then copies the rows when a copy is wanted.
// Batches of at most 64 tokens on the decode path are routed and dispatched
// by one workgroup (small_dispatch).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "route_wave.h"

namespace rde {
namespace {

constexpr int kScanThreads = 256;

// Inclusive prefix sum over the 64 lanes of a wavefront: a Kogge-Stone scan
// inside each row of 16 lanes by DPP row shifts (lanes shifted in from
// outside the row read 0), then the totals of the lower rows.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane) {
    x += (int32_t)__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (int32_t)__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (int32_t)__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (int32_t)__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    const int32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
                  r2 = __builtin_amdgcn_readlane(x, 47);
    if (lane >= 16) x += r0;
    if (lane >= 32) x += r1;
    if (lane >= 48) x += r2;
    return x;
}

// Block-wide exclusive scan of up to kScanThreads * per-thread values held in
// LDS array `v` (n entries, in place); returns the total.  Two arrays at once.
// Called by all kScanThreads threads of the block.
__device__ void block_scan2(int32_t* a, int32_t* b, int n, int32_t* tot_a, int32_t* tot_b) {
    __shared__ int32_t sa[kScanThreads], sb[kScanThreads];
    const int tid = threadIdx.x;
    if (n <= kScanThreads) {
        // one value per thread: wavefront scans, then the wavefront totals
        constexpr int NWV = kScanThreads / kWave;
        const int lane = tid & (kWave - 1), wv = tid / kWave;
        const int32_t va = tid < n ? a[tid] : 0, vb = tid < n ? b[tid] : 0;
        const int32_t ia = wave_incl_scan(va, lane), ib = wave_incl_scan(vb, lane);
        if (lane == kWave - 1) {
            sa[wv] = ia;
            sb[wv] = ib;
        }
        __syncthreads();
        int32_t pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            if (w < wv) {
                pa += sa[w];
                pb += sb[w];
            }
            ta += sa[w];
            tb += sb[w];
        }
        if (tid < n) {
            a[tid] = pa + ia - va;
            b[tid] = pb + ib - vb;
        }
        if (tid == 0) {
            *tot_a = ta;
            *tot_b = tb;
        }
        __syncthreads();
        return;
    }
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int lo = tid * per, hi = min(n, lo + per);
    int32_t ra = 0, rb = 0;
    for (int i = lo; i < hi; ++i) {
        ra += a[i];
        rb += b[i];
    }
    sa[tid] = ra;
    sb[tid] = rb;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int32_t xa = tid >= off ? sa[tid - off] : 0;
        int32_t xb = tid >= off ? sb[tid - off] : 0;
        __syncthreads();
        sa[tid] += xa;
        sb[tid] += xb;
        __syncthreads();
    }
    int32_t ea = sa[tid] - ra, eb = sb[tid] - rb;  // exclusive prefix of this thread's run
    for (int i = lo; i < hi; ++i) {
        int32_t ta = a[i], tb = b[i];
        a[i] = ea;
        b[i] = eb;
        ea += ta;
        eb += tb;
    }
    if (tid == kScanThreads - 1) {
        *tot_a = sa[tid];
        *tot_b = sb[tid];
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void count_rank_kernel(
    const int32_t* __restrict__ ids, int64_t Q, int k, int E, int ebits, int C, int bm,
    int32_t* __restrict__ rexp, int32_t* __restrict__ lrank, int32_t* __restrict__ partial,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ mt_off,
    int32_t* __restrict__ ctrl, int32_t* __restrict__ route_dst, int32_t* __restrict__ row_src,
    int64_t r_max, int delay, int local_scan) {
    extern __shared__ int32_t lds[];  // [kCountWaves][E] during counting; [2][E] in the scan
    __shared__ int s_last;
    __shared__ int32_t s_tot[2];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    for (int i = tid; i < kCountWaves * E; i += blockDim.x) lds[i] = 0;
    __syncthreads();

    int32_t* hist = lds + wv * E;
    const int64_t q0 = (int64_t)blockIdx.x * kCountBlock + (int64_t)wv * (kWave * kCountPerLane);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int rank_w[kCountPerLane], ex[kCountPerLane];
    int n_bad = 0;
    // slot of a route in its token (q mod k) with no division per step: the
    // lane's offset mod k once, and the step base's slot advanced by 64 mod k
    const int lmk = lane % k, s64 = kWave % k;
    int jb = (int)(q0 % k);
    // all of this lane's ids first: one memory latency instead of one per step
#pragma unroll
    for (int it = 0; it < kCountPerLane; ++it) {
        const int64_t q = q0 + it * kWave + lane;
        ex[it] = q < Q ? ids[q] : -1;
    }
#pragma unroll
    for (int it = 0; it < kCountPerLane; ++it) {
        const int64_t q = q0 + it * kWave + lane;
        const bool inq = q < Q;
        int e = ex[it];
        const bool inrange = inq && e >= 0 && e < E;
        // lanes of this 64-route step holding the same (in-range) expert
        uint64_t peers = __ballot(inrange);
        for (int b = 0; b < ebits; ++b) {
            const bool bit = inrange && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        // duplicate: an earlier slot of the same token holds the same expert.
        // The token's slots are consecutive routes, so those in this step are
        // the lanes just below; slots before the step (k not dividing the
        // step) are read back from memory.
        bool dup = false;
        if (inrange) {
            int j = jb + lmk;               // q mod k: the route's slot in its token
            if (j >= k) j -= k;
            const int first = lane - j;   // lane of the token's slot 0 (may be < 0)
            dup = (peers & lt & ~((first > 0) ? (~0ull >> (64 - first)) : 0ull)) != 0;
            for (int jj = 0; !dup && jj < -first; ++jj) dup = ids[q - j + jj] == e;
        }
        jb += s64;
        if (jb >= k) jb -= k;
        if (inq && (!inrange || dup)) {
            e = -2;
            ++n_bad;
        }
        if (inq) rexp[q] = e;
        const bool valid = e >= 0;
        peers &= ~__ballot(dup);  // the group of well-formed routes with this expert
        int r = 0;
        if (valid) {
            const int before = __popcll(peers & lt);
            r = hist[e] + before;          // every lane reads before any lane writes
            if (before == 0) hist[e] += __popcll(peers);
        }
        rank_w[it] = r;
        ex[it] = e;
    }
    // malformed routes: one atomic per wave
    const uint64_t badm = __ballot(n_bad > 0);
    const int wave_bad = wave_sum_i32(n_bad);
    if (badm && lane == 0) atomicAdd(&ctrl[CTRL_BAD_ROUTES], wave_bad);
    __syncthreads();
    // one block (at most kCountBlock routes): its totals are the counts and no
    // other block takes part, so they stay in registers
    constexpr int kMaxEPerThread = 4;
    const bool single = gridDim.x == 1 && E <= kMaxEPerThread * (int)blockDim.x;
    int32_t tot[kMaxEPerThread];
    for (int i = 0, e = tid; e < E; ++i, e += blockDim.x) {
        int32_t run = 0;
        for (int w = 0; w < kCountWaves; ++w) {
            const int32_t c = lds[w * E + e];
            lds[w * E + e] = run;
            run += c;
        }
        if (single) {
            if (i < kMaxEPerThread) tot[i] = run;
        } else if (local_scan) {
            partial[(int64_t)blockIdx.x * E + e] = run;   // read by the next kernel
        } else {
            // write-through to the device-coherent level: the last block reads it
            __hip_atomic_store(&partial[(int64_t)blockIdx.x * E + e], run, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kCountPerLane; ++it) {
        const int64_t q = q0 + it * kWave + lane;
        rank_w[it] = ex[it] >= 0 ? hist[ex[it]] + rank_w[it] : -1;   // rank in the block
        if (q < Q) lrank[q] = rank_w[it];
    }

    int32_t* kept = lds;
    int32_t* tiles = lds + E;
    // offsets and the m-tile table from kept[] / tiles[] (all threads)
    auto finish = [&]() {
        __syncthreads();
        block_scan2(kept, tiles, E, &s_tot[0], &s_tot[1]);
        for (int e = tid; e < E; e += blockDim.x) {
            offsets[e] = kept[e];
            mt_off[e] = tiles[e];
        }
        if (tid == 0) {
            offsets[E] = s_tot[0];
            mt_off[E] = s_tot[1];
        }
    };
    if (single) {
        __syncthreads();   // every thread is done reading the histograms
        for (int i = 0, e = tid; e < E; ++i, e += blockDim.x) {
            partial[e] = 0;   // the only block's base
            counts[e] = tot[i];
            const int32_t kp = tot[i] < C ? tot[i] : C;
            kept[e] = kp;
            tiles[e] = (kp + bm - 1) / bm;
        }
        finish();
        if (route_dst != nullptr) {
            // the only block: its ranks are final, so it places the routes
            // (kept[] holds the offsets after the scan)
#pragma unroll
            for (int it = 0; it < kCountPerLane; ++it) {
                const int64_t q = q0 + it * kWave + lane;
                if (q >= Q) continue;
                const int e = ex[it];
                int32_t row = -2;
                if (e >= 0) {
                    row = rank_w[it] < C ? kept[e] + rank_w[it] : -1;
                    if (row >= 0) row_src[row] = (int32_t)q;
                }
                route_dst[q] = row;
            }
            for (int64_t r = s_tot[0] + tid; r < r_max; r += blockDim.x) row_src[r] = -1;
        }
        return;
    }

    // the scatter kernel scans the per-block totals itself
    if (local_scan) return;

    // ---- last block: per-block bases, counts, offsets, m-tile table ----
    // Only the per-block totals cross blocks inside this kernel.  They were
    // stored write-through (agent-scope atomic stores); once every thread's
    // stores have completed the ticket is taken, and the last block reads
    // them with agent-scope atomic loads.  No fence is needed, so the L2
    // holds on to its dirty lines (an agent-scope fence writes back the
    // whole L2 of the XCD).  Everything else this kernel writes is read by
    // later kernels.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // `delay`: block 0 holds back its ticket (about 8k clocks per step), so
    // that it arrives last and reads every other block's totals; a test of the
    // hand-off sets it from the host (0 otherwise)
    if (blockIdx.x == 0)
        for (int i = 0; i < delay; ++i) __builtin_amdgcn_s_sleep(127);
    if (tid == 0)
        s_last = (__hip_atomic_fetch_add(&ctrl[CTRL_TICKET], 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    const int nb = gridDim.x;
    for (int e = tid; e < E; e += blockDim.x) {
        int32_t run = 0;
        for (int b0 = 0; b0 < nb; b0 += 8) {
            // eight blocks' totals in flight at once
            int32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                c[i] = b0 + i < nb ? __hip_atomic_load(&partial[(int64_t)(b0 + i) * E + e],
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (b0 + i < nb) {
                    partial[(int64_t)(b0 + i) * E + e] = run;
                    run += c[i];
                }
        }
        counts[e] = run;
        const int32_t kp = run < C ? run : C;
        kept[e] = kp;
        tiles[e] = (kp + bm - 1) / bm;
    }
    finish();
    if (tid == 0) ctrl[CTRL_TICKET] = 0;
}

__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int bm, int32_t* __restrict__ mt_off) {
    extern __shared__ int32_t lds[];
    __shared__ int32_t s_tot[2];
    int32_t* tiles = lds;
    int32_t* dummy = lds + E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int32_t kp = offsets[e + 1] - offsets[e];
        tiles[e] = (kp + bm - 1) / bm;
        dummy[e] = 0;
    }
    __syncthreads();
    block_scan2(tiles, dummy, E, &s_tot[0], &s_tot[1]);
    for (int e = threadIdx.x; e < E; e += blockDim.x) mt_off[e] = tiles[e];
    if (threadIdx.x == 0) mt_off[E] = s_tot[0];
}

template <typename V>
__global__ __launch_bounds__(256) void scatter_kernel(
    const V* __restrict__ x, int H_vec, int k, int E, int C, int64_t r_max,
    const int32_t* __restrict__ rexp, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ route_dst, int32_t* __restrict__ row_src, V* __restrict__ x_disp) {
    __shared__ int32_t s_row[32];
    const int t = blockIdx.x, tid = threadIdx.x;
    if (tid < k) {
        const int64_t q = (int64_t)t * k + tid;
        const int e = rexp[q];
        int32_t row;
        if (e < 0) {
            row = -2;
        } else {
            const int32_t r = base[(q / kCountBlock) * E + e] + lrank[q];
            row = r < C ? offsets[e] + r : -1;
            if (row >= 0) row_src[row] = (int32_t)q;
        }
        route_dst[q] = row;
        s_row[tid] = row;
    }
    // rows R .. r_max-1 of row_src are unused: -1 (grid-stride over all blocks)
    const int64_t R = offsets[E];
    for (int64_t r = R + (int64_t)blockIdx.x * blockDim.x + tid; r < r_max;
         r += (int64_t)gridDim.x * blockDim.x)
        row_src[r] = -1;
    __syncthreads();
    if (x_disp == nullptr) return;  // metadata only (slot-indexed expert GEMMs read x in place)
    const V* src = x + (int64_t)t * H_vec;
    for (int c = tid; c < H_vec; c += blockDim.x) {
        const V v = src[c];
        for (int j = 0; j < k; ++j) {
            const int32_t row = s_row[j];
            if (row >= 0) x_disp[(int64_t)row * H_vec + c] = v;
        }
    }
}

// Metadata only (the expert GEMMs read x in place): one thread per route.
__global__ __launch_bounds__(256) void scatter_meta_kernel(
    int64_t Q, int E, int C, int64_t r_max, const int32_t* __restrict__ rexp,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ route_dst,
    int32_t* __restrict__ row_src) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid < Q) {
        const int e = rexp[gid];
        int32_t row;
        if (e < 0) {
            row = -2;
        } else {
            const int32_t r = base[(gid / kCountBlock) * E + e] + lrank[gid];
            row = r < C ? offsets[e] + r : -1;
            if (row >= 0) row_src[row] = (int32_t)gid;
        }
        route_dst[gid] = row;
    }
    // rows R .. r_max-1 of row_src are unused: -1
    for (int64_t r = offsets[E] + gid; r < r_max; r += (int64_t)gridDim.x * blockDim.x) row_src[r] = -1;
}

// Metadata scatter with its own scan, for launches whose per-block totals
// are few (count blocks x experts <= kLocalScanMax): every block reads the
// count kernel's per-block totals into LDS and forms the per-block bases,
// counts and offsets itself, so the count kernel needs no hand-off between
// its blocks.  One thread per route; block 0 also writes counts, offsets and
// the m-tile table (tile rows bm).  (With the row copy, one block per token,
// the repeated scan cost more than the hand-off saves: measured at 16384
// routes, count 11.8 -> 8.0 us but scatter 12.6 -> 17.4 us.)
__global__ __launch_bounds__(256) void scatter_scan_kernel(
    int64_t Q, int E, int C, int bm, int nb, int64_t r_max, const int32_t* __restrict__ rexp,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ cnt, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ mt_off, int32_t* __restrict__ route_dst,
    int32_t* __restrict__ row_src) {
    extern __shared__ int32_t lds[];   // [nb][E] totals -> bases, then kept[E], tiles[E]
    __shared__ int32_t s_tot[2];
    const int tid = threadIdx.x;
    int32_t* kept = lds + nb * E;
    int32_t* tiles = kept + E;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + tid;
    int e = -1, lr = 0;
    if (q < Q) {
        e = rexp[q];
        lr = lrank[q];
    }
    for (int i = tid; i < nb * E; i += blockDim.x) lds[i] = cnt[i];
    __syncthreads();
    // per expert: bases over the count blocks, raw count, kept rows, tiles
    for (int x = tid; x < E; x += blockDim.x) {
        int32_t run = 0;
        for (int b = 0; b < nb; ++b) {
            const int32_t c = lds[b * E + x];
            lds[b * E + x] = run;
            run += c;
        }
        if (blockIdx.x == 0) counts[x] = run;
        const int32_t kp = run < C ? run : C;
        kept[x] = kp;
        tiles[x] = (kp + bm - 1) / bm;
    }
    __syncthreads();
    block_scan2(kept, tiles, E, &s_tot[0], &s_tot[1]);   // kept -> offsets, tiles -> m-tile table
    if (blockIdx.x == 0) {
        for (int x = tid; x < E; x += blockDim.x) {
            offsets[x] = kept[x];
            mt_off[x] = tiles[x];
        }
        if (tid == 0) {
            offsets[E] = s_tot[0];
            mt_off[E] = s_tot[1];
        }
    }
    if (q < Q) {
        int32_t row = -2;
        if (e >= 0) {
            const int32_t r = lds[(int)(q / kCountBlock) * E + e] + lr;
            row = r < C ? kept[e] + r : -1;
            if (row >= 0) row_src[row] = (int32_t)q;
        }
        route_dst[q] = row;
    }
    // rows R .. r_max-1 of row_src are unused: -1 (grid-stride over all blocks)
    for (int64_t r = s_tot[0] + q; r < r_max; r += (int64_t)gridDim.x * blockDim.x) row_src[r] = -1;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// 32-bit word copy (preselected ids / weights into the caller's metadata
// outputs): a kernel rather than a copy command, so a captured graph holds
// kernel nodes only.
__global__ void copy_u32_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

// ---- small batches: routing and the whole dispatch in one workgroup ---------
// For T <= kSmallMaxT tokens (T*k <= 2048 routes) one 1024-thread workgroup
// routes the tokens (or takes the caller's ids), ranks the routes, scans the
// counts and places every route, so no block hand-off and no further launch is
// needed.  Wave w ranks routes [128 w, 128 w + 128) in two 64-route steps,
// exactly as the count kernel does; the ids live in LDS.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;        // 16
constexpr int kSmallTokPerWave = kSmallMaxT / kSmallWaves;  // 4
constexpr int kSmallSteps = 2;                            // 64-route steps per wave

// Exclusive scan of one value per thread over the workgroup (1024 threads);
// returns the thread's exclusive prefix and writes the total to *tot.
__device__ int32_t block_exclusive_scan_1024(int32_t v, int32_t* s_wsum, int32_t* tot) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int32_t x = wave_incl_scan(v, lane);
    if (lane == kWave - 1) s_wsum[wv] = x;
    __syncthreads();
    if (wv == 0) {
        const int32_t u = wave_incl_scan(lane < kSmallWaves ? s_wsum[lane] : 0, lane);
        if (lane < kSmallWaves) s_wsum[lane] = u;   // inclusive over waves
    }
    __syncthreads();
    const int32_t before = wv > 0 ? s_wsum[wv - 1] : 0;
    *tot = s_wsum[kSmallWaves - 1];
    __syncthreads();
    return before + x - v;
}

template <int EPL, bool SIG>
__global__ __launch_bounds__(kSmallThreads) void small_dispatch_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ ids_in, int T, int k, int E, int ebits, int C, int bm, int renorm,
    float scale, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ mt_off,
    int32_t* __restrict__ row_src, int64_t r_max, int32_t* __restrict__ route_dst,
    int32_t* __restrict__ ctrl) {
    extern __shared__ int32_t lds[];          // hist [kSmallWaves][E], then offsets [E + 1]
    __shared__ int32_t s_ids[kSmallMaxT * 32];
    __shared__ int32_t s_wsum[2][kSmallWaves];
    __shared__ int32_t s_tot[2];
    int32_t* hist = lds;
    int32_t* s_off = lds + kSmallWaves * E;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int Q = T * k;

    // ---- routes ----
    if (ids_in != nullptr) {
        for (int q = tid; q < Q; q += kSmallThreads) s_ids[q] = ids_in[q];
    } else {
        float v[kSmallTokPerWave][EPL];
#pragma unroll
        for (int i = 0; i < kSmallTokPerWave; ++i) {   // all rows first: one memory latency
            const int t = wv + kSmallWaves * i;
            if (t < T) load_logits<EPL>(logits + (int64_t)t * E, E, lane, v[i]);
        }
#pragma unroll
        for (int i = 0; i < kSmallTokPerWave; ++i) {
            const int t = wv + kSmallWaves * i;
            if (t >= T) break;  // wave-uniform
            int id;
            float wt;
            route_row<EPL, SIG>(v[i], bias, E, k, renorm, scale, lane, id, wt);
            if (lane < k) {
                ids_out[t * k + lane] = id;
                w_out[t * k + lane] = wt;
                s_ids[t * k + lane] = id;
            }
        }
    }
    for (int i = tid; i < kSmallWaves * E; i += kSmallThreads) hist[i] = 0;
    __syncthreads();

    // ---- stable ranks within each wave's 128 routes (see count_rank_kernel) ----
    int32_t* wh = hist + wv * E;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int rank_w[kSmallSteps], ex[kSmallSteps];
    int n_bad = 0;
    const int lmk = lane % k, s64 = kWave % k;
    int jb = (wv * (kWave * kSmallSteps)) % k;
#pragma unroll
    for (int it = 0; it < kSmallSteps; ++it) {
        const int q = wv * (kWave * kSmallSteps) + it * kWave + lane;
        const bool inq = q < Q;
        int e = inq ? s_ids[q] : -1;
        const bool inrange = inq && e >= 0 && e < E;
        uint64_t peers = __ballot(inrange);
        for (int b = 0; b < ebits; ++b) {
            const bool bit = inrange && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        bool dup = false;
        if (inrange) {
            int j = jb + lmk;   // q mod k (see count_rank_kernel)
            if (j >= k) j -= k;
            const int first = lane - j;
            dup = (peers & lt & ~((first > 0) ? (~0ull >> (64 - first)) : 0ull)) != 0;
            for (int jj = 0; !dup && jj < -first; ++jj) dup = s_ids[q - j + jj] == e;
        }
        jb += s64;
        if (jb >= k) jb -= k;
        if (inq && (!inrange || dup)) {
            e = -2;
            ++n_bad;
        }
        const bool valid = e >= 0;
        peers &= ~__ballot(dup);
        int r = 0;
        if (valid) {
            const int before = __popcll(peers & lt);
            r = wh[e] + before;
            if (before == 0) wh[e] += __popcll(peers);
        }
        rank_w[it] = r;
        ex[it] = e;
    }
    const int wave_bad = wave_sum_i32(n_bad);
    if (wave_bad && lane == 0) atomicAdd(&ctrl[CTRL_BAD_ROUTES], wave_bad);
    __syncthreads();

    // ---- per-expert totals, wave bases, exclusive scans ----
    int32_t kept = 0, tiles = 0;
    for (int e = tid; e < E; e += kSmallThreads) {   // E <= 1024: one expert per thread
        int32_t run = 0;
        for (int w = 0; w < kSmallWaves; ++w) {
            const int32_t c = hist[w * E + e];
            hist[w * E + e] = run;
            run += c;
        }
        counts[e] = run;
        kept = run < C ? run : C;
        tiles = (kept + bm - 1) / bm;
    }
    const int32_t off_e = block_exclusive_scan_1024(kept, s_wsum[0], &s_tot[0]);
    const int32_t mt_e = block_exclusive_scan_1024(tiles, s_wsum[1], &s_tot[1]);
    if (tid < E) {
        offsets[tid] = off_e;
        mt_off[tid] = mt_e;
        s_off[tid] = off_e;
    }
    if (tid == 0) {
        offsets[E] = s_tot[0];
        mt_off[E] = s_tot[1];
        s_off[E] = s_tot[0];
    }
    __syncthreads();

    // ---- place every route ----
#pragma unroll
    for (int it = 0; it < kSmallSteps; ++it) {
        const int q = wv * (kWave * kSmallSteps) + it * kWave + lane;
        if (q >= Q) continue;
        const int e = ex[it];
        int32_t row = -2;
        if (e >= 0) {
            const int32_t r = hist[wv * E + e] + rank_w[it];
            row = r < C ? s_off[e] + r : -1;
            if (row >= 0) row_src[row] = q;
        }
        route_dst[q] = row;
    }
    for (int64_t r = s_off[E] + tid; r < r_max; r += kSmallThreads) row_src[r] = -1;
}

// ---- one workgroup for the whole count-first dispatch of small batches ----
// The multi-block count kernel pays three round trips through the device-
// coherent level for its hand-off (write-through totals, the ticket, the
// last block's reload).  Up to kPlaceMaxQ routes, one 1024-thread workgroup
// instead ranks every route itself: wave w takes the contiguous routes
// [64 PER w, 64 PER (w + 1)) in PER 64-route steps, ranks them by ballots
// over the expert bits against its running LDS histogram (as count_rank
// does), then the per-expert totals are prefix-summed over the 16 waves,
// scanned into offsets and the m-tile table, and every route is placed
// (route_dst, row_src) with no second launch.  A lane keeps each of its
// routes as one packed word: (expert + 2) << 21 | in-wave rank.
template <int PER>
__global__ __launch_bounds__(kSmallThreads) void count_place_kernel(
    const int32_t* __restrict__ ids, int Q, int k, int E, int ebits, int C, int bm,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ mt_off,
    int32_t* __restrict__ row_src, int64_t r_max, int32_t* __restrict__ route_dst,
    int32_t* __restrict__ ctrl) {
    extern __shared__ int32_t lds[];   // hist [kSmallWaves][E], then offsets [E + 1]
    __shared__ int32_t s_wsum[2][kSmallWaves], s_tot[2];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    int32_t* hist = lds;
    int32_t* s_off = lds + kSmallWaves * E;
    for (int i = tid; i < kSmallWaves * E; i += kSmallThreads) hist[i] = 0;
    __syncthreads();
    int32_t* wh = hist + wv * E;
    const int q0 = wv * (kWave * PER);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t pk[PER];
    int n_bad = 0;
    const int lmk = lane % k, s64 = kWave % k;
    int jb = q0 % k;
    // this lane's ids first: one memory latency for all of them
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int q = q0 + it * kWave + lane;
        pk[it] = q < Q ? (uint32_t)ids[q] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int q = q0 + it * kWave + lane;
        const bool inq = q < Q;
        int e = (int)pk[it];
        const bool inrange = inq && e >= 0 && e < E;
        uint64_t peers = __ballot(inrange);
        for (int b = 0; b < ebits; ++b) {
            const bool bit = inrange && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        // duplicate: an earlier slot of the same token holds the same expert
        // (slots before this 64-route step are read back from memory)
        bool dup = false;
        if (inrange) {
            int j = jb + lmk;   // q mod k (see count_rank_kernel)
            if (j >= k) j -= k;
            const int first = lane - j;
            dup = (peers & lt & ~((first > 0) ? (~0ull >> (64 - first)) : 0ull)) != 0;
            for (int jj = 0; !dup && jj < -first; ++jj) dup = ids[q - j + jj] == e;
        }
        jb += s64;
        if (jb >= k) jb -= k;
        if (inq && (!inrange || dup)) {
            e = -2;
            ++n_bad;
        }
        peers &= ~__ballot(dup);
        int r = 0;
        if (e >= 0) {
            const int before = __popcll(peers & lt);
            r = wh[e] + before;          // every lane reads before any lane writes
            if (before == 0) wh[e] += __popcll(peers);
        }
        pk[it] = inq ? ((uint32_t)(e + 2) << 21) | (uint32_t)r : 0u;
    }
    const int wave_bad = wave_sum_i32(n_bad);
    if (wave_bad && lane == 0) atomicAdd(&ctrl[CTRL_BAD_ROUTES], wave_bad);
    __syncthreads();

    // per-expert totals (wave bases in place), kept counts and tiles, scans
    int32_t kept = 0, tiles = 0;
    for (int e = tid; e < E; e += kSmallThreads) {   // E <= 1024: one expert per thread
        int32_t run = 0;
        for (int w = 0; w < kSmallWaves; ++w) {
            const int32_t c = hist[w * E + e];
            hist[w * E + e] = run;
            run += c;
        }
        counts[e] = run;
        kept = run < C ? run : C;
        tiles = (kept + bm - 1) / bm;
    }
    const int32_t off_e = block_exclusive_scan_1024(kept, s_wsum[0], &s_tot[0]);
    const int32_t mt_e = block_exclusive_scan_1024(tiles, s_wsum[1], &s_tot[1]);
    if (tid < E) {
        offsets[tid] = off_e;
        mt_off[tid] = mt_e;
        s_off[tid] = off_e;
    }
    if (tid == 0) {
        offsets[E] = s_tot[0];
        mt_off[E] = s_tot[1];
        s_off[E] = s_tot[0];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < PER; ++it) {
        const int q = q0 + it * kWave + lane;
        if (q >= Q) continue;
        const uint32_t w = pk[it];
        const int e = (int)(w >> 21) - 2;
        int32_t row = -2;
        if (e >= 0) {
            const int32_t r = hist[wv * E + e] + (int32_t)(w & 0x1FFFFFu);
            row = r < C ? s_off[e] + r : -1;
            if (row >= 0) row_src[row] = q;
        }
        route_dst[q] = row;
    }
    for (int64_t r = s_off[E] + tid; r < r_max; r += kSmallThreads) row_src[r] = -1;
}

// Row copies of placed routes: one block per token stores its row (read
// once) to every kept row of its routes (route_dst >= 0).
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint4* __restrict__ x, int H_vec, int k,
                                                        const int32_t* __restrict__ route_dst,
                                                        uint4* __restrict__ x_disp) {
    __shared__ int32_t s_row[32];
    const int t = blockIdx.x, tid = threadIdx.x;
    if (tid < k) s_row[tid] = route_dst[(int64_t)t * k + tid];
    __syncthreads();
    const uint4* src = x + (int64_t)t * H_vec;
    for (int c = tid; c < H_vec; c += blockDim.x) {
        const uint4 v = src[c];
        for (int j = 0; j < k; ++j) {
            const int32_t row = s_row[j];
            if (row >= 0) x_disp[(int64_t)row * H_vec + c] = v;
        }
    }
}

}  // namespace

hipError_t launch_copy_u32(void* dst, const void* src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(copy_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)dst,
                       (const uint32_t*)src, n);
    return hipGetLastError();
}

hipError_t launch_small_dispatch(const float* logits, const float* bias, const int32_t* ids_in,
                                int T, int k, int E, int C, int bm, int score_func, int renorm,
                                float scale, int32_t* ids, float* w, int32_t* counts,
                                int32_t* offsets, int32_t* mt_off, int32_t* row_src, int64_t r_max,
                                int32_t* route_dst, int32_t* ctrl, hipStream_t s) {
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    const size_t lds = sizeof(int32_t) * ((size_t)kSmallWaves * E + E + 1);
    auto go = [&](auto epl) {
        constexpr int EPL = decltype(epl)::value;
        if (score_func == MOE_SIGMOID)
            hipLaunchKernelGGL((small_dispatch_kernel<EPL, true>), dim3(1), dim3(kSmallThreads), lds, s,
                               logits, bias, ids_in, T, k, E, ebits, C, bm, renorm, scale, ids, w,
                               counts, offsets, mt_off, row_src, r_max, route_dst, ctrl);
        else
            hipLaunchKernelGGL((small_dispatch_kernel<EPL, false>), dim3(1), dim3(kSmallThreads), lds,
                               s, logits, bias, ids_in, T, k, E, ebits, C, bm, renorm, scale, ids, w,
                               counts, offsets, mt_off, row_src, r_max, route_dst, ctrl);
    };
    if (E <= 64) go(std::integral_constant<int, 1>{});
    else if (E <= 128) go(std::integral_constant<int, 2>{});
    else if (E <= 256) go(std::integral_constant<int, 4>{});
    else if (E <= kSmallMaxE) go(std::integral_constant<int, 8>{});
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_count_rank(const int32_t* ids, int T, int k, int E, int C, int bm, int32_t* rexp,
                             int32_t* lrank, int32_t* partial, int32_t* counts, int32_t* offsets,
                             int32_t* mt_off, int32_t* ctrl, hipStream_t s, int32_t* route_dst,
                             int32_t* row_src, int64_t r_max, int local_scan) {
    // MOE_COUNT_DELAY (read once): hold back block 0's ticket by that many
    // steps of about 8k clocks, so a test can make it the last block to arrive
    static const int delay = [] {
        const char* e = std::getenv("MOE_COUNT_DELAY");
        return e ? std::atoi(e) : 0;
    }();
    const int64_t Q = (int64_t)T * k;
    const int nb = count_blocks(Q) > 0 ? count_blocks(Q) : 1;
    int ebits = 1;
    while ((1 << ebits) < E) ++ebits;
    const size_t lds = sizeof(int32_t) * (size_t)kCountWaves * E;
    if (route_dst != nullptr && nb != 1) return hipErrorInvalidValue;   // placement needs the one block
    if (local_scan && !local_scan_fits(Q, E)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(count_rank_kernel, dim3(nb), dim3(kWave * kCountWaves), lds, s, ids, Q, k, E,
                       ebits, C, bm, rexp, lrank, partial, counts, offsets, mt_off, ctrl, route_dst,
                       row_src, r_max, delay, local_scan);
    return hipGetLastError();
}

hipError_t launch_count_place(const int32_t* ids, int T, int k, int E, int C, int bm,
                              int32_t* counts, int32_t* offsets, int32_t* mt_off, int32_t* row_src,
                              int64_t r_max, int32_t* route_dst, int32_t* ctrl, hipStream_t s) {
    const int64_t Q = (int64_t)T * k;
    if (Q <= 0 || Q > kPlaceMaxQ) return hipErrorInvalidValue;
    int ebits = 1;
    while ((1 << ebits) < E) ++ebits;
    const size_t lds = sizeof(int32_t) * ((size_t)kSmallWaves * E + E + 1);
    const int per = (int)((Q + kSmallThreads - 1) / kSmallThreads);   // routes per lane
    auto go = [&](auto per_c) {
        constexpr int PER = decltype(per_c)::value;
        hipLaunchKernelGGL((count_place_kernel<PER>), dim3(1), dim3(kSmallThreads), lds, s, ids, (int)Q, k,
                           E, ebits, C, bm, counts, offsets, mt_off, row_src, r_max, route_dst, ctrl);
    };
    static_assert(kPlaceMaxQ <= 4 * kSmallThreads, "at most 4 routes per lane");
    if (per <= 2) go(std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, 4>{});
    return hipGetLastError();
}

hipError_t launch_copy_rows(const void* x, int T, int H, int k, int elem_bytes, const int32_t* route_dst,
                            void* x_disp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int H_vec = (int)((int64_t)H * elem_bytes / 16);   // H * elem_bytes is a multiple of 256
    hipLaunchKernelGGL(copy_rows_kernel, dim3(T), dim3(256), 0, s, (const uint4*)x, H_vec, k, route_dst,
                       (uint4*)x_disp);
    return hipGetLastError();
}

hipError_t launch_tile_table(const int32_t* offsets, int E, int C, int bm, int32_t* mt_off,
                             hipStream_t s) {
    (void)C;
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(256), sizeof(int32_t) * 2 * (size_t)E, s,
                       offsets, E, bm, mt_off);
    return hipGetLastError();
}

hipError_t launch_scatter(const void* x, int T, int H, int k, int E, int C, int elem_bytes,
                          int64_t r_max, const int32_t* rexp, const int32_t* lrank,
                          const int32_t* base, const int32_t* offsets, int32_t* route_dst,
                          int32_t* row_src, void* x_disp, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (x_disp == nullptr) {
        const int64_t Q = (int64_t)T * k;
        hipLaunchKernelGGL(scatter_meta_kernel, dim3((unsigned)((Q + 255) / 256)), dim3(256), 0, s, Q, E, C,
                           r_max, rexp, lrank, base, offsets, route_dst, row_src);
        return hipGetLastError();
    }
    const int H_vec = (int)((int64_t)H * elem_bytes / 16);  // H*elem_bytes is a multiple of 256
    hipLaunchKernelGGL(scatter_kernel<uint4>, dim3(T), dim3(256), 0, s, (const uint4*)x, H_vec, k, E,
                       C, r_max, rexp, lrank, base, offsets, route_dst, row_src, (uint4*)x_disp);
    return hipGetLastError();
}

hipError_t launch_scatter_scan(int T, int k, int E, int C, int bm, int64_t r_max, const int32_t* rexp,
                               const int32_t* lrank, const int32_t* cnt, int32_t* counts, int32_t* offsets,
                               int32_t* mt_off, int32_t* route_dst, int32_t* row_src, hipStream_t s) {
    const int64_t Q = (int64_t)T * k;
    if (!local_scan_fits(Q, E)) return hipErrorInvalidValue;
    const int nb = count_blocks(Q);
    const size_t lds = sizeof(int32_t) * ((size_t)nb * E + 2 * (size_t)E);
    hipLaunchKernelGGL(scatter_scan_kernel, dim3((unsigned)((Q + 255) / 256)), dim3(256), lds, s, Q, E, C, bm, nb,
                       r_max, rexp, lrank, cnt, counts, offsets, mt_off, route_dst, row_src);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace rde
