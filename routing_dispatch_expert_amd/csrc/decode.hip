// Slot-indexed expert GEMMs for decode-shaped batches (few rows per expert).
//
// The fleet megakernel report (MoE optimisation steps: "expert = idx[slot]
// read at run time") replaces per-expert dense launches by tasks that read
// the expert of a slot at run time and stream only the touched experts'
// weights; PR 33963 switches kernels on the route count ("128-route
// prefill-tiles dispatch threshold").  Here, when the batch has few rows per
// expert, the expert GEMMs run as this kernel instead of the tiled grouped
// GEMM: every touched expert's weights are streamed once, split into small
// units spread over all wavefronts of the chip, and the activation rows are
// read in place through row_src (the expert-contiguous row copy is skipped).
//
// Work unit: one wavefront computes 32 weight rows x up to 32 activation
// rows with v_mfma_f32_32x32x16_bf16, K streamed in groups of 64.
//   SwiGLU: the 32 weight rows are 16 gate rows and the 16 matching up rows,
//           so for acc register r < 8 the lane holds gate(n) and in r + 8 the
//           matching up(n): 16 output columns of h per unit.
//   other:  32 weight rows = 32 output columns.
// The MFMA is issued as W x A^T: lane l holds activation row (l % 32) and
// weight rows n = 8*(r/4) + 4*(l/32) + r%4 for acc register r.
//
// For launches with few units, the 4 wavefronts of a workgroup work on one
// unit at a time, each on a quarter of K, or each pair of wavefronts on one
// unit, each on half of K (the host chooses from the unit count and K); the
// partial sums are added in LDS in wavefront order.
//
// K order: a work item starts at K group (13 expert + 7 block) mod its group
// count and wraps (see Item::rot).
//
// Loads: each wavefront owns a private 32 KB LDS ring of stages (4 stages of
// 32 activation rows and 32 weight rows of 128 bytes) filled by direct
// global -> LDS loads; it waits only on its own vector-memory counter (no
// workgroup barrier), so each wavefront keeps all stages but the one being
// multiplied in flight.  When no expert can hold more than 8 rows (batches
// of at most 8 tokens) a stage stages only 8 activation rows (5 KB): the
// ring then holds 6 stages and keeps 20 KB of weights in flight instead of
// 12 KB.  Activation rows 8..31 of the MFMA then repeat rows 0..7; their
// output rows are never stored.  Within a 64-wide K group, lane half h supplies K elements
// [32h + 8j, 32h + 8j + 8) to MFMA step j (the same permutation of K for both
// operands leaves the product unchanged), so each lane's bytes for a group
// are one 64-byte run.  16-byte chunk c of row r sits at chunk slot
// c ^ ((r ^ r >> 3) & 7): the fragment reads are free of bank conflicts.
#include <type_traits>

#include "route_wave.h"

namespace rde {
namespace {

constexpr int kDWaves = 4;          // wavefronts per workgroup
constexpr int kDRing = 32768;       // LDS ring bytes per wavefront
constexpr int kDGroupK = 64;        // K elements per stage
constexpr int kDStageRows = 1024;   // kept rows whose routes (and weights) are staged in LDS

// Stage layout: AR activation rows then 32 weight rows, 128 bytes each.
template <bool SMALLM>
struct DRing {
    static constexpr int AR = SMALLM ? 8 : 32;        // activation rows staged
    static constexpr int A_BYTES = AR * 128;
    static constexpr int STAGE = A_BYTES + 4096;
    static constexpr int NST = kDRing / STAGE;        // 4 or 6 stages
    static constexpr int PER = AR / 8 + 4;            // DMA instructions per stage
};

__device__ __forceinline__ uint32_t lds_addr_d(const void* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// One direct global -> LDS load of 16 bytes per lane (see gemm.hip): lane l
// writes LDS `lds` + 16*l; `lds` is wave-uniform.  M0 is saved and restored.
__device__ __forceinline__ void dma16_d(const void* g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(lds)
        : "memory");
}

// Wait until at most PER x n of this wavefront's vector-memory operations are
// outstanding (n = stages issued after the one needed; PER DMA instructions
// per stage).
template <int PER>
__device__ __forceinline__ void wait_stages(int n) {
    switch (n) {
        case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER) : "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;   // never less than needed
    }
}

// Expert owning tile ti: the largest g with tbl[g] <= ti (tbl non-decreasing,
// tbl[0] = 0; experts without rows have tbl[g] == tbl[g + 1]).
__device__ __forceinline__ int find_tile_group(const int32_t* tbl, int n_groups, int ti) {
    int lo = 0, hi = n_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tbl[mid] <= ti) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int dswz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ float silu_mul_d(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}


// Epilogue of one work item: lane holds activation row m = lane % 32 and the
// weight rows n = 8*(r/4) + 4*(lane/32) + r%4 of acc register r.
template <int EPI, bool FP8>
__device__ __forceinline__ void epilogue(const DecodeSeg& s, int group, int blk, int m0, int mrows,
                                         int row_base, int32_t q, float cw, const f32x16& acc,
                                         int lane) {
    const int m = lane & 31;
    if (m >= mrows) return;
    const int64_t orow = (s.offsets == nullptr) ? (int64_t)(m0 + m) : (int64_t)(row_base + m0 + m);
    const int c4 = 4 * (lane >> 5);
    if (EPI == EPI_SWIGLU) {
        __bf16* o = (__bf16*)s.out + orow * s.ldo + (int64_t)group * s.out_col_per_group;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int col = blk * 16 + 8 * q + c4;
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float gv = acc[4 * q + j], uv = acc[8 + 4 * q + j];
                if (FP8) {
                    const float* sc = s.bscale + (int64_t)group * s.N_w;
                    gv *= sc[col + j];
                    uv *= sc[s.I + col + j];
                }
                hv[j] = silu_mul_d(gv, uv);
            }
            *(uint2*)(o + col) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
        return;
    }
    const int64_t drow = EPI == EPI_COMBINE ? (int64_t)q : orow;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int col = blk * 32 + 8 * q + c4;
        if (col >= s.N_w) continue;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = acc[4 * q + j];
            if (FP8) v[j] *= s.bscale[(int64_t)group * s.N_w + col + j];
            if (EPI == EPI_RELU2) v[j] = v[j] > 0.0f ? v[j] * v[j] : 0.0f;
            if (EPI == EPI_COMBINE) v[j] *= cw;
        }
        if (EPI == EPI_F32) {
            *(float4*)((float*)s.out + drow * s.ldo + col) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            const int64_t oc = (EPI == EPI_RELU2) ? (int64_t)group * s.out_col_per_group + col : col;
            *(uint2*)((__bf16*)s.out + drow * s.ldo + oc) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
}

// Inclusive prefix sum over a wavefront (DPP row shifts, then the lower rows'
// totals) and an exclusive one over a 256-thread workgroup.
__device__ __forceinline__ int32_t wave_incl_scan_d(int32_t x, int lane) {
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
// Exclusive scan over the workgroup's 256 threads; s_w (kDWaves ints) must
// not be written again before the workgroup's next barrier.
__device__ int32_t block_excl_scan_256(int32_t v, int32_t* s_w, int32_t& tot) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int32_t x = wave_incl_scan_d(v, lane);
    if (lane == kWave - 1) s_w[wv] = x;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < kDWaves; ++w) {
        if (w < wv) before += s_w[w];
    }
    tot = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    return before + x - v;
}

// Routing and count-first dispatch of a batch of at most kFuseMaxT tokens
// (softmax or sigmoid, at most kFuseMaxE experts), done by every workgroup of a gate/up
// launch with the same result: routes by the wave routing of route_wave.h
// (wave w routes tokens w, w + 4, ...), stable ranks of the T*k <= 256 routes
// (wave w ranks routes 64 w .. 64 w + 63 by ballots over the expert bits, as
// the count kernel does), per-expert totals, exclusive scans of min(count, C)
// and of the 32-row tile counts, then each kept route's row.  The offsets,
// tile table and each row's route land in the kernel's LDS tables; workgroup 0
// also writes ids, weights (when it routed), counts, offsets, the tile table,
// row_src (rows past the kept ones -1) and route_dst.  Preselected routes are
// read instead of routed; malformed ones are counted and marked as in the
// count kernel.  `scratch` (LDS, 4 E + T k ints) is
// free again on return.
static_assert(kFuseMaxQ == kDWaves * kWave, "one 64-route rank step per wavefront");
static_assert(kFuseMaxQ <= kDStageRows && kFuseMaxE <= 4 * kWave && kFuseMaxE <= kDecodeMaxGroups,
              "fused routes staged in LDS; wave routing with 4 experts per lane");
static_assert(sizeof(int32_t) * (kDWaves * kFuseMaxE + kFuseMaxQ) <= (size_t)kDWaves * kDRing,
              "fused dispatch scratch fits in the ring space");
__device__ void fused_dispatch(const DecodeFused& f, int32_t* scratch, int32_t* s_mt, int32_t* s_off,
                               int32_t* s_rs, int32_t* s_w) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const bool writer = blockIdx.x == 0;
    const int T = f.T, k = f.k, E = f.E, Q = T * k;
    int32_t* hist = scratch;            // [kDWaves][E]
    int32_t* sid = scratch + kDWaves * E;   // [Q]
    if (f.ids_in != nullptr) {
        for (int i = tid; i < Q; i += blockDim.x) sid[i] = f.ids_in[i];   // the caller's routes
    } else {
        // experts per lane as in the other routing kernels (1, 2 or 4): the
        // same wave routing, so the same weights
        auto route_tokens = [&](auto epl_c) {
            constexpr int EPL = decltype(epl_c)::value;
            constexpr int TPW = kFuseMaxT / kDWaves;   // tokens per wavefront
            float v[TPW][EPL];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {   // all rows first: one memory latency
                const int t = wv + kDWaves * i;
                if (t < T) load_logits<EPL>(f.logits + (int64_t)t * E, E, lane, v[i]);
            }
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int t = wv + kDWaves * i;
                if (t >= T) break;   // wave-uniform
                int id;
                float wt;
                if (f.sigmoid) route_row<EPL, true>(v[i], f.bias, E, k, f.renorm, f.scale, lane, id, wt);
                else route_row<EPL, false>(v[i], nullptr, E, k, f.renorm, f.scale, lane, id, wt);
                if (lane < k) {
                    sid[t * k + lane] = id;
                    if (writer) {
                        f.ids[t * k + lane] = id;
                        f.w[t * k + lane] = wt;
                    }
                }
            }
        };
        if (E <= kWave) route_tokens(std::integral_constant<int, 1>{});
        else if (E <= 2 * kWave) route_tokens(std::integral_constant<int, 2>{});
        else route_tokens(std::integral_constant<int, 4>{});
    }
    for (int i = tid; i < kDWaves * E; i += blockDim.x) hist[i] = 0;
    __syncthreads();

    // ---- stable ranks within each wave's 64 routes ----
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int q = wv * kWave + lane;
    const bool inq = q < Q;
    int e = inq ? sid[q] : -1;
    const bool inrange = inq && e >= 0 && e < E;
    uint64_t peers = __ballot(inrange);
    for (int b = 0; b < f.ebits; ++b) {
        const bool bit = inrange && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    bool dup = false;
    if (inrange) {
        const int t = q / k, j = q - t * k;
        const int first = lane - j;
        dup = (peers & lt & ~((first > 0) ? (~0ull >> (64 - first)) : 0ull)) != 0;
        for (int jj = 0; !dup && jj < -first; ++jj) dup = sid[t * k + jj] == e;
    }
    int n_bad = 0;
    if (inq && (!inrange || dup)) {
        e = -2;
        n_bad = 1;
    }
    peers &= ~__ballot(dup);
    int32_t* wh = hist + wv * E;
    int rank = 0;
    if (e >= 0) {
        const int before = __popcll(peers & lt);
        rank = wh[e] + before;          // every lane reads before any lane writes
        if (before == 0) wh[e] += __popcll(peers);
    }
    if (writer) {   // workgroup-uniform: only workgroup 0 records malformed routes
        const int wave_bad = wave_sum_i32(n_bad);
        if (wave_bad && lane == 0) atomicAdd(&f.ctrl[CTRL_BAD_ROUTES], wave_bad);
    }
    __syncthreads();

    // ---- per-expert totals and wave bases, then the scans (one expert per thread) ----
    int32_t kept = 0, tiles = 0;
    if (tid < E) {
        int32_t run = 0;
        for (int w = 0; w < kDWaves; ++w) {
            const int32_t c = hist[w * E + tid];
            hist[w * E + tid] = run;
            run += c;
        }
        if (writer) f.counts[tid] = run;
        kept = run < f.C ? run : f.C;
        tiles = (kept + kDecodeBM - 1) / kDecodeBM;
    }
    // one scan of both: kept rows in the high half, 32-row tiles in the low
    // half (sums at most T k <= 256 and E + T k / 32 <= 264: no carry between them)
    static_assert(kFuseMaxQ < (1 << 15) && kFuseMaxE + kFuseMaxQ / kDecodeBM < (1 << 16), "packed scan halves");
    int32_t tot_p;
    const int32_t sc = block_excl_scan_256((kept << 16) | tiles, s_w, tot_p);
    const int32_t off_e = sc >> 16, mt_e = sc & 0xffff;
    const int32_t tot_k = tot_p >> 16, tot_t = tot_p & 0xffff;
    if (tid < E) {
        s_off[tid] = off_e;
        s_mt[tid] = mt_e;
        if (writer) {
            f.offsets[tid] = off_e;
            f.mt[tid] = mt_e;
        }
    }
    if (tid == 0) {
        s_off[E] = tot_k;
        s_mt[E] = tot_t;
        if (writer) {
            f.offsets[E] = tot_k;
            f.mt[E] = tot_t;
        }
    }
    __syncthreads();

    // ---- place every route ----
    if (inq) {
        int32_t row = -2;
        if (e >= 0) {
            const int32_t r = hist[wv * E + e] + rank;
            row = r < f.C ? s_off[e] + r : -1;
            if (row >= 0) {
                s_rs[row] = q / k;   // the gate/up launch gathers: the row's token
                if (writer) f.row_src[row] = q;
            }
        }
        if (writer) f.route_dst[q] = row;
    }
    if (writer)
        for (int64_t r = tot_k + tid; r < f.r_max; r += blockDim.x) f.row_src[r] = -1;
    __syncthreads();
}

// One work item: a unit (32 weight rows of one expert) times a block of up to
// 32 of the expert's activation rows, over this wavefront's K range.
struct Item {
    int64_t u;              // unit index over the launch
    int si, group, blk;     // segment, expert, 32-row weight block
    int base, rows, m0;     // expert's first row, its row count, this block's first row
    int mrows;              // rows in this block
    int g0, nK;             // first K group of this wavefront, K groups
    int rot;                // K group this wavefront starts at (0 .. nK-1), then wraps
    int32_t q;              // combine epilogue: route of this lane's row
    float cw;               // and its weight
    const char* asrc[4];
    const char* bsrc[4];
    int dummy;              // (SPL = 2) a position past the last unit: only the pair's barriers
};

// Units are numbered segment by segment; within a segment, group-major with
// the 32-row weight blocks fastest.  SPL = 4: a workgroup takes one unit at
// a time and its wavefronts split the unit's K range (each streams a quarter
// of the weight rows through its own ring; the partial sums meet in LDS), for
// launches with few units.  SPL = 2: each pair of wavefronts takes a unit and
// splits its K in halves.  SPL = 1: every wavefront takes units on its own,
// dealt to workgroups first (unit u to workgroup u % grid, wavefront
// u / grid), so that a launch with fewer units than wavefronts still spreads
// them over every CU.  Work items exist only for experts
// with rows (the dispatch's 32-row tile table, kept in LDS with the experts'
// row ranges).
template <int EPI0, int EPI1, bool FP8, int SPL, bool SMALLM, bool FUSED>
__global__ __launch_bounds__(kDWaves * 64, 1) void decode_gemm_kernel(DecodeArgs d) {
    using RG = DRing<SMALLM>;
    __shared__ __attribute__((aligned(1024))) unsigned char rings[kDWaves][kDRing];

    // wave index in a scalar register: the work item, and with it the segment
    // descriptor, is then wave-uniform (scalar loads, no vector-memory wait)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // tile table and row ranges of segment 0 when it is routed
    __shared__ int32_t s_mt[kDecodeMaxGroups + 1], s_off[kDecodeMaxGroups + 1];
    // and, for batches of at most kDStageRows kept rows, each row's token
    // (launches that gather their activation rows) or route and combine
    // weight (down projection): a work item then finds its activation rows
    // and weights in LDS instead of through two dependent global loads made
    // while its ring is empty, and divides by k nowhere
    __shared__ int32_t s_rs[kDStageRows];
    __shared__ float s_rw[EPI0 == EPI_COMBINE ? kDStageRows : 1];
    bool staged = false;   // workgroup-uniform
    if (FUSED) {
        // this launch routes and dispatches the batch itself (the ring space is
        // free until the first work item)
        __shared__ int32_t s_w4[kDWaves];
        fused_dispatch(d.fused, (int32_t*)&rings[0][0], s_mt, s_off, s_rs, s_w4);
        staged = true;   // kept rows <= T k <= kFuseMaxQ <= kDStageRows
    } else if (d.seg[0].mt) {
        // The tables and the routes of the first rows are read in the same
        // round trip (the kept rows, at most row_src's length, are known only
        // from the tables): for each row, the token of its route for launches
        // that gather their activation rows, the route itself and its weight
        // for the combine epilogue.  Rows past the kept ones hold -1.
        const bool want = d.seg[0].gather || EPI0 == EPI_COMBINE;
        const int npre = want ? (int)min((int64_t)kDStageRows, d.rs_len) : 0;
        const int ng = d.seg[0].n_groups, tid = threadIdx.x;
        constexpr int NT = kDWaves * kWave, TJ = (kDecodeMaxGroups + NT) / NT, RJ = kDStageRows / NT;
        static_assert(kDStageRows % NT == 0, "staged rows: whole passes of the workgroup");
        // every load is issued before any value is used: one memory latency
        int32_t tm[TJ], to[TJ], qv[RJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int i = tid + NT * j;
            if (i <= ng) {
                tm[j] = d.seg[0].mt[i];
                to[j] = d.seg[0].offsets[i];
            }
        }
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int i = tid + NT * j;
            if (i < npre) qv[j] = d.row_src[i];
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int i = tid + NT * j;
            if (i <= ng) {
                s_mt[i] = tm[j];
                s_off[i] = to[j];
            }
        }
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int i = tid + NT * j;
            if (i < npre) {
                const int32_t q = qv[j];
                s_rs[i] = EPI0 == EPI_COMBINE ? q : q / d.k_top;
                if (EPI0 == EPI_COMBINE) s_rw[i] = q >= 0 ? d.route_w[q] : 0.0f;
            }
        }
        __syncthreads();
        const int R = s_off[d.seg[0].n_groups];
        staged = want && R <= npre;
    }
    // work items: 32-row tiles x weight blocks; routed segments own tiles only
    // for experts with rows (tile table), uniform ones ceil(rows / 32) per group
    auto items = [&](int si) -> int64_t {
        const DecodeSeg& s = d.seg[si];
        const int64_t tiles = s.mt ? (int64_t)(si == 0 ? s_mt[s.n_groups] : s.mt[s.n_groups])
                                   : (int64_t)s.n_groups * ((s.uniform_rows + kDecodeBM - 1) / kDecodeBM);
        return tiles * s.blocks;
    };
    const int64_t n0 = items(0);
    const int64_t n1 = d.n_seg > 1 ? items(1) : 0;
    const int64_t total = n0 + n1;
    // Positions: SPL = 4 takes one unit per workgroup at a time (position
    // b + G r for workgroup b), its wavefronts splitting the unit's K; SPL = 2
    // one unit per pair of wavefronts (position j G + b + 2 G r for pair j).
    // SPL = 1: every wavefront takes whole units (position w G + b + 4 G r for wavefront w),
    // and with tail_split only the complete rounds may run that way: the last,
    // partial round (positions from tail0) is then taken one unit per
    // workgroup and split, so that a fraction of the wavefronts do not each
    // stream one more whole unit while the others wait.
    // Used when there is at least one complete round and the partial one
    // holds at most one unit per workgroup: larger tails cost each split unit
    // its own ring fill and measured slower.
    const int64_t WA = (int64_t)gridDim.x * kDWaves;
    const bool hybrid = SPL == 1 && d.tail_split && total >= WA && total % WA != 0 &&
                        total % WA <= (int64_t)gridDim.x;
    const int64_t tail0 = hybrid ? (total / WA) * WA : total;
    constexpr int SLOTS = kDWaves / SPL;   // units a workgroup works on at a time
    const int64_t first = (int64_t)(wave / SPL) * gridDim.x + blockIdx.x;
    const int64_t stride = (int64_t)SLOTS * gridDim.x;
    // Position p of the loop (slot p % stride, round p / stride) -> unit.  When
    // segment 1's units are longer (the shared experts' down projection runs
    // over their concatenated intermediates), they go to slots that get one
    // unit fewer than the others, in the first round; the routed units take
    // the remaining positions in order.  A bijection on [0, total), the same
    // in every workgroup.
    const int64_t rounds = (total + stride - 1) / stride;
    const int64_t full = total - (rounds - 1) * stride;   // slots with `rounds` units
    const bool spread = !hybrid && n1 > 0 && d.n_seg > 1 && d.seg[1].K > d.seg[0].K &&
                        full < stride && full + n1 <= stride && full <= n0;
    auto unit_at = [&](int64_t p) -> int64_t {
        if (!spread || p < full) return p;
        if (p < full + n1) return n0 + (p - full);
        return p - n1;
    };
    unsigned char* ring = rings[wave];
    const uint32_t ring0 = __builtin_amdgcn_readfirstlane(lds_addr_d(ring));
    const int r32 = lane & 31, h = lane >> 5;
    const int dr = lane >> 3, dsl = lane & 7;   // DMA: instruction i covers rows 8i + lane/8, chunk slot lane%8

    // this wavefront's K range and DMA sources of the item's block m0
    // ways: wavefronts sharing the unit (1, 2 or 4), each taking a 1/ways of its K
    auto setup = [&](Item& it, int m0, int ways) {
        const DecodeSeg& s = d.seg[it.si];
        it.m0 = m0;
        it.mrows = min(kDecodeBM, it.rows - m0);
        const int nKall = s.K / kDGroupK;
        const int kq = (nKall + ways - 1) / ways;
        it.g0 = min(nKall, (wave % ways) * kq);
        it.nK = min(nKall, it.g0 + kq) - it.g0;
        // units running at the same time start at different K groups, so the
        // weight rows (a power-of-two stride apart) are not all read at the
        // same column offset, which would load a few memory channels only;
        // the start depends on the expert and the weight block alone, so a
        // row's summation order never depends on the other tokens
        it.rot = it.nK > 0 ? (it.group * 13 + it.blk * 7) % it.nK : 0;
        const bool fp8 = FP8 && it.si == 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + dr;                 // row within the 32-row block
            const int c = dsl ^ dswz(r);              // logical chunk loaded into slot dsl
            if (i < RG::AR / 8) {
                const int m = min(r, it.mrows - 1);
                int64_t arow;
                if (s.offsets == nullptr) arow = (int64_t)(m0 + m);                            // uniform rows
                else if (s.gather) {                                                             // token of the route
                    const int rr = it.base + m0 + m;
                    arow = staged && it.si == 0 ? (int64_t)s_rs[rr] : (int64_t)(d.row_src[rr] / d.k_top);
                }
                else arow = (int64_t)(it.base + m0 + m);
                it.asrc[i] = (const char*)s.A + (arow * s.lda) * 2 + c * 16;
            }
            int n;
            if ((it.si == 0 ? EPI0 : EPI1) == EPI_SWIGLU) n = r < 16 ? it.blk * 16 + r : s.I + it.blk * 16 + (r - 16);
            else n = min(it.blk * 32 + r, s.N_w - 1);
            // e4m3 rows hold 64 bytes per K group: chunk c < 4 only (slots >= 4 unused)
            it.bsrc[i] = (const char*)s.B + ((int64_t)it.group * s.b_group_stride + (int64_t)n * s.k_seg) * (fp8 ? 1 : 2) +
                         (fp8 ? (c & 3) * 16 : c * 16);
        }
    };
    // item u: segment, expert (tile table), 32-row block, weight block
    auto make = [&](int64_t u, Item& it, int ways) {
        it.u = u;                        // loop position
        it.dummy = SPL == 2 && u >= total;
        if (it.dummy) {
            it.si = 0;
            it.nK = 0;
            return;
        }
        const int64_t un = unit_at(u);   // the unit it holds
        it.si = un < n0 ? 0 : 1;
        const DecodeSeg& s = d.seg[it.si];
        const int64_t lu = it.si == 0 ? un : un - n0;
        const int ti = (int)(lu / s.blocks);
        it.blk = (int)(lu - (int64_t)ti * s.blocks);
        int m0;
        if (s.mt) {
            // routed segments come first (segment 0): table and row ranges in LDS
            it.group = __builtin_amdgcn_readfirstlane(find_tile_group(s_mt, s.n_groups, ti));
            it.base = __builtin_amdgcn_readfirstlane(s_off[it.group]);
            it.rows = __builtin_amdgcn_readfirstlane(s_off[it.group + 1]) - it.base;
            m0 = __builtin_amdgcn_readfirstlane((ti - s_mt[it.group]) * kDecodeBM);
        } else {
            const int tpg = (s.uniform_rows + kDecodeBM - 1) / kDecodeBM;
            it.group = ti / tpg;
            m0 = (ti - it.group * tpg) * kDecodeBM;
            it.base = 0;
            it.rows = s.uniform_rows;
        }
        setup(it, m0, ways);
        if ((it.si == 0 ? EPI0 : EPI1) == EPI_COMBINE) {
            const int m = min(lane & 31, it.mrows - 1);
            const int rr = it.base + m0 + m;
            if (staged && it.si == 0) {
                it.q = s_rs[rr];
                it.cw = s_rw[rr];
            } else {
                it.q = d.row_src[rr];
                it.cw = d.route_w[it.q];
            }
        }
    };
    auto issue = [&](const Item& it, int gk, int slot) {
        const DecodeSeg& s = d.seg[it.si];
        const bool fp8 = FP8 && it.si == 0;
        int gr = gk + it.rot;
        if (gr >= it.nK) gr -= it.nK;
        const int k0 = (it.g0 + gr) * kDGroupK;
        const int seg = k0 / s.k_seg;
        const int64_t kb = (int64_t)seg * s.b_seg_stride + (k0 - seg * s.k_seg);
        const uint32_t st = ring0 + slot * RG::STAGE;
#pragma unroll
        for (int i = 0; i < RG::AR / 8; ++i)
            dma16_d(it.asrc[i] + (int64_t)k0 * 2, __builtin_amdgcn_readfirstlane(st + i * 1024));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16_d(it.bsrc[i] + kb * (fp8 ? 1 : 2), __builtin_amdgcn_readfirstlane(st + RG::A_BYTES + i * 1024));
    };

    // The loop, once for launches that split their partial last round
    // (HYB: whether the current unit is split is a run-time state) and once
    // for the others (fixed by SPL); `hybrid` is workgroup-uniform.
    auto run = [&](auto hyb_c) {
        constexpr bool HYB = decltype(hyb_c)::value;
        Item cur, nxt;
        // the phase-1 positions of every wavefront of a workgroup are equally many,
        // and the phase-2 positions are the workgroup's: both tests are
        // workgroup-uniform where it matters (SPL = 4, and the switch to phase 2)
        bool sp = SPL == 4;   // (HYB) the current unit is split over the workgroup's wavefronts
        int64_t pstride = stride, pend = SPL == 1 ? tail0 : total;
        if (SPL == 2) {
            // both pairs of a workgroup take as many positions as the first
            // pair has units (the second pair's last may be past the end), so
            // that they meet at the same barriers
            const int64_t r2 = blockIdx.x < total ? (total - blockIdx.x + stride - 1) / stride : 0;
            pend = first + stride * r2;
        }
        int64_t p0 = first;
        if (p0 >= pend) {
            if (!HYB || tail0 + blockIdx.x >= total) return;
            sp = true;
            p0 = tail0 + blockIdx.x;
            pstride = gridDim.x;
            pend = total;
        }
        make(p0, cur, HYB ? (sp ? kDWaves : 1) : SPL);
        int issued = 0, consumed = 0;  // stages of this wavefront's stream
        int pre = 0;                   // stages of `cur` already issued
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        while (true) {
            for (; pre < min(RG::NST - 1, cur.nK); ++pre) issue(cur, pre, (issued++) % RG::NST);
            int64_t pn = cur.u + pstride;
            bool has_next = pn < pend;
            if (HYB && !has_next && !sp && tail0 + blockIdx.x < total) {
                has_next = true;   // then the workgroup's share of the partial round
                pn = tail0 + blockIdx.x;
            }
            const bool cur_fp8 = FP8 && cur.si == 0;

            f32x16 acc;
    #pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            for (int gk = 0; gk < cur.nK; ++gk) {
                wait_stages<RG::PER>(min(RG::NST - 2, cur.nK - 1 - gk));
                const unsigned char* sa = ring + (consumed % RG::NST) * RG::STAGE;
                const unsigned char* sb = sa + RG::A_BYTES;
                const int ra = SMALLM ? (r32 & 7) : r32;   // activation row of this lane's fragment
                bf16x8 af[4], bfr[4];
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 4 * h + j;
                    af[j] = *(const bf16x8*)(sa + ra * 128 + ((c ^ dswz(ra)) * 16));
                    if (cur_fp8) {
                        // 8 e4m3 codes at byte (32h + 8j) of the 64-byte row group
                        const int byte = 32 * h + 8 * j;
                        const int cc = byte >> 4;
                        bfr[j] = e4m3x8_to_bf16x8(*(const uint2*)(sb + r32 * 128 + ((cc ^ dswz(r32)) * 16) + (byte & 15)));
                    } else {
                        bfr[j] = *(const bf16x8*)(sb + r32 * 128 + ((c ^ dswz(r32)) * 16));
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage read before it is refilled
                ++consumed;
                const int s3 = gk + RG::NST - 1;
                if (s3 < cur.nK) issue(cur, s3, (issued++) % RG::NST);
    #pragma unroll
                for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[j], acc, 0, 0, 0);
            }

            // ---- sum the wavefronts' K shares in a fixed order (wave 0 first) ----
            // Each wavefront's ring is idle here (its stages are all consumed), so
            // it holds the wavefront's partial sums; the second barrier keeps the
            // rings from being refilled before wavefront 0 has read them.
            // (groups of `wy` wavefronts: the first of each group owns the unit)
            bool owner = true;
            const int wy = HYB ? (sp ? kDWaves : 1) : SPL;
            if (wy > 1) {
                const int w0 = wave - wave % wy;
                if (wave > w0) {
                    float* mine = (float*)ring;
    #pragma unroll
                    for (int r = 0; r < 16; ++r) mine[r * 64 + lane] = acc[r];
                }
                __syncthreads();
                if (wave == w0) {
                    for (int w = w0 + 1; w < w0 + wy; ++w) {
                        const float* theirs = (const float*)rings[w];
    #pragma unroll
                        for (int r = 0; r < 16; ++r) acc[r] += theirs[r * 64 + lane];
                    }
                }
                __syncthreads();
                owner = wave == w0 && !cur.dummy;
            }
            if (owner) {
                if (cur.si == 0)
                    epilogue<EPI0, FP8>(d.seg[0], cur.group, cur.blk, cur.m0, cur.mrows, cur.base, cur.q, cur.cw, acc, lane);
                else
                    epilogue<EPI1, false>(d.seg[1], cur.group, cur.blk, cur.m0, cur.mrows, cur.base, cur.q, cur.cw, acc, lane);
            }
            if (!has_next) break;
            // the next item is set up with nothing of this wavefront's ring in
            // flight: its lookups (row gather, combine weights) are plain loads
            // whose waits would otherwise drain the ring
            if (HYB && !sp && pn >= tail0) {
                sp = true;
                pstride = gridDim.x;
                pend = total;
            }
            make(pn, nxt, HYB ? (sp ? kDWaves : 1) : SPL);
            cur = nxt;
            pre = 0;
        }
    };
    if (hybrid) run(std::true_type{});
    else run(std::false_type{});
}

}  // namespace

hipError_t launch_decode_gemm(const DecodeArgs& d, int w_dtype, int split, int small_m, int grid,
                              hipStream_t st) {
    const bool fp8 = w_dtype == MOE_E4M3;
    const int e0 = d.seg[0].epi;
    const int e1 = d.n_seg > 1 ? d.seg[1].epi : ((e0 == EPI_SWIGLU || e0 == EPI_RELU2) ? EPI_SWIGLU : EPI_F32);
    dim3 g(grid), b(kDWaves * 64);
    if (split != 1 && split != 2 && split != 4) return hipErrorInvalidValue;
    // split: wavefronts per unit
#define RDE_L(A, B, F8, S, SM, FU) hipLaunchKernelGGL((decode_gemm_kernel<A, B, F8, S, SM, FU>), g, b, 0, st, d)
#define RDE_S(A, B, F8, SM, FU)                    \
    if (split == 4) RDE_L(A, B, F8, 4, SM, FU);    \
    else if (split == 2) RDE_L(A, B, F8, 2, SM, FU); \
    else RDE_L(A, B, F8, 1, SM, FU);
    if (d.use_fused) {
        // routing inside the launch: bf16 gate/up projections only
#define RDE_DECF(A, SM) RDE_S(A, EPI_SWIGLU, false, SM, true)
        if (fp8 || e1 != EPI_SWIGLU) return hipErrorInvalidValue;
        if (e0 == EPI_SWIGLU) {
            if (small_m) { RDE_DECF(EPI_SWIGLU, true) }
            else { RDE_DECF(EPI_SWIGLU, false) }
        } else if (e0 == EPI_RELU2) {
            if (small_m) { RDE_DECF(EPI_RELU2, true) }
            else { RDE_DECF(EPI_RELU2, false) }
        } else {
            return hipErrorInvalidValue;
        }
#undef RDE_DECF
        return hipGetLastError();
    }
#define RDE_DEC4(A, B, SM)                   \
    if (fp8) { RDE_S(A, B, true, SM, false) }  \
    else { RDE_S(A, B, false, SM, false) }
#define RDE_DEC(A, B)                      \
    if (e0 == A && e1 == B) {              \
        if (small_m) { RDE_DEC4(A, B, true) } \
        else { RDE_DEC4(A, B, false) }     \
        return hipGetLastError();          \
    }
    RDE_DEC(EPI_SWIGLU, EPI_SWIGLU)
    RDE_DEC(EPI_RELU2, EPI_SWIGLU)
    RDE_DEC(EPI_COMBINE, EPI_F32)
    RDE_DEC(EPI_STORE, EPI_F32)
    RDE_DEC(EPI_F32, EPI_F32)
#undef RDE_DEC
#undef RDE_DEC4
#undef RDE_S
#undef RDE_L
    return hipErrorInvalidValue;
}

}  // namespace rde
