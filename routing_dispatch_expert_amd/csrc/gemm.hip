// Grouped expert GEMMs of the MoE layer.
//
// Expert FFN (onnxruntime PR 33963 "Description": default SwiGLU experts and
// ReLU-square gate/down experts; BF16 store boundaries with FP32
// accumulation; the fleet megakernel report's EXPERT_W13_SILU and EXPERT_W2
// tasks: gate/up projection with fused SiLU, then the down projection).
//
// Both projections are "NT" products: activations A [rows, K] and weights
// B [N, K] both have K contiguous, C = A B^T.  Rows of one expert are
// contiguous in A (count-first dispatch), so an expert's work is a run of
// m-tiles.  With `gather`, the gate/up projection reads each row of an expert
// straight from the token-ordered input (row r is token row_src[r] / k), so
// the expert-contiguous copy of the input is never written; the m-tile prefix over experts (mt_off, built on the device by the
// dispatch) maps a tile index to its expert with a binary search in LDS.
// Empty experts own no tiles; an overflowing expert owns ceil(C / BM).  The
// grid is persistent: each workgroup strides over tile indices, so the grid
// never depends on the routing and no host synchronisation is needed.
//
// bf16 kernel: 512 threads = 8 waves, block tile BM x BN x BK =
// 256 x 256 x 64, wave tile 128 x 64 = 4 x 2 MFMA v_mfma_f32_32x32x16_bf16
// blocks, one workgroup per CU.  Operands go straight from global memory to
// a 2-stage LDS ring of 64 KB stages (global_load_lds_dwordx4): each operand
// row of a k-tile is one whole 128-byte line, requested once, and one
// k-tile (64 KB) is in flight while the other is multiplied, one barrier
// per k-tile; an XOR chunk swizzle keeps the fragment reads free of bank
// conflicts.  The ring runs on across the tiles of a workgroup (the next
// tile's first k-tile loads during the current tile's last one).
//
// Tiles of at most 64 rows (light experts: mostly weight streaming) use
// another layout of the same LDS: 3 stages of 40 KB (8 KB of A rows, 32 KB of
// weights), so two k-tiles of weights are in flight instead of one; the ring
// runs on across tiles of the same layout and restarts at a change.  (Tiles
// of 33 to 64 rows went from 170 to 120 us in the gate/up GEMM of the skewed
// workload with it.)  In a batch that mixes experts of at most 32 rows with
// heavy ones (more than 256 rows), the
// workgroups of odd XCDs take their tiles in descending order, so that while
// half the chip multiplies heavy experts' tiles (MFMA-bound) the other half
// streams light experts' weights (HBM-bound).  Either change alone measured
// no faster on the skewed workload; both together took it from 3838 to 3505
// us per layer.  Rows of a tile past the end of its
// expert cost neither loads (16-row groups) nor MFMAs (32-row blocks).  bf16
// results are regrouped in a small per-wave LDS patch so that stores write
// 64 contiguous bytes per row.
//
// SwiGLU needs gate and up of the same output column in the same lane: the
// B tile of a wave column holds 32 gate rows then the 32 matching up rows,
// so acc[.][0] and acc[.][1] hold g and u of identical (row, column); a
// 256-row B tile yields 128 output columns.
//
// e4m3 weights stay e4m3 in LDS and are widened to bf16 exactly when a
// fragment is read (the hardware converts OCP e4m3 to float32; every e4m3
// value is a bf16 value); the per-row scale multiplies the float32
// accumulator.  Their k-tiles are 64 wide, so that a weight row still
// arrives in 64-byte pieces and a tile takes half as many k-tiles: the ring
// then has 3 stages of 48 KB, and the epilogue's output patch borrows the
// ring slot of the k-tile just multiplied.
#include <type_traits>

#include "common.h"

namespace rde {
namespace {

constexpr int BM = kGemmBM, BN = 256, BK = 32;
constexpr int kMaxGroupsLds = 1024;

// Largest g with s_mt[g] * nt <= L (s_mt non-decreasing, s_mt[0] = 0).
__device__ __forceinline__ int find_group(const int32_t* s_mt, int n_groups, int64_t L, int nt) {
    int lo = 0, hi = n_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)s_mt[mid] * nt <= L) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}


// ---- bf16 MFMA kernel --------------------------------------------------------
// Block tile BM x BN x BK = 256 x 256 x 32, 8 waves, a ring of kStages LDS
// stages filled by direct global -> LDS loads (global_load_lds_dwordx4: lane l
// of a wave writes the 16 bytes it loads to LDS base + 16*l).  kStages - 1
// k-tiles are in flight while one is multiplied; one barrier per k-tile.
// (e4m3 weights: 64-wide k-tiles in a ring of 3 stages, 2 in flight.)
//
// Each tile walks K starting at a rotated k-tile (see `rot` below).
//
// LDS rows of a bf16 stage are 64 bytes (4 chunks of 16 B).  Chunk c of row r
// is stored at chunk slot c ^ swz(r), swz(r) = (r1 ^ r3) | r2 << 1 (r_i = bit i
// of r): 8 consecutive rows reading one logical chunk hit 8 distinct 16-byte
// slots modulo 128 bytes, and 16 consecutive rows hit 16 distinct slots
// modulo 256 bytes, so the fragment reads are free of bank conflicts whether
// the LDS serves 8 or 16 lanes of a ds_read_b128 per clock.  A DMA block of one
// wave instruction is 16 rows x 64 B; lane l fills row l/4, slot l%4 and so
// loads the row's logical chunk (l%4) ^ swz(row).
//
// e4m3 k-tiles are 64 wide: a B row is 64 e4m3 bytes in the same swizzled
// 64-byte layout, and A holds two such 64-byte halves (k 0..31, k 32..63)
// one after the other.
constexpr int A_STAGE = BM * BK * 2;          // bytes of one 64-byte-row A half (16 KB)
constexpr int B_STAGE = BN * 64;              // 256 rows x 64 B (16 KB)
constexpr int W_STAGE = BM * 128;             // bf16: 256 rows x 128 B (one operand, 32 KB)
constexpr int kOutPitch = 80;                 // bytes per row of a wave's 32 x 32 bf16 output patch

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 1 | (((r >> 2) & 1) << 1); }
// 128-byte rows (bf16 k-tiles): chunk c of row r at slot c ^ swz8(r).  8
// consecutive rows reading one logical chunk hit 8 distinct slots, and 16
// consecutive rows hit 16 distinct 16-byte positions of a 256-byte bank
// window (rows r and r + 8 differ in bit 0 of the slot, and odd rows start
// 128 bytes in), so the fragment reads are free of bank conflicts whether
// the LDS serves 8 or 16 lanes of a ds_read_b128 per clock.  swz8 depends on
// bits 0..3 of the row only.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// LDS byte address of a __shared__ object (32-bit, as the hardware sees it).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// One direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at LDS address `lds` + 16*l; `lds` must be wave-uniform.
// Written as inline assembly so that the compiler's wait-count pass, which
// cannot tell the ring's stages apart, does not drain every in-flight load
// before each LDS read: the k-loop orders the ring itself with an explicit
// vmcnt wait and a barrier.  M0 (the LDS base register of the instruction)
// is saved and restored around the load.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
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

// The same for 4 bytes per lane (global_load_lds_dword): lane l's dword
// lands at `lds` + 4*l.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(lds)
        : "memory");
}

// Wait until at most N of this thread's vector-memory operations are
// outstanding, then workgroup barrier.  No memory fence: LDS written by
// global_load_lds is complete once the issuing thread's vmcnt has dropped
// past it.
template <int N>
__device__ __forceinline__ void waitcnt_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with a count known only at run time (0 .. 16).
__device__ __forceinline__ void wait_barrier_dyn(int n) {
    switch (n) {
        case 1: waitcnt_barrier<1>(); break;
        case 2: waitcnt_barrier<2>(); break;
        case 3: waitcnt_barrier<3>(); break;
        case 4: waitcnt_barrier<4>(); break;
        case 5: waitcnt_barrier<5>(); break;
        case 6: waitcnt_barrier<6>(); break;
        case 7: waitcnt_barrier<7>(); break;
        case 8: waitcnt_barrier<8>(); break;
        case 9: waitcnt_barrier<9>(); break;
        case 10: waitcnt_barrier<10>(); break;
        case 11: waitcnt_barrier<11>(); break;
        case 12: waitcnt_barrier<12>(); break;
        case 13: waitcnt_barrier<13>(); break;
        case 14: waitcnt_barrier<14>(); break;
        case 15: waitcnt_barrier<15>(); break;
        case 16: waitcnt_barrier<16>(); break;
        default: waitcnt_barrier<0>(); break;   // never smaller than needed
    }
}

// Wave tile 128 x 64: wave (wm, wn) owns the 32-row blocks wm, wm+2, wm+4,
// wm+6 (interleaved, so a half-filled tile keeps both M-waves busy) and B
// rows wn*64 .. wn*64+63.  wm = wave / 4: the waves of a workgroup are dealt
// round-robin over the 4 SIMDs of the CU, so on a tile of at most 32 rows
// (where only wm = 0 has MFMA work) the 4 busy waves have a SIMD each.  The MFMA is issued as B x A^T so each lane ends
// with 4 consecutive output columns of one row: for acc register r of a
// 32x32 block, row = lane % 32, column = 8*(r/4) + 4*(lane/32) + r%4.
//
// NW is the number of waves (2 x NW/2).  NW = 4 gives 128 x 128 wave tiles
// (a third fewer LDS fragment reads per MFMA); with one wave per SIMD and no
// explicit fragment double-buffering it measured slower than NW = 8 at every
// batch size, so only NW = 8 is built.  With NW = 4 every A row group of a
// tile would be loaded.
template <int EPI, bool FP8, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int NT = NW * 64;                  // threads
    constexpr bool WIDE = !FP8;                  // bf16: 128-byte operand rows (64 k per k-tile)
    constexpr int BKT = 64;                      // k per k-tile
    constexpr int AM = WIDE ? 1 : BKT / BK;      // A pieces per k-tile (e4m3: two 64-byte halves)
    constexpr int STG = FP8 ? 3 : 2;             // ring stages (3 x 48 KB or 2 x 64 KB)
    constexpr int A_ST = WIDE ? W_STAGE : AM * A_STAGE;   // bytes of one A stage
    constexpr int B_ST = WIDE ? W_STAGE : B_STAGE;        // bytes of one B stage
    constexpr int RB = WIDE ? 128 : 64;          // LDS bytes per operand row
    constexpr int DR = 1024 / RB;                // rows per DMA instruction: 8 or 16
    constexpr int WB = FP8 ? 1 : 2;              // weight bytes per element
    constexpr bool OUT_IN_RING = FP8;            // epilogue patch in the ring slot just used
    constexpr int BW = BN / (NW / 2);            // B rows (wave tile columns) per wave: 64 or 128
    constexpr int NBW = BW / 32;                 // 32-column MFMA blocks per wave: 2 or 4
    constexpr int LB = BN / DR / NW;             // B DMA instructions per thread per k-tile
    constexpr int GA = BM / DR / NW;             // A row groups (DR rows) per wave: 2 or 4
    static_assert(!OUT_IN_RING || NW * 32 * kOutPitch <= A_ST, "output patch fits in an A stage");
    static_assert(!WIDE || NW == 8, "the 128-byte-row plan is laid out for 8 waves");
    // bf16 ring layouts in one arena: 2 stages of 64 KB (A 32 KB, then B 32 KB)
    // for tiles of more than 64 rows, 3 stages of 40 KB (A 8 KB for at most 64
    // rows, then B 32 KB) for lighter tiles, which then keep two k-tiles of
    // weights in flight instead of one.  e4m3: 3 stages, the A stages first.
    constexpr int LSTG = 3, LSTAGE = 8192 + W_STAGE;
    constexpr int RING_BYTES = WIDE ? 2 * 2 * W_STAGE : STG * (A_ST + B_ST);
    static_assert(!WIDE || LSTG * LSTAGE <= RING_BYTES, "light stages fit the arena");
    __shared__ __attribute__((aligned(1024))) unsigned char sRing[RING_BYTES];
    // stage bases; the layout (light or not) is a compile-time argument
    auto slotA = [&](auto lt_c, int slot) -> unsigned char* {
        constexpr bool LT = decltype(lt_c)::value;
        if (!WIDE) return sRing + slot * A_ST;
        return sRing + (LT ? slot * LSTAGE : slot * 2 * W_STAGE);
    };
    auto slotB = [&](auto lt_c, int slot) -> unsigned char* {
        constexpr bool LT = decltype(lt_c)::value;
        if (!WIDE) return sRing + STG * A_ST + slot * B_ST;
        return sRing + (LT ? slot * LSTAGE + 8192 : slot * 2 * W_STAGE + W_STAGE);
    };
    using Heavy = std::false_type;
    using Light = std::true_type;
    __shared__ int32_t s_mt[kMaxGroupsLds + 1], s_off[kMaxGroupsLds + 1];
    __shared__ __attribute__((aligned(16))) unsigned char sOut[OUT_IN_RING ? 1 : NW][OUT_IN_RING ? 16 : 32 * kOutPitch];
    // EPI_COMBINE: the tile's routes and their weights, loaded during the
    // k-loop by direct-to-LDS loads (plain loads in the epilogue would wait
    // for every k-tile of the next tile already in flight)
    __shared__ int32_t s_rq[EPI == EPI_COMBINE ? BM : 1];
    __shared__ float s_rw[EPI == EPI_COMBINE ? BM : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / (NW / 2), wn = wave % (NW / 2);
    const bool uniform = a.mt_off == nullptr;
    int total_mt, tiles_per_group = 0;
    if (uniform) {
        tiles_per_group = (a.uniform_rows + BM - 1) / BM;
        total_mt = tiles_per_group * a.n_groups;
    } else {
        for (int i = tid; i <= a.n_groups; i += NT) {
            s_mt[i] = a.mt_off[i];
            s_off[i] = a.offsets[i];   // row ranges: LDS reads in the tile set-up
        }
        __syncthreads();
        total_mt = s_mt[a.n_groups];
    }
    const int ntl = a.n_tiles;
    const int64_t total = (int64_t)total_mt * ntl;
    // a batch mixing light experts (at most 32 rows: weight streaming) with
    // heavy ones (more than 256 rows: MFMA-bound)
    bool mixed = false;
    if (WIDE && !uniform) {
        int lt = 0, hv = 0;
        for (int i = tid; i < a.n_groups; i += NT) {
            const int n = s_off[i + 1] - s_off[i];
            lt |= n > 0 && n <= 32;
            hv |= n > 256;
        }
        mixed = __syncthreads_or(lt) && __syncthreads_or(hv);
    }

    // Tiles are ordered (group, n-tile, m-tile) with the m-tile fastest, and
    // consecutive tile indices go to workgroups of one XCD (workgroups are
    // dealt round-robin over the 8 XCDs): the m-tiles sharing a weight tile
    // and the n-tiles sharing activation rows meet in the same L2.
    const int G = gridDim.x;
    const int vid = ((G & 7) == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;

    const char* Ab = (const char*)a.A;
    const char* Bb = (const char*)a.B;
    const int nk = a.K / BKT;

    // DMA plan.  A: wave w fills the DR-row groups w + NW*i (row DR*group +
    // lane/(RB/16)), i < GA; with 8 waves a group wholly past the expert's
    // last row is not loaded, so a half-filled tile issues half the A traffic
    // and every wave keeps A groups while rows > 128; e4m3 k-tiles load each
    // 16-row group twice (both 64-byte halves).  B: wave w fills rows
    // w*DR*LB + DR*b + lane/(RB/16) (b < LB): 128 bytes per row (64 bf16), or
    // 64 (64 e4m3).
    const int dr = WIDE ? (lane >> 3) : (lane >> 2), ds = WIDE ? (lane & 7) : (lane & 3);
    auto swzr = [](int r) { return WIDE ? swz8(r) : swz(r); };

    // wave-uniform LDS bases of this wave's DMA blocks in ring slot 0
    const uint32_t rq0 = __builtin_amdgcn_readfirstlane(lds_addr(s_rq) + wave * 256);
    // this wave's DMA bases in the arena (wave-uniform); a stage adds its offset
    const uint32_t la0 = __builtin_amdgcn_readfirstlane(lds_addr(sRing) + wave * 1024);
    const uint32_t lb0 = __builtin_amdgcn_readfirstlane(lds_addr(sRing) + wave * LB * 1024);
    const uint32_t rw0 = __builtin_amdgcn_readfirstlane(lds_addr(s_rw) + wave * 256);
    // routes of the epilogue staged in LDS: needs k-tiles 1, 5 and 9 (see the k-loop)
    const bool route_pf = EPI == EPI_COMBINE && nk >= 10;
    static_assert(!WIDE || GA * NW * DR == BM, "A row groups cover the tile");

    // A tile's place in the problem and this thread's DMA sources (byte
    // offsets at k = 0).  la = A groups this wave loads (0 .. GA).
    // bf16 (128-byte rows): only the A row indices and the B row base depend on
    // the tile; the chunk offsets depend on the lane alone (every A group of a
    // wave shares one swizzle, and B rows alternate between two), and a wave's
    // B rows are consecutive weight rows, so instruction b adds 8 b rows.
    struct Tile {
        int g, nt, a_row0, rows, rot, la, lbv;
        int light;              // bf16 tile of at most 64 rows: the 3-stage light layout
        int64_t ga[WIDE ? 1 : GA];
        int32_t ar[WIDE ? GA : 1];
        int64_t gbase;          // the expert's weights (wave-uniform)
        uint32_t gb[WIDE ? 1 : LB];   // per-lane weight offsets within them (bf16: row base)
    };
    const uint32_t a_chunk = (uint32_t)(ds ^ swz8(8 * wave + dr)) * 16;
    const uint32_t b_chunk = (uint32_t)(ds ^ swz8(32 * wave + dr)) * 16;
    auto make_tile = [&](int64_t Lt) {
        Tile t;
        int cnt, ml;
        if (uniform) {
            t.g = (int)(Lt / ((int64_t)tiles_per_group * ntl));
            const int loc = (int)(Lt - (int64_t)t.g * tiles_per_group * ntl);
            cnt = tiles_per_group;
            t.nt = loc / cnt;
            ml = loc - t.nt * cnt;
            t.a_row0 = ml * BM;
            t.rows = min(BM, a.uniform_rows - t.a_row0);
        } else {
            t.g = __builtin_amdgcn_readfirstlane(find_group(s_mt, a.n_groups, Lt, ntl));
            cnt = s_mt[t.g + 1] - s_mt[t.g];
            const int loc = (int)(Lt - (int64_t)s_mt[t.g] * ntl);
            t.nt = loc / cnt;
            ml = loc - t.nt * cnt;
            // an expert's n rows are spread evenly over its cnt = ceil(n / BM)
            // m-tiles, so that a remainder of a few rows does not get a tile
            // of its own that streams the whole weight tile for almost no
            // MFMA work.  per = ceil(n / cnt) <= BM, rounded up to whole
            // 32-row MFMA blocks while the last tile keeps at least one row;
            // (cnt - 1) per < n <= cnt per either way
            const int e0 = s_off[t.g], e1 = s_off[t.g + 1], n = e1 - e0;
            int per = (n + cnt - 1) / cnt;
            const int p32 = (per + 31) & ~31;
            if (p32 <= BM && (cnt - 1) * p32 < n) per = p32;
            t.a_row0 = e0 + ml * per;
            t.rows = min(per, e1 - t.a_row0);
        }
        const int g = t.g, nt = t.nt, rows = t.rows;
        // B row r of the tile: for SwiGLU each wave's BW rows are BW/2 gate
        // rows and the matching BW/2 up rows
        auto brow_of = [&](int r) {
            if (EPI == EPI_SWIGLU) {
                const int w2 = r / BW, rr = r % BW;
                return (rr < BW / 2) ? (nt * 128 + w2 * (BW / 2) + rr)
                                     : (a.I + nt * 128 + w2 * (BW / 2) + rr - BW / 2);
            }
            return min(nt * BN + r, a.N_w - 1);   // rows past N (ragged last tile): clamped
        };
        // A rows: with gather, the tokens of the tile's routes, all looked up
        // before any is used (one wait for the lookups)
        int64_t ar[GA];
#pragma unroll
        for (int i = 0; i < GA; ++i) ar[i] = t.a_row0 + min((wave + NW * i) * DR + dr, rows - 1);
        if (a.gather) {
            int32_t q[GA];
#pragma unroll
            for (int i = 0; i < GA; ++i) q[i] = a.row_src[ar[i]];
#pragma unroll
            for (int i = 0; i < GA; ++i) ar[i] = q[i] / a.k_top;
        }
        t.gbase = (int64_t)g * a.b_group_stride * WB;
        if (WIDE) {
#pragma unroll
            for (int i = 0; i < GA; ++i) t.ar[i] = (int32_t)ar[i];
            // B rows wave*32 .. +31 (every one of them past N_w in a wave that
            // loads none: N_w is a multiple of 128)
            t.gb[0] = (uint32_t)brow_of(wave * 32 + dr) * (uint32_t)a.k_seg * WB;
            t.lbv = EPI == EPI_SWIGLU || nt * BN + wave * 32 < a.N_w;
        } else {
#pragma unroll
            for (int i = 0; i < GA; ++i) {
                const int ra = (wave + NW * i) * DR + dr;
                t.ga[i] = ar[i] * a.lda * 2 + ((ds ^ swzr(ra)) * 16);
            }
#pragma unroll
            for (int b = 0; b < LB; ++b) {
                const int rb = wave * DR * LB + DR * b + dr;
                t.gb[b] = (uint32_t)brow_of(rb) * (uint32_t)a.k_seg * WB + ((ds ^ swzr(rb)) * 16);
            }
            t.lbv = 1;
        }
        // K order: the tile starts at k-tile `rot` and wraps.  Tiles of
        // different experts running at the same time then read different
        // column offsets of their rows, so weight rows with a power-of-two
        // stride do not all land on the same memory channels.  The n-tiles of
        // one expert share the rotation: they walk the expert's activation
        // rows in the same order at about the same time, so those rows are
        // fetched into L2 once and reused.  rot depends only on the expert, so
        // a row's summation order never depends on the other tokens.
        t.rot = (g * 13) % nk;
        t.light = WIDE && rows <= 64;
        if (WIDE) {
            int la = 0;
#pragma unroll
            for (int i = 0; i < GA; ++i) la += DR * (wave + NW * i) < rows;
            t.la = __builtin_amdgcn_readfirstlane(la);
        } else {
            t.la = NW == 8 ? __builtin_amdgcn_readfirstlane((16 * wave < rows) + (16 * (wave + 8) < rows)) : GA;
        }
        return t;
    };
    // Load k-tile s (in the tile's own K order) of tile t into ring slot `slot`.
    auto issue = [&](auto lt_c, const Tile& t, int s, int slot, int part = -1) {
        int kr = s + t.rot;
        if (kr >= nk) kr -= nk;
        const int k0 = kr * BKT;
        const int seg = k0 / a.k_seg;
        const int64_t bo = (int64_t)seg * a.b_seg_stride + (k0 - seg * a.k_seg);
        const uint32_t la = la0 + (uint32_t)(slotA(lt_c, slot) - sRing);
        const uint32_t lb = lb0 + (uint32_t)(slotB(lt_c, slot) - sRing);
        if (WIDE) {
#pragma unroll
            for (int i = 0; i < GA; ++i)
                if (t.la > i) dma16(Ab + (int64_t)t.ar[i] * a.lda * 2 + a_chunk + (int64_t)k0 * 2, la + i * NW * 1024);
            if (t.lbv) {
                const char* bsrc = Bb + t.gbase + bo * WB;
                const uint32_t bstep = 8u * (uint32_t)a.k_seg * WB;   // 8 weight rows
#pragma unroll
                for (int b = 0; b < LB; ++b)
                    dma16(bsrc + (t.gb[0] + b * bstep + ((b & 1) ? (b_chunk ^ 16u) : b_chunk)), lb + b * 1024);
            }
            return;
        }
        // e4m3: part 0 the B rows, part 1 + h the A half h; -1 all of them
#pragma unroll
        for (int h = 0; h < AM; ++h)
#pragma unroll
            for (int i = 0; i < GA; ++i)
                if ((part < 0 || part == 1 + h) && t.la > i)
                    dma16(Ab + t.ga[i] + (int64_t)(k0 + h * BK) * 2, la + h * A_STAGE + i * NW * 1024);
        if (part <= 0) {
#pragma unroll
            for (int b = 0; b < LB; ++b) dma16(Bb + t.gbase + t.gb[b] + bo * WB, lb + b * 1024);
        }
    };

    // The load ring runs across tiles: while a tile's last STG - 1
    // k-tiles are multiplied, the next tile's first ones are loaded, so the
    // pipeline never drains between tiles.  Ring slot of k-tile s of a tile =
    // (sbase + s) % STG, sbase = k-tiles of this workgroup's earlier tiles (mod STG).
    // Every wait bounds the number of this thread's DMA instructions issued
    // after the awaited k-tile; other outstanding loads and stores (the
    // next tile's row lookups, the epilogue's stores) only make it stricter.
    // This workgroup's tiles are vid + i G (i < n_mine).  In a batch mixing
    // light and heavy experts the workgroups of odd XCDs take theirs in
    // descending order, so that while half the chip multiplies heavy experts'
    // tiles the other half streams light experts' weights.
    if (vid >= total) return;  // workgroup-uniform; nothing in flight
    const int64_t n_mine = (total - 1 - vid) / G + 1;
    const bool reverse = mixed && (blockIdx.x & 1);
    auto tile_at = [&](int64_t i) { return (int64_t)vid + (reverse ? n_mine - 1 - i : i) * G; };
    auto stages = [](bool light) { return FP8 ? 3 : (light ? LSTG : 2); };
    auto ringS = [](int x, int S) { return S == 2 ? (x & 1) : (int)((unsigned)x % 3u); };
    Tile cur = make_tile(tile_at(0));
    int sbase = 0;
    // first k-tiles (nk >= 2: K >= 128)
    if (cur.light) {
        for (int st = 0; st < LSTG - 1; ++st) issue(Light{}, cur, st, st);
    } else {
        for (int st = 0; st < STG - 1; ++st) issue(Heavy{}, cur, st, st);
    }

    const int rA = lane & 31, half = lane >> 5;
    // This lane's fragment rows are rA plus multiples of 32, and swz depends on
    // bits 1..3 of the row only: every row block shares the swizzle of rA, so
    // two per-lane byte offsets (logical chunk half, and 2 + half) serve all
    // of them, and the blocks differ by compile-time constants.
    const int zr = swz(rA);
    const int loff0 = rA * 64 + ((half ^ zr) * 16), loff1 = rA * 64 + (((2 + half) ^ zr) * 16);
    // 128-byte rows: step ks reads logical chunk 2 ks + half; swz8 depends on
    // bits 0..3 of the row, so the row blocks share these four offsets too
    int loffw[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) loffw[ks] = rA * 128 + (((2 * ks + half) ^ swz8(rA)) * 16);
    for (int64_t it = 0; it < n_mine; ++it) {
        const bool has_next = it + 1 < n_mine;
        const Tile nxt = has_next ? make_tile(tile_at(it + 1)) : cur;
        const int S = stages(cur.light);
        // the ring runs on into the next tile only when it has the same layout
        const bool chain = has_next && nxt.light == cur.light;
        const int lc = (cur.lbv ? LB : 0) + AM * cur.la;                // this tile's DMA count per k-tile
        const int cn = chain ? (nxt.lbv ? LB : 0) + AM * nxt.la : 0;    // and the next tile's
        const int g = cur.g, nt = cur.nt, a_row0 = cur.a_row0, rows = cur.rows;

        f32x16 acc[4][NBW];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        // active row blocks of this wave: wm + 2*mb is active iff 32*(wm + 2*mb) < rows,
        // i.e. mb < n_act (a prefix); waves whose 64 B rows lie past N (ragged last
        // n-tile) have none.  Wave-uniform, kept in a scalar register.
        const bool col_ok = EPI == EPI_SWIGLU || nt * BN + wn * BW < a.N_w;
        const int n_act = __builtin_amdgcn_readfirstlane(
            col_ok ? max(0, min(4, (rows - 32 * wm + 63) / 64)) : 0);

        // the pipelined k-loop, specialised on the number NA of active row
        // blocks of the wave's MFMAs and the number LA of A groups it loads
        auto kloop = [&](auto na_c, auto la_c, auto lt_c) {
            constexpr int NA = decltype(na_c)::value;
            constexpr int LA = decltype(la_c)::value;
            constexpr int LC = LB + AM * LA;   // this tile's DMA count per k-tile
            constexpr bool LT = decltype(lt_c)::value;
            constexpr int SS = FP8 ? 3 : (LT ? LSTG : 2);   // stages of this layout
            // ring slot of a running k-tile count (non-negative: no signed modulo)
            auto slot_of = [](int x) { return SS == 2 ? (x & 1) : (int)((unsigned)x % (unsigned)SS); };
            for (int kt = 0; kt < nk; ++kt) {
                // in flight behind k-tile kt: k-tiles kt + 1 .. kt + STG - 2, of
                // this tile or (at the end) of the next one
                if (SS == 2) {
                    // nothing is issued after k-tile kt before this wait
                    waitcnt_barrier<0>();
                } else if (FP8) {
                    if (kt + 1 < nk) waitcnt_barrier<LC>();
                    else wait_barrier_dyn(cn);
                } else {
                    // light layout: k-tile kt + 1 (this tile's, or the next tile's first) is behind it
                    wait_barrier_dyn(kt + 1 < nk ? lc : cn);
                }
                const int s = kt + SS - 1;
                // e4m3 tiles with MFMA work: the loads of k-tile kt + 2 (needed
                // two steps from now) are spread over this step's K steps, the
                // B rows first, so that no wave stalls in issue before its MFMAs
                constexpr bool SPREAD = FP8 && NA > 0;
                auto issue_part = [&](int part) {
                    if (s < nk) issue(lt_c, cur, s, slot_of(sbase + s), part);
                    else if (chain) issue(lt_c, nxt, s - nk, slot_of(sbase + s), part);
                };
                if (!SPREAD) issue_part(-1);
                if (EPI == EPI_COMBINE && route_pf && wave < 4) {
                    // waves 0..3 stage the routes of tile rows 64 wave + lane at
                    // k-tile 1 (every wave has left the previous tile's
                    // epilogue), then their weights at k-tile 5 (the routes
                    // were loaded before k-tile 5 was, so they have landed);
                    // the weights have landed by the barrier of k-tile 9
                    if (kt == 1) {
                        dma4(a.row_src + a_row0 + min(64 * wave + lane, rows - 1), rq0);
                    } else if (kt == 5) {
                        dma4(a.route_w + s_rq[64 * wave + lane], rw0);
                    }
                }
                if (NA == 0) continue;
                const int slot = slot_of(sbase + kt);
                const unsigned char* sb = slotB(lt_c, slot);
#pragma unroll
                for (int ks = 0; ks < BKT / 16; ++ks) {
                    // this lane's k = 16 ks + 8 half .. + 7: logical 16-byte chunk c
                    // of the 64-byte A half ks / 2 and of a bf16 B row; in an e4m3
                    // B row, the 8-byte piece `half` of chunk ks
                    const int lo = WIDE ? loffw[ks] : ((ks & 1) ? loff1 : loff0);   // chunk c = 2 (ks & 1) + half
                    const unsigned char* sa = slotA(lt_c, slot) + (WIDE ? 0 : (ks >> 1) * A_STAGE);
                    if (SPREAD && ks < 1 + AM) issue_part(ks);
                    bf16x8 bv[NBW], av[NA > 0 ? NA : 1];
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        const int r0 = wn * BW + nb * 32;   // row rA of this block: r0 + rA
                        if (FP8) {
                            bv[nb] = e4m3x8_to_bf16x8(*(const uint2*)(sb + (r0 + rA) * 64 + ((ks ^ zr) * 16) + half * 8));
                        } else {
                            bv[nb] = *(const bf16x8*)(sb + r0 * RB + lo);
                        }
                    }
#pragma unroll
                    for (int mb = 0; mb < NA; ++mb) {
                        av[mb] = *(const bf16x8*)(sa + (wm + 2 * mb) * 32 * RB + lo);
                    }
#pragma unroll
                    for (int mb = 0; mb < NA; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NBW; ++nb)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[nb], av[mb], acc[mb][nb], 0, 0, 0);
                    if constexpr (WIDE && NA == 4) {
                        // keep the fragment reads ahead of the MFMAs that use them
                        // (near the register limit the scheduler otherwise waits on
                        // each read): B 0-1 and A 0-1, 2 MFMAs, A 2-3, 6 MFMAs
                        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
                    } else if constexpr (NA > 0) {
                        // all of the step's reads, then its MFMAs (e4m3: the
                        // widening of the B fragments falls in between)
                        __builtin_amdgcn_sched_group_barrier(0x100, NBW + NA, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, NBW * NA, 0);
                    }
                }
            }
        };
        auto by_la = [&](auto na_c) {
            constexpr int NA = decltype(na_c)::value;
            if constexpr (WIDE) {
                // waits need no compile-time DMA count; on a light tile a
                // wave has at most one active row block
                if constexpr (NA <= 1) {
                    if (cur.light) {
                        kloop(na_c, std::integral_constant<int, 0>{}, Light{});
                        return;
                    }
                }
                kloop(na_c, std::integral_constant<int, 0>{}, Heavy{});
            } else if (NW != 8) {
                kloop(na_c, std::integral_constant<int, GA>{}, Heavy{});   // every A group loaded
            } else if (cur.la == 2) {
                kloop(na_c, std::integral_constant<int, 2>{}, Heavy{});
            } else if (cur.la == 1) {
                kloop(na_c, std::integral_constant<int, 1>{}, Heavy{});
            } else {
                kloop(na_c, std::integral_constant<int, 0>{}, Heavy{});
            }
        };
        switch (n_act) {
            case 4: by_la(std::integral_constant<int, 4>{}); break;
            case 3: by_la(std::integral_constant<int, 3>{}); break;
            case 2: by_la(std::integral_constant<int, 2>{}); break;
            case 1: by_la(std::integral_constant<int, 1>{}); break;
            default: by_la(std::integral_constant<int, 0>{}); break;
        }

        // ---- epilogue: lane owns row (lane % 32) of each active row block and
        // columns 8*i + 4*(lane/32) + 0..3 of each 32-column block.  bf16
        // results pass through the wave's own LDS patch, so that each store
        // instruction writes 16 rows x 64 contiguous bytes instead of 16-byte
        // pieces of 32 rows; float32 results are stored directly ----
        const int c4 = 4 * (lane >> 5);
        unsigned char* so;
        if (OUT_IN_RING) {
            // every wave has read its last fragments of the k-tile just
            // multiplied (its LDS reads are complete before the barrier); its
            // slot is refilled only after the next tile's first barrier
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            so = slotA(Heavy{}, ringS(sbase + nk - 1, S)) + wave * 32 * kOutPitch;
        } else {
            so = sOut[wave];
        }
        const int sr = lane >> 2, sq = lane & 3;   // store phase: row (of 16), 16-byte chunk
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (mb >= n_act) continue;
            const int rb = (wm + 2 * mb) * 32;
            const int row = rb + (lane & 31);
            // lanes past the expert's last row compute on a valid row and store nothing
            const int64_t orow = (int64_t)a_row0 + min(row, rows - 1);
            if (EPI == EPI_F32) {
                if (row >= rows) continue;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int col = nt * BN + wn * BW + nb * 32 + 8 * i + c4;
                        float v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            v[j] = acc[mb][nb][4 * i + j];
                            if (FP8) v[j] *= a.bscale[(int64_t)g * a.N_w + col + j];
                        }
                        *(float4*)((float*)a.out + orow * a.ldo + col) = make_float4(v[0], v[1], v[2], v[3]);
                    }
                continue;
            }
            float cw = 1.0f;
            int32_t q = 0;
            if (EPI == EPI_COMBINE) {
                if (route_pf) {
                    q = s_rq[min(row, rows - 1)];
                    cw = s_rw[min(row, rows - 1)];
                } else {
                    q = a.row_src[orow];
                    cw = a.route_w[q];
                }
            }
            // SwiGLU: gate block nb pairs with up block nb + NBW/2
            constexpr int NB = EPI == EPI_SWIGLU ? NBW / 2 : NBW;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // one 32 x 32 block at a time: the scheduler may not hoist the
                // accumulator reads of later blocks (they would all be live)
                __builtin_amdgcn_sched_barrier(0);
                // output columns of this 32-column block
                const int col0 = EPI == EPI_SWIGLU ? nt * 128 + wn * (BW / 2) + nb * 32 : nt * BN + wn * BW + nb * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = col0 + 8 * i + c4;
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (EPI == EPI_SWIGLU) {
                            float gv = acc[mb][nb][4 * i + j], uv = acc[mb][nb + NBW / 2][4 * i + j];
                            if (FP8) {
                                gv *= a.bscale[(int64_t)g * a.N_w + col + j];
                                uv *= a.bscale[(int64_t)g * a.N_w + a.I + col + j];
                            }
                            v[j] = silu_mul(gv, uv);
                        } else {
                            v[j] = acc[mb][nb][4 * i + j];
                            if (FP8) v[j] *= a.bscale[(int64_t)g * a.N_w + col + j];
                            if (EPI == EPI_RELU2) v[j] = v[j] > 0.0f ? v[j] * v[j] : 0.0f;
                            if (EPI == EPI_COMBINE) v[j] *= cw;
                        }
                    }
                    *(uint2*)(so + (lane & 31) * kOutPitch + (8 * i + c4) * 2) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
                // the wave's LDS operations run in order: the reads below see
                // the writes above, and the next block's writes follow them
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int r = sr + 16 * j;
                    const uint4 u = *(const uint4*)(so + r * kOutPitch + sq * 16);
                    int64_t drow = (int64_t)a_row0 + rb + r;
                    if (EPI == EPI_COMBINE) drow = __shfl(q, r, kWave);
                    const int64_t oc = (EPI == EPI_SWIGLU || EPI == EPI_RELU2)
                                           ? (int64_t)g * a.out_col_per_group + col0 + sq * 8
                                           : col0 + sq * 8;
                    if (rb + r < rows) *(uint4*)((__bf16*)a.out + drow * a.ldo + oc) = u;
                }
            }
        }
        if (!has_next) break;
        if (chain) {
            sbase = ringS(sbase + nk, S);
        } else {
            // the next tile takes the other layout and nothing of it was
            // issued: once every wave is past its last reads of this tile's
            // stages, its first k-tiles start a fresh ring
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            sbase = 0;
            if (nxt.light) {
                for (int st = 0; st < LSTG - 1; ++st) issue(Light{}, nxt, st, st);
            } else {
                for (int st = 0; st < STG - 1; ++st) issue(Heavy{}, nxt, st, st);
            }
        }
        cur = nxt;
    }
}

// ---- float32 kernel (float32 activations and weights) -----------------------
// 64 x 64 output block per tile, BK = 16, 256 threads each computing 4 rows x
// 4 B-columns {2tx, 2tx+1, 32+2tx, 33+2tx}.  For SwiGLU the 64 B rows of a
// tile are 32 gate rows then the matching 32 up rows (32 output columns).
constexpr int FBM = kGemmF32BM, FBN = 64, FBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
    __shared__ float sA[FBK][FBM + 4];
    __shared__ float sB[FBK][FBN + 4];
    __shared__ int32_t s_mt[kMaxGroupsLds + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const bool uniform = a.mt_off == nullptr;
    int total_mt, tiles_per_group = 0;
    if (uniform) {
        tiles_per_group = (a.uniform_rows + FBM - 1) / FBM;
        total_mt = tiles_per_group * a.n_groups;
    } else {
        for (int i = tid; i <= a.n_groups; i += blockDim.x) s_mt[i] = a.mt_off[i];
        __syncthreads();
        total_mt = s_mt[a.n_groups];
    }
    const int64_t total = (int64_t)total_mt * a.n_tiles;
    const float* A = (const float*)a.A;
    const float* B = (const float*)a.B;
    for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = (int)(tile / a.n_tiles);
        const int nt = (int)(tile - (int64_t)mt * a.n_tiles);
        int g, rows, a_row0;
        if (uniform) {
            g = mt / tiles_per_group;
            a_row0 = (mt - g * tiles_per_group) * FBM;
            rows = min(FBM, a.uniform_rows - a_row0);
        } else {
            g = find_group(s_mt, a.n_groups, mt, 1);
            const int e0 = a.offsets[g], e1 = a.offsets[g + 1];
            a_row0 = e0 + (mt - s_mt[g]) * FBM;
            rows = min(FBM, e1 - a_row0);
        }
        // loads: A row lr = tid/4, k chunk 4*(tid%4); B row lr likewise
        const int lr = tid >> 2, lk = (tid & 3) * 4;
        const int arow = a_row0 + (lr < rows ? lr : rows - 1);
        int brow;
        if (EPI == EPI_SWIGLU) brow = lr < 32 ? nt * 32 + lr : a.I + nt * 32 + lr - 32;
        else brow = nt * FBN + lr;
        const float* bp = B + (int64_t)g * a.b_group_stride + (int64_t)brow * a.k_seg;
        float acc[4][4] = {};
        for (int k0 = 0; k0 < a.K; k0 += FBK) {
            const int seg = k0 / a.k_seg, kl = k0 - seg * a.k_seg;
            const float4 va = *(const float4*)(A + (int64_t)arow * a.lda + k0 + lk);
            const float4 vb = *(const float4*)(bp + (int64_t)seg * a.b_seg_stride + kl + lk);
            __syncthreads();
            sA[lk + 0][lr] = va.x; sA[lk + 1][lr] = va.y; sA[lk + 2][lr] = va.z; sA[lk + 3][lr] = va.w;
            sB[lk + 0][lr] = vb.x; sB[lk + 1][lr] = vb.y; sB[lk + 2][lr] = vb.z; sB[lk + 3][lr] = vb.w;
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < FBK; ++kk) {
                float av[4], bv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
                bv[0] = sB[kk][2 * tx];
                bv[1] = sB[kk][2 * tx + 1];
                bv[2] = sB[kk][32 + 2 * tx];
                bv[3] = sB[kk][33 + 2 * tx];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = ty * 4 + i;
            if (row >= rows) continue;
            const int64_t orow = a_row0 + row;
            float* out = (float*)a.out;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = nt * 32 + 2 * tx + j;
                    const float gt = acc[i][j], up = acc[i][j + 2];
                    out[orow * a.ldo + (int64_t)g * a.out_col_per_group + col] =
                        gt / (1.0f + expf(-gt)) * up;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = nt * FBN + (j < 2 ? 2 * tx + j : 32 + 2 * tx + (j - 2));
                    const float v = acc[i][j];
                    if (EPI == EPI_RELU2) {
                        out[orow * a.ldo + (int64_t)g * a.out_col_per_group + col] = v > 0.0f ? v * v : 0.0f;
                    } else if (EPI == EPI_STORE || EPI == EPI_F32) {
                        out[orow * a.ldo + col] = v;
                    } else {  // EPI_COMBINE
                        const int32_t q = a.row_src[orow];
                        out[(int64_t)q * a.ldo + col] = a.route_w[q] * v;
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int w_dtype, int grid, hipStream_t s) {
    const bool fp8 = w_dtype == MOE_E4M3;
#define RDE_GEMM_CASE(E)                                                                                  \
    case E:                                                                                               \
        if (fp8) hipLaunchKernelGGL((gemm_bf16_kernel<E, true, 8>), dim3(grid), dim3(512), 0, s, a);      \
        else hipLaunchKernelGGL((gemm_bf16_kernel<E, false, 8>), dim3(grid), dim3(512), 0, s, a);         \
        break;
    switch (a.epi) {
        RDE_GEMM_CASE(EPI_SWIGLU)
        RDE_GEMM_CASE(EPI_RELU2)
        RDE_GEMM_CASE(EPI_STORE)
        RDE_GEMM_CASE(EPI_COMBINE)
        RDE_GEMM_CASE(EPI_F32)
        default: return hipErrorInvalidValue;
    }
#undef RDE_GEMM_CASE
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, int grid, hipStream_t s) {
    switch (a.epi) {
        case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, dim3(grid), dim3(256), 0, s, a); break;
        case EPI_RELU2: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RELU2>, dim3(grid), dim3(256), 0, s, a); break;
        case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, dim3(grid), dim3(256), 0, s, a); break;
        case EPI_COMBINE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_COMBINE>, dim3(grid), dim3(256), 0, s, a); break;
        case EPI_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_F32>, dim3(grid), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rde
