// Internal declarations of the gfx950 MoE library: vector types, small
// device helpers and the kernel launchers called by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace rde {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWave = 64;

// Two floats -> two bf16 (round to nearest even) in one packed dword, low
// half first: a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// 8 OCP e4m3 codes (two dwords, lowest byte first) -> 8 bf16, exact: every
// e4m3 value is a bf16 value.  gfx950 converts a pair of e4m3 codes straight
// to a pair of bf16 (v_cvt_scalef32_pk_bf16_fp8; the scale 1.0 leaves the
// values unchanged), 4 instructions for 8 weights.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint2 v) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
    const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
    return __builtin_bit_cast(bf16x8, u);
}

// ---- workspace control words (first 256 bytes of ws) --------------------
enum CtrlWord {
    CTRL_BAD_ROUTES = 0,   // malformed routes seen since the last moe_error
    CTRL_TICKET = 1,       // arrival counter of the count kernel's blocks
    CTRL_WORDS = 64
};

// ---- count-first dispatch ------------------------------------------------
// Routes per block of the count/rank kernel: 4 waves x 8 routes per lane.
constexpr int kCountWaves = 4;
constexpr int kCountPerLane = 8;
constexpr int kCountBlock = kWave * kCountWaves * kCountPerLane;   // 2048

inline int count_blocks(int64_t Q) { return (int)((Q + kCountBlock - 1) / kCountBlock); }

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int score_func, int renorm, float scale, int32_t* ids, float* w,
                        hipStream_t s);

// ids -> rexp (validated expert or -2), lrank (rank inside its block),
// partial (per-block counts, turned into per-block bases by the last block),
// counts, offsets and the m-tile table of the grouped GEMM (tile rows bm).
// With route_dst given and at most kCountBlock routes (one block), the kernel
// also places the routes (route_dst, row_src with -1 from the kept rows up to
// r_max), so no metadata scatter is needed.
// local_scan (several blocks, local_scan_fits): the blocks only publish
// their totals in partial and launch_scatter_scan does the rest.
hipError_t launch_count_rank(const int32_t* ids, int T, int k, int E, int C, int bm,
                             int32_t* rexp, int32_t* lrank, int32_t* partial,
                             int32_t* counts, int32_t* offsets, int32_t* mt_off,
                             int32_t* ctrl, hipStream_t s, int32_t* route_dst = nullptr,
                             int32_t* row_src = nullptr, int64_t r_max = 0, int local_scan = 0);

// Several count blocks whose per-block totals (blocks x experts words) are
// few enough for every block of the metadata scatter to scan them itself:
// the count kernel then needs no hand-off between its blocks (its ticket,
// the write-through totals and the last block's scan cost more than each
// scatter block reading the totals from L2: 16384 routes over 128 experts,
// count 11.8 -> 8.0 us, metadata scatter 3.8 -> 4.1 us).
constexpr int kLocalScanMax = 2048;
inline bool local_scan_fits(int64_t Q, int E) {
    const int nb = count_blocks(Q);
    return nb > 1 && (int64_t)nb * E <= kLocalScanMax;
}
// After launch_count_rank(..., local_scan = 1), for the expert GEMMs that
// read rows in place: per-block bases, counts, offsets, the m-tile table
// (tile rows bm), route_dst and row_src (-1 from the kept rows up to r_max).
hipError_t launch_scatter_scan(int T, int k, int E, int C, int bm, int64_t r_max, const int32_t* rexp,
                               const int32_t* lrank, const int32_t* cnt, int32_t* counts, int32_t* offsets,
                               int32_t* mt_off, int32_t* route_dst, int32_t* row_src, hipStream_t s);

// At most kPlaceMaxQ routes: one 1024-thread workgroup ranks every route,
// writes counts, offsets and the m-tile table, and places every route
// (route_dst, row_src with -1 past the kept rows); no cross-block hand-off.
// Above it the chain of 64-route ranking steps of one workgroup costs more
// than the hand-off (measured: 16384 routes 34 against 21 us with the
// multi-block kernel and its scatter launch; 2048 routes 13.6 against 18.5).
constexpr int64_t kPlaceMaxQ = 4096;
hipError_t launch_count_place(const int32_t* ids, int T, int k, int E, int C, int bm,
                              int32_t* counts, int32_t* offsets, int32_t* mt_off, int32_t* row_src,
                              int64_t r_max, int32_t* route_dst, int32_t* ctrl, hipStream_t s);
// x -> x_disp copies of routes already placed (route_dst).
hipError_t launch_copy_rows(const void* x, int T, int H, int k, int elem_bytes, const int32_t* route_dst,
                            void* x_disp, hipStream_t s);

// route_dst, row_src and the x -> x_disp row copies.
hipError_t launch_scatter(const void* x, int T, int H, int k, int E, int C, int elem_bytes,
                          int64_t r_max, const int32_t* rexp, const int32_t* lrank,
                          const int32_t* base, const int32_t* offsets,
                          int32_t* route_dst, int32_t* row_src, void* x_disp, hipStream_t s);

// offsets -> m-tile table (for moe_expert_ffn, whose caller passes offsets only).
hipError_t launch_tile_table(const int32_t* offsets, int E, int C, int bm, int32_t* mt_off,
                             hipStream_t s);

// ---- grouped GEMM ------------------------------------------------------------
enum Epilogue {
    EPI_SWIGLU = 0,   // out[row, col] = act dtype of silu(gate) * up
    EPI_RELU2 = 1,    // out[row, col] = act dtype of max(acc, 0)^2
    EPI_STORE = 2,    // out[row, col] = act dtype of acc
    EPI_COMBINE = 3,  // out[row_src[row], col] = act dtype of w[row_src[row]] * acc
    EPI_F32 = 4       // out[row, col] = float acc (shared-expert sum)
};

struct GemmArgs {
    const void* A;          // activations, rows of lda elements (act dtype)
    int64_t lda;
    const void* B;          // weights [n_groups][N_w][K] (w dtype)
    int64_t b_group_stride; // elements between groups (experts)
    int64_t b_seg_stride;   // elements between K segments (concatenated shared experts)
    int k_seg;              // K-segment length (== K when B is not segmented)
    const float* bscale;    // e4m3 per-row scales [n_groups][N_w] or null
    int K;
    int N_w;                // rows of B per group
    int n_tiles;            // column tiles per m-tile
    int n_groups;
    const int32_t* offsets; // [n_groups+1] first A row of each group; null = uniform
    const int32_t* mt_off;  // [n_groups+1] m-tile prefix; null = uniform
    int uniform_rows;       // rows per group when offsets is null (A rows shared)
    int epi;
    void* out;
    int64_t ldo;
    int64_t out_col_per_group;  // column offset added per group (concatenated h)
    const float* route_w;       // EPI_COMBINE
    const int32_t* row_src;     // EPI_COMBINE; with gather, also the A-row map
    int I;                      // EPI_SWIGLU: up rows start at I in B
    int gather;                 // A row r is row row_src[r] / k_top of A (x in token order)
    int k_top;
};

constexpr int kGemmBM = 256;   // rows per m-tile of the bf16 MFMA kernel
constexpr int kGemmF32BM = 64; // rows per m-tile of the f32 kernel

hipError_t launch_gemm_bf16(const GemmArgs& a, int w_dtype, int grid, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, int grid, hipStream_t s);

// ---- slot-indexed expert GEMMs for decode-shaped batches ---------------------
// One segment: the routed experts (offsets != null: rows offsets[g] ..
// offsets[g+1], activation row = row_src[row] / k_top when gather, else the
// row itself) or the shared experts (offsets == null: uniform_rows rows,
// activation row = row).  blocks = units per group (16 output columns for
// SwiGLU, 32 otherwise).
constexpr int kDecodeBM = 32;        // activation rows per decode work item
constexpr int kDecodeMaxGroups = 1024;
struct DecodeSeg {
    const void* A;
    int64_t lda;
    int gather;
    const int32_t* offsets;     // routed: expert row ranges (and mt); uniform: NULL
    const int32_t* mt;          // routed: prefix over experts of ceil(rows / kDecodeBM)
    int uniform_rows;
    const void* B;
    int64_t b_group_stride;
    int64_t b_seg_stride;
    int k_seg;
    const float* bscale;
    int N_w, K, I;
    int epi;
    void* out;
    int64_t ldo;
    int64_t out_col_per_group;
    int n_groups;
    int blocks;
};
// Routing and dispatch done inside the gate/up launch for batches of at most
// kFuseMaxT tokens and kFuseMaxQ routes over at most kFuseMaxE experts with
// internal (softmax or sigmoid) routing or preselected routes: every
// workgroup computes the routes, ranks, offsets and tile table into LDS and
// workgroup 0 writes the metadata that later launches and the caller read.
constexpr int kFuseMaxT = 8;     // more tokens measured slower: the routing then delays the first weight load
constexpr int kFuseMaxQ = 256;   // one 64-route step per wavefront of the launch
constexpr int kFuseMaxE = 256;
struct DecodeFused {
    const float* logits;    // [T, E]
    const int32_t* ids_in;  // [T, k] preselected routes (then logits, ids and w are unused), or NULL
    const float* bias;      // [E] selection-only correction (sigmoid), or NULL
    int sigmoid;
    int T, k, E, ebits, C, renorm;
    float scale;
    int32_t* ids;           // [T, k]
    float* w;               // [T, k]
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E + 1]
    int32_t* mt;            // [E + 1], 32-row tiles
    int32_t* row_src;       // [r_max]
    int32_t* route_dst;     // [T, k]
    int32_t* ctrl;
    int64_t r_max;
};
struct DecodeArgs {
    DecodeSeg seg[2];
    int n_seg;
    const int32_t* row_src;
    int64_t rs_len;         // entries of row_src (0: none)
    int k_top;
    const float* route_w;
    int use_fused;          // segment 0's routes come from `fused`
    DecodeFused fused;
    int tail_split;         // whole units in complete rounds, the last partial round split over a workgroup's wavefronts
};
// small_m: no group has more than 8 rows (the 8-row staging of the decode ring)
hipError_t launch_decode_gemm(const DecodeArgs& d, int w_dtype, int split, int small_m, int grid,
                              hipStream_t s);

// ---- combine -----------------------------------------------------------------
// out[t] = sum_j (route_dst >= 0) coef * y[src] (+ y_shared[t]); NaN row when a
// route of t is malformed.  gather: src = route_dst[q], coef = w[q];
// slots: src = q, coef = 1 (the weights were applied in the GEMM epilogue).
hipError_t launch_combine(const void* y, int gather, const int32_t* route_dst, const float* w,
                          const float* y_shared, void* out, int T, int k, int H, int act_dtype,
                          hipStream_t s);

// Batches of at most kSmallMaxT tokens over at most kSmallMaxE experts: routing (or the caller's ids), ranks,
// counts, offsets, m-tile table, row_src and route_dst in one workgroup.
constexpr int kSmallMaxT = 64;
constexpr int kSmallMaxE = 512;
hipError_t launch_small_dispatch(const float* logits, const float* bias, const int32_t* ids_in,
                                int T, int k, int E, int C, int bm, int score_func, int renorm,
                                float scale, int32_t* ids, float* w, int32_t* counts,
                                int32_t* offsets, int32_t* mt_off, int32_t* row_src, int64_t r_max,
                                int32_t* route_dst, int32_t* ctrl, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_copy_u32(void* dst, const void* src, int64_t n, hipStream_t s);

int device_cu_count();

}  // namespace rde
