// C ABI of the MoE layer forward (declarations and contracts: include/moe.h).
//
// This layer validates every host-visible argument before anything is
// enqueued, carves the caller's workspace, and enqueues the kernels on the
// caller's stream.  It allocates nothing and never synchronises, except in
// moe_error.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"

namespace rde {

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t ctrl, partial, lrank, rexp, mt_off, ids, w, counts, offsets, row_src, route_dst;
    size_t x_disp, h, h_sh, ybuf, y_shared, total;
};

inline int64_t r_max_of(const moe_problem& p) {
    const int64_t a = (int64_t)p.T * p.k, b = (int64_t)p.E * p.C;
    return a < b ? a : b;
}
inline float route_scale_of(const moe_problem& p) { return p.route_scale == 0.0f ? 1.0f : p.route_scale; }
inline int act_bytes(const moe_problem& p) { return p.act_dtype == MOE_F32 ? 4 : 2; }
inline int gemm_bm(const moe_problem& p) { return p.act_dtype == MOE_F32 ? kGemmF32BM : kGemmBM; }

moe_status check_problem(const moe_problem* pp) {
    if (!pp) return MOE_ERR_ARG;
    const moe_problem& p = *pp;
    if (p.T < 0 || p.H <= 0 || p.E <= 0 || p.k <= 0 || p.I <= 0 || p.C <= 0) return MOE_ERR_ARG;
    if (p.k > 32 || p.k > p.E) return MOE_ERR_ARG;
    if (p.act_dtype != MOE_F32 && p.act_dtype != MOE_BF16) return MOE_ERR_ARG;
    if (p.w_dtype != MOE_F32 && p.w_dtype != MOE_BF16 && p.w_dtype != MOE_E4M3) return MOE_ERR_ARG;
    if ((p.w_dtype == MOE_F32) != (p.act_dtype == MOE_F32)) return MOE_ERR_ARG;
    if (p.act != MOE_SWIGLU && p.act != MOE_RELU2) return MOE_ERR_ARG;
    if (p.renormalize != 0 && p.renormalize != 1) return MOE_ERR_ARG;
    if (p.score_func != MOE_SOFTMAX && p.score_func != MOE_SIGMOID) return MOE_ERR_ARG;
    if (!(p.route_scale >= 0.0f) || p.route_scale == INFINITY) return MOE_ERR_ARG;
    if (p.n_shared < 0 || p.n_shared > 8) return MOE_ERR_ARG;
    if (p.n_shared > 0 && p.I_shared <= 0) return MOE_ERR_ARG;
    if (p.E > 1024) return MOE_ERR_UNSUPPORTED;
    if (p.H % 128 || p.I % 128) return MOE_ERR_UNSUPPORTED;
    if (p.n_shared > 0 && p.I_shared % 128) return MOE_ERR_UNSUPPORTED;
    const int64_t Q = (int64_t)p.T * p.k;
    if (Q >= INT_MAX / 2) return MOE_ERR_UNSUPPORTED;  // route and row indices are int32
    // one expert's weight matrix is addressed with 32-bit offsets in the GEMMs
    const int64_t wb = p.w_dtype == MOE_F32 ? 4 : 2;
    const int64_t lim = (int64_t)1 << 31;
    if (2 * (int64_t)p.I * p.H * wb >= lim) return MOE_ERR_UNSUPPORTED;
    if (p.n_shared > 0 && 2 * (int64_t)p.I_shared * p.H * 4 >= lim) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

Layout layout_of(const moe_problem& p) {
    Layout L;
    const int64_t Q = (int64_t)p.T * p.k, R = r_max_of(p);
    const int nb = count_blocks(Q) > 0 ? count_blocks(Q) : 1;
    const size_t ab = (size_t)act_bytes(p);
    const int groups = p.E > p.n_shared ? p.E : p.n_shared;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up(bytes > 0 ? bytes : 1); return at; };
    L.ctrl = take(sizeof(int32_t) * CTRL_WORDS);
    L.partial = take(sizeof(int32_t) * (size_t)nb * p.E);
    L.lrank = take(sizeof(int32_t) * (size_t)Q);
    L.rexp = take(sizeof(int32_t) * (size_t)Q);
    L.mt_off = take(sizeof(int32_t) * (size_t)(groups + 2));
    L.ids = take(sizeof(int32_t) * (size_t)Q);
    L.w = take(sizeof(float) * (size_t)Q);
    L.counts = take(sizeof(int32_t) * (size_t)p.E);
    L.offsets = take(sizeof(int32_t) * (size_t)(p.E + 1));
    L.row_src = take(sizeof(int32_t) * (size_t)R);
    L.route_dst = take(sizeof(int32_t) * (size_t)Q);
    L.x_disp = take(ab * (size_t)R * p.H);
    L.h = take(ab * (size_t)R * p.I);
    L.h_sh = take(p.n_shared ? ab * (size_t)p.T * p.n_shared * p.I_shared : 0);
    L.ybuf = take(ab * (size_t)Q * p.H);
    L.y_shared = take(p.n_shared ? sizeof(float) * (size_t)p.T * p.H : 0);
    L.total = o;
    return L;
}

template <typename T_>
T_* at(void* ws, size_t off) { return (T_*)((char*)ws + off); }

inline bool aligned16(const void* q) { return ((uintptr_t)q & 15) == 0; }

moe_status check_ws(const moe_problem& p, void* ws, size_t ws_bytes, Layout* L) {
    if (!ws || ((uintptr_t)ws & (kAlign - 1))) return MOE_ERR_WORKSPACE;
    *L = layout_of(p);
    if (ws_bytes < L->total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Persistent grid of the bf16 GEMM: one 512-thread workgroup per CU (its LDS
// stages take most of the CU's 160 KB), a multiple of 8 (XCD count).
int gemm_grid(int64_t tiles_upper) {
    int g = device_cu_count();
    g = (g + 7) / 8 * 8;
    if (tiles_upper < g) g = (int)((tiles_upper + 7) / 8 * 8);
    return g > 8 ? g : 8;
}

// GEMM1 (A -> h) over the routed experts, tile table mt_off.  A is x_disp,
// or x in token order read through row_src when row_src is given (bf16).
hipError_t run_gemm1(const moe_problem& p, const void* A, const int32_t* offsets,
                     const int32_t* mt_off, const void* w13, const float* s13, void* h,
                     hipStream_t s, const int32_t* row_src = nullptr) {
    GemmArgs a = {};
    a.A = A;
    a.row_src = row_src;
    a.gather = row_src != nullptr;
    a.k_top = p.k;
    a.lda = p.H;
    a.B = w13;
    a.N_w = p.act == MOE_SWIGLU ? 2 * p.I : p.I;
    a.b_group_stride = (int64_t)a.N_w * p.H;
    a.b_seg_stride = 0;
    a.k_seg = p.H;
    a.bscale = s13;
    a.K = p.H;
    a.n_groups = p.E;
    a.offsets = offsets;
    a.mt_off = mt_off;
    a.epi = p.act == MOE_SWIGLU ? EPI_SWIGLU : EPI_RELU2;
    a.out = h;
    a.ldo = p.I;
    a.out_col_per_group = 0;
    a.I = p.I;
    const int64_t R = r_max_of(p);
    if (p.act_dtype == MOE_F32) {
        a.n_tiles = p.act == MOE_SWIGLU ? p.I / 32 : p.I / 64;
        return launch_gemm_f32(a, gemm_grid((R / kGemmF32BM + p.E) * a.n_tiles), s);
    }
    a.n_tiles = p.act == MOE_SWIGLU ? p.I / 128 : (p.I + 255) / 256;
    return launch_gemm_bf16(a, p.w_dtype, gemm_grid((R / kGemmBM + p.E) * a.n_tiles), s);
}

// GEMM2 (h -> y) over the routed experts, epilogue EPI_STORE (y_disp) or
// EPI_COMBINE (weighted rows into the token-ordered slot buffer).
hipError_t run_gemm2(const moe_problem& p, const void* h, const int32_t* offsets,
                     const int32_t* mt_off, const void* w2, const float* s2, int epi, void* out,
                     const float* route_w, const int32_t* row_src, hipStream_t s) {
    GemmArgs a = {};
    a.A = h;
    a.lda = p.I;
    a.B = w2;
    a.N_w = p.H;
    a.b_group_stride = (int64_t)p.H * p.I;
    a.k_seg = p.I;
    a.bscale = s2;
    a.K = p.I;
    a.n_groups = p.E;
    a.offsets = offsets;
    a.mt_off = mt_off;
    a.epi = epi;
    a.out = out;
    a.ldo = p.H;
    a.route_w = route_w;
    a.row_src = row_src;
    a.I = p.I;
    const int64_t R = r_max_of(p);
    if (p.act_dtype == MOE_F32) {
        a.n_tiles = p.H / 64;
        return launch_gemm_f32(a, gemm_grid((R / kGemmF32BM + p.E) * a.n_tiles), s);
    }
    a.n_tiles = (p.H + 255) / 256;
    return launch_gemm_bf16(a, p.w_dtype, gemm_grid((R / kGemmBM + p.E) * a.n_tiles), s);
}

// Shared experts: h_sh [T, S*Is] = SwiGLU over every token for each expert s,
// then y_shared [T, H] (float32) = h_sh @ [W2_0 | W2_1 | ...]^T as one
// product whose K runs over the concatenated shared intermediates.
hipError_t run_shared(const moe_problem& p, const void* x, const void* w13_sh, const void* w2_sh,
                      void* h_sh, float* y_shared, hipStream_t s) {
    const int S = p.n_shared, Is = p.I_shared;
    const int wdt = p.act_dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
    GemmArgs a = {};
    a.A = x;
    a.lda = p.H;
    a.B = w13_sh;
    a.N_w = 2 * Is;
    a.b_group_stride = (int64_t)2 * Is * p.H;
    a.k_seg = p.H;
    a.K = p.H;
    a.n_groups = S;
    a.uniform_rows = p.T;
    a.epi = EPI_SWIGLU;
    a.out = h_sh;
    a.ldo = (int64_t)S * Is;
    a.out_col_per_group = Is;
    a.I = Is;
    hipError_t e;
    const int bm = p.act_dtype == MOE_F32 ? kGemmF32BM : kGemmBM;
    const int64_t mt = (int64_t)((p.T + bm - 1) / bm);
    if (p.act_dtype == MOE_F32) {
        a.n_tiles = Is / 32;
        e = launch_gemm_f32(a, gemm_grid(mt * S * a.n_tiles), s);
    } else {
        a.n_tiles = Is / 128;
        e = launch_gemm_bf16(a, wdt, gemm_grid(mt * S * a.n_tiles), s);
    }
    if (e != hipSuccess) return e;
    GemmArgs b = {};
    b.A = h_sh;
    b.lda = (int64_t)S * Is;
    b.B = w2_sh;
    b.N_w = p.H;
    b.b_group_stride = 0;
    b.k_seg = Is;
    b.b_seg_stride = (int64_t)p.H * Is;
    b.K = S * Is;
    b.n_groups = 1;
    b.uniform_rows = p.T;
    b.epi = EPI_F32;
    b.out = y_shared;
    b.ldo = p.H;
    if (p.act_dtype == MOE_F32) {
        b.n_tiles = p.H / 64;
        return launch_gemm_f32(b, gemm_grid(mt * b.n_tiles), s);
    }
    b.n_tiles = (p.H + 255) / 256;
    return launch_gemm_bf16(b, wdt, gemm_grid(mt * b.n_tiles), s);
}

inline hipError_t mark(const moe_meta& m, int stage, hipStream_t s) {
    if (!m.stage_events || !m.stage_events[stage]) return hipSuccess;
    return hipEventRecord((hipEvent_t)m.stage_events[stage], s);
}

// ---- decode-shaped batches ---------------------------------------------------
// Batches with few rows per expert run the expert GEMMs as slot-indexed
// units (decode.hip): every touched expert's weights stream once over all
// wavefronts and activation rows are read in place.  The switch point is an
// average of kDecodeRowsPerExpert routes per expert (PR 33963 switches its
// kernels on the route count, at 128 routes for 240 experts); the
// environment variable MOE_DECODE_ROWS_PER_EXPERT overrides it (read once).
constexpr int kDecodeRowsPerExpert = 12;

int decode_rows_per_expert() {
    static const int v = [] {
        const char* e = std::getenv("MOE_DECODE_ROWS_PER_EXPERT");
        return e ? std::atoi(e) : kDecodeRowsPerExpert;
    }();
    return v;
}

bool decode_mode(const moe_problem& p) {
    return p.act_dtype == MOE_BF16 && (int64_t)p.T * p.k <= (int64_t)decode_rows_per_expert() * p.E;
}

int decode_grid() { return device_cu_count(); }  // 4 wavefronts x 32 KB LDS ring per CU

// mt: prefix over experts of ceil(rows / kDecodeBM) (the dispatch's m-tile
// table built with that tile height).
DecodeSeg routed_seg1(const moe_problem& p, const void* A, int gather, const int32_t* offsets,
                      const int32_t* mt, const void* w13, const float* s13, void* h) {
    DecodeSeg s = {};
    s.A = A;
    s.lda = p.H;
    s.gather = gather;
    s.offsets = offsets;
    s.mt = mt;
    s.B = w13;
    s.N_w = p.act == MOE_SWIGLU ? 2 * p.I : p.I;
    s.b_group_stride = (int64_t)s.N_w * p.H;
    s.k_seg = p.H;
    s.bscale = s13;
    s.K = p.H;
    s.I = p.I;
    s.epi = p.act == MOE_SWIGLU ? EPI_SWIGLU : EPI_RELU2;
    s.out = h;
    s.ldo = p.I;
    s.n_groups = p.E;
    s.blocks = p.act == MOE_SWIGLU ? p.I / 16 : p.I / 32;
    return s;
}

DecodeSeg routed_seg2(const moe_problem& p, const void* h, const int32_t* offsets, const int32_t* mt,
                      const void* w2, const float* s2, int epi, void* out) {
    DecodeSeg s = {};
    s.A = h;
    s.lda = p.I;
    s.offsets = offsets;
    s.mt = mt;
    s.B = w2;
    s.N_w = p.H;
    s.b_group_stride = (int64_t)p.H * p.I;
    s.k_seg = p.I;
    s.bscale = s2;
    s.K = p.I;
    s.epi = epi;
    s.out = out;
    s.ldo = p.H;
    s.n_groups = p.E;
    s.blocks = (p.H + 31) / 32;
    return s;
}

DecodeSeg shared_seg1(const moe_problem& p, const void* x, const void* w13_sh, void* h_sh) {
    const int Is = p.I_shared;
    DecodeSeg s = {};
    s.A = x;
    s.lda = p.H;
    s.uniform_rows = p.T;
    s.B = w13_sh;
    s.N_w = 2 * Is;
    s.b_group_stride = (int64_t)2 * Is * p.H;
    s.k_seg = p.H;
    s.K = p.H;
    s.I = Is;
    s.epi = EPI_SWIGLU;
    s.out = h_sh;
    s.ldo = (int64_t)p.n_shared * Is;
    s.out_col_per_group = Is;
    s.n_groups = p.n_shared;
    s.blocks = Is / 16;
    return s;
}

DecodeSeg shared_seg2(const moe_problem& p, const void* h_sh, const void* w2_sh, float* y_shared) {
    const int Is = p.I_shared;
    DecodeSeg s = {};
    s.A = h_sh;
    s.lda = (int64_t)p.n_shared * Is;
    s.uniform_rows = p.T;
    s.B = w2_sh;
    s.N_w = p.H;
    s.b_group_stride = 0;
    s.k_seg = Is;
    s.b_seg_stride = (int64_t)p.H * Is;
    s.K = p.n_shared * Is;
    s.epi = EPI_F32;
    s.out = y_shared;
    s.ldo = p.H;
    s.n_groups = 1;
    s.blocks = (p.H + 31) / 32;
    return s;
}

// max_rows: a bound on the rows of any group known to hold (-1: none); 8 or
// fewer selects the 8-row activation staging.
// fused: the launch routes and dispatches the batch itself (gate/up only).
// rs_len: entries of row_src.
hipError_t run_decode(const DecodeSeg* a, const DecodeSeg* b, const int32_t* row_src, int64_t rs_len, int k,
                      const float* route_w, int w_dtype, int64_t route_count, int max_rows,
                      hipStream_t s, const DecodeFused* fused = nullptr) {
    DecodeArgs d = {};
    d.seg[0] = a ? *a : *b;
    d.n_seg = 1;
    if (fused) {
        d.use_fused = 1;
        d.fused = *fused;
    }
    if (a && b) {
        d.seg[1] = *b;
        d.n_seg = 2;
    }
    d.row_src = row_src;
    d.rs_len = row_src ? rs_len : 0;
    d.k_top = k;
    d.route_w = route_w;
    // a routed segment (tile table staged in LDS) can only be the first one
    if (d.n_seg > 1 && d.seg[1].offsets) return hipErrorInvalidValue;
    if (d.seg[0].offsets && (!d.seg[0].mt || d.seg[0].n_groups > kDecodeMaxGroups)) return hipErrorInvalidValue;
    // When the launch has fewer units than the chip has wavefronts, split
    // each unit's K over 2 or 4 wavefronts of a workgroup, choosing the split
    // with the fewest K groups on the longest wavefront's path: a first round
    // of the longest units (the shared experts' down projections go first),
    // then rounds of the shortest, each costing its K groups per wavefront
    // plus 4 for the ring fill, the partial sums and the epilogue; ties go to
    // the wider split.  The number of touched experts is on the device; the
    // host bounds it by min(E, T*k).
    int64_t units = 0;
    int kmin = INT_MAX, kmax = 0;
    for (int i = 0; i < d.n_seg; ++i) {
        const DecodeSeg& g = d.seg[i];
        const int64_t groups = g.offsets ? std::min<int64_t>(g.n_groups, route_count) : g.n_groups;
        units += groups * g.blocks;
        kmin = std::min(kmin, g.K);
        kmax = std::max(kmax, g.K);
    }
    const int64_t waves = (int64_t)decode_grid() * 4;
    int split = 1;
    if (units < waves) {
        const int64_t nk_long = kmax / 64, nk_short = kmin / 64;   // K groups of 64
        int64_t best = -1;
        for (int s : {4, 2, 1}) {
            const int64_t rounds = (units + waves / s - 1) / (waves / s);
            const int64_t cost = (nk_long + s - 1) / s + 4 + (rounds - 1) * ((nk_short + s - 1) / s + 4);
            if (best < 0 || cost < best) {
                best = cost;
                split = s;
            }
        }
    }
    // MOE_DECODE_SPLIT = 1, 2 or 4 (read on every call) forces the split of
    // every decode launch, so tests can run each form over several rounds
    if (const char* f = std::getenv("MOE_DECODE_SPLIT")) {
        const int v = std::atoi(f);
        if (v == 1 || v == 2 || v == 4) split = v;
    }
    // otherwise the partial last round is split over a workgroup's
    // wavefronts when each still gets >= 5 K groups of 64 (K >= 1280; shorter
    // streams are mostly ring fill, and measured slower split than whole)
    d.tail_split = split == 1 && kmin >= 1280;
    // the shared experts are always bf16; a segment list that starts with them
    // runs the bf16 instantiation
    const int small_m = (max_rows >= 0 && max_rows <= 8) ? 1 : 0;
    return launch_decode_gemm(d, a ? w_dtype : MOE_BF16, split, small_m, decode_grid(), s);
}

moe_status check_ptrs16(std::initializer_list<const void*> ps) {
    for (const void* q : ps)
        if (!q || !aligned16(q)) return MOE_ERR_ARG;
    return MOE_OK;
}

}  // namespace
}  // namespace rde

using namespace rde;

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported problem";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

moe_status moe_workspace_bytes(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_ARG;
    *bytes = layout_of(*p).total;
    return MOE_OK;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < sizeof(int32_t) * CTRL_WORDS) return MOE_ERR_WORKSPACE;
    return hip_status(launch_fill_i32((int32_t*)ws, CTRL_WORDS, 0, (hipStream_t)stream));
}

moe_status moe_route(const moe_problem* p, const float* logits, const float* score_bias,
                     int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (score_bias && p->score_func != MOE_SIGMOID) return MOE_ERR_ARG;
    Layout L;
    if ((st = check_ws(*p, ws, ws_bytes, &L)) != MOE_OK) return st;
    if (p->T == 0) return MOE_OK;
    if (!logits || !ids || !w) return MOE_ERR_ARG;
    return hip_status(launch_route(logits, score_bias, p->T, p->E, p->k, p->score_func, p->renormalize,
                                   route_scale_of(*p), ids, w, (hipStream_t)stream));
}

moe_status moe_dispatch(const moe_problem* p, const void* x, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* row_src, int32_t* route_dst, void* x_disp,
                        void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    Layout L;
    if ((st = check_ws(*p, ws, ws_bytes, &L)) != MOE_OK) return st;
    if (!counts || !offsets) return MOE_ERR_ARG;
    if (p->T > 0 && (check_ptrs16({x, x_disp}) != MOE_OK || !ids || !row_src || !route_dst))
        return MOE_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    const int64_t Q = (int64_t)p->T * p->k;
    if (Q > 0 && Q <= kPlaceMaxQ) {
        // one workgroup counts, scans and places every route; then the copies
        hipError_t e = launch_count_place(ids, p->T, p->k, p->E, p->C, gemm_bm(*p), counts, offsets,
                                          at<int32_t>(ws, L.mt_off), row_src, r_max_of(*p), route_dst,
                                          at<int32_t>(ws, L.ctrl), s);
        if (e != hipSuccess) return MOE_ERR_HIP;
        return hip_status(launch_copy_rows(x, p->T, p->H, p->k, act_bytes(*p), route_dst, x_disp, s));
    }
    hipError_t e = launch_count_rank(ids, p->T, p->k, p->E, p->C, gemm_bm(*p), at<int32_t>(ws, L.rexp),
                                     at<int32_t>(ws, L.lrank), at<int32_t>(ws, L.partial), counts,
                                     offsets, at<int32_t>(ws, L.mt_off), at<int32_t>(ws, L.ctrl), s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_scatter(x, p->T, p->H, p->k, p->E, p->C, act_bytes(*p), r_max_of(*p),
                                     at<int32_t>(ws, L.rexp), at<int32_t>(ws, L.lrank),
                                     at<int32_t>(ws, L.partial), offsets, route_dst, row_src, x_disp, s));
}

moe_status moe_expert_ffn(const moe_problem* p, const void* x_disp, const int32_t* offsets,
                          const void* w13, const void* w2, const float* s13, const float* s2,
                          void* y_disp, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    Layout L;
    if ((st = check_ws(*p, ws, ws_bytes, &L)) != MOE_OK) return st;
    if (p->T == 0 || r_max_of(*p) == 0) return MOE_OK;
    if (check_ptrs16({x_disp, w13, w2, y_disp}) != MOE_OK || !offsets) return MOE_ERR_ARG;
    if ((p->w_dtype == MOE_E4M3) != (s13 != nullptr && s2 != nullptr)) return MOE_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    void* h = at<void>(ws, L.h);
    int32_t* mt = at<int32_t>(ws, L.mt_off);
    if (decode_mode(*p)) {
        if (launch_tile_table(offsets, p->E, p->C, kDecodeBM, mt, s) != hipSuccess) return MOE_ERR_HIP;
        const DecodeSeg g1 = routed_seg1(*p, x_disp, 0, offsets, mt, w13, s13, h);
        if (run_decode(&g1, nullptr, nullptr, 0, p->k, nullptr, p->w_dtype, (int64_t)p->T * p->k, -1, s) != hipSuccess) return MOE_ERR_HIP;
        const DecodeSeg g2 = routed_seg2(*p, h, offsets, mt, w2, s2, EPI_STORE, y_disp);
        return hip_status(run_decode(&g2, nullptr, nullptr, 0, p->k, nullptr, p->w_dtype, (int64_t)p->T * p->k, -1, s));
    }
    if (launch_tile_table(offsets, p->E, p->C, gemm_bm(*p), mt, s) != hipSuccess) return MOE_ERR_HIP;
    if (run_gemm1(*p, x_disp, offsets, mt, w13, s13, h, s) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(run_gemm2(*p, h, offsets, mt, w2, s2, EPI_STORE, y_disp, nullptr, nullptr, s));
}

moe_status moe_shared_ffn(const moe_problem* p, const void* x, const void* w13_sh, const void* w2_sh,
                          float* y_shared, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    Layout L;
    if ((st = check_ws(*p, ws, ws_bytes, &L)) != MOE_OK) return st;
    if (p->n_shared == 0) return MOE_ERR_ARG;
    if (p->T == 0) return MOE_OK;
    if (check_ptrs16({x, w13_sh, w2_sh, y_shared}) != MOE_OK) return MOE_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (decode_mode(*p)) {
        void* h_sh = at<void>(ws, L.h_sh);
        const DecodeSeg g1 = shared_seg1(*p, x, w13_sh, h_sh);
        // shared experts: every group holds exactly T rows
        if (run_decode(nullptr, &g1, nullptr, 0, p->k, nullptr, MOE_BF16, (int64_t)p->T * p->k, p->T, s) != hipSuccess) return MOE_ERR_HIP;
        const DecodeSeg g2 = shared_seg2(*p, h_sh, w2_sh, y_shared);
        return hip_status(run_decode(nullptr, &g2, nullptr, 0, p->k, nullptr, MOE_BF16, (int64_t)p->T * p->k, p->T, s));
    }
    return hip_status(run_shared(*p, x, w13_sh, w2_sh, at<void>(ws, L.h_sh), y_shared, s));
}

moe_status moe_combine(const moe_problem* p, const void* y_disp, const int32_t* route_dst,
                       const float* w, const float* y_shared, void* out, void* ws, size_t ws_bytes,
                       void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    Layout L;
    if ((st = check_ws(*p, ws, ws_bytes, &L)) != MOE_OK) return st;
    if (p->T == 0) return MOE_OK;
    if (check_ptrs16({out}) != MOE_OK || !route_dst || !w) return MOE_ERR_ARG;
    if (r_max_of(*p) > 0 && check_ptrs16({y_disp}) != MOE_OK) return MOE_ERR_ARG;
    if (y_shared && !aligned16(y_shared)) return MOE_ERR_ARG;
    return hip_status(launch_combine(y_disp, 1, route_dst, w, y_shared, out, p->T, p->k, p->H,
                                     p->act_dtype, (hipStream_t)stream));
}

moe_status moe_forward(const moe_problem* p, const void* x, const float* logits,
                       const float* score_bias, const int32_t* ids_in, const float* w_in, const void* w13, const void* w2, const float* s13,
                       const float* s2, const void* w13_sh, const void* w2_sh, void* out,
                       const moe_meta* meta, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (score_bias && p->score_func != MOE_SIGMOID) return MOE_ERR_ARG;
    Layout L;
    if ((st = check_ws(*p, ws, ws_bytes, &L)) != MOE_OK) return st;
    const moe_problem& P = *p;
    const bool pre = ids_in != nullptr || w_in != nullptr;
    if (pre && !(ids_in && w_in)) return MOE_ERR_ARG;
    if (P.T > 0) {
        if (check_ptrs16({x, w13, w2, out}) != MOE_OK) return MOE_ERR_ARG;
        if (!pre && !logits) return MOE_ERR_ARG;
        if ((P.w_dtype == MOE_E4M3) != (s13 != nullptr && s2 != nullptr)) return MOE_ERR_ARG;
        if (P.n_shared && check_ptrs16({w13_sh, w2_sh}) != MOE_OK) return MOE_ERR_ARG;
    }
    moe_meta m = {};
    if (meta) m = *meta;
    // router outputs; preselected routes are read in place unless the caller
    // asked for a copy in its metadata outputs
    int32_t* ids_out = m.ids ? m.ids : at<int32_t>(ws, L.ids);
    float* w_out = m.w ? m.w : at<float>(ws, L.w);
    const int32_t* ids = (pre && !m.ids) ? ids_in : ids_out;
    const float* w = (pre && !m.w) ? w_in : w_out;
    int32_t* counts = m.counts ? m.counts : at<int32_t>(ws, L.counts);
    int32_t* offsets = m.offsets ? m.offsets : at<int32_t>(ws, L.offsets);
    int32_t* row_src = m.row_src ? m.row_src : at<int32_t>(ws, L.row_src);
    int32_t* route_dst = m.route_dst ? m.route_dst : at<int32_t>(ws, L.route_dst);
    hipStream_t s = (hipStream_t)stream;
    const int64_t Q = (int64_t)P.T * P.k;
    const bool dec = decode_mode(P);
    // bf16 layers read expert rows in place (no expert-contiguous copy of x)
    const bool in_place = dec || P.act_dtype == MOE_BF16;
    void* x_disp = at<void>(ws, L.x_disp);
    int32_t* mt = at<int32_t>(ws, L.mt_off);
    // the m-tile table serves the grouped GEMM (its tile height) or the
    // slot-indexed decode GEMMs (32-row work items)
    const int tile_bm = dec ? kDecodeBM : gemm_bm(P);
    hipError_t e = mark(m, MOE_STAGE_BEGIN, s);
    if (e == hipSuccess && pre) {
        // preselected routes: copied only into metadata outputs the caller gave
        if (m.ids && m.ids != ids_in) e = launch_copy_u32(m.ids, ids_in, Q, s);
        if (e == hipSuccess && m.w && m.w != w_in) e = launch_copy_u32(m.w, w_in, Q, s);
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
    // batches of a few tokens with internal routing: the gate/up decode launch
    // routes and dispatches them itself, one launch fewer
    const bool fused = dec && P.T > 0 && P.T <= kFuseMaxT && Q <= kFuseMaxQ &&
                       P.E <= kFuseMaxE && P.w_dtype == MOE_BF16;
    if (fused) {
        for (int st = MOE_STAGE_ROUTE; e == hipSuccess && st <= MOE_STAGE_SCATTER; ++st) e = mark(m, st, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
    } else if (in_place && P.T <= kSmallMaxT && P.E <= kSmallMaxE) {
        // small batch: routing and the whole dispatch in one workgroup
        e = launch_small_dispatch(pre ? nullptr : logits, score_bias, pre ? ids_in : nullptr, P.T,
                                  P.k, P.E, P.C, tile_bm, P.score_func, P.renormalize,
                                  route_scale_of(P), ids_out, w_out, counts, offsets, mt, row_src,
                                  r_max_of(P), route_dst, at<int32_t>(ws, L.ctrl), s);
        for (int st = MOE_STAGE_ROUTE; e == hipSuccess && st <= MOE_STAGE_SCATTER; ++st) e = mark(m, st, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
    } else {
        if (!pre && P.T > 0)
            e = launch_route(logits, score_bias, P.T, P.E, P.k, P.score_func, P.renormalize,
                             route_scale_of(P), ids_out, w_out, s);
        if (e == hipSuccess) e = mark(m, MOE_STAGE_ROUTE, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
        if (Q > 0 && Q <= kPlaceMaxQ) {
            // one workgroup counts, scans and places every route (no hand-off
            // between blocks); float32 layers then copy their rows
            e = launch_count_place(ids, P.T, P.k, P.E, P.C, tile_bm, counts, offsets, mt, row_src,
                                   r_max_of(P), route_dst, at<int32_t>(ws, L.ctrl), s);
            if (e == hipSuccess) e = mark(m, MOE_STAGE_COUNT, s);
            if (e == hipSuccess && !in_place)
                e = launch_copy_rows(x, P.T, P.H, P.k, act_bytes(P), route_dst, x_disp, s);
        } else {
            // routes that fit one count block are placed by that block when no
            // rows are copied: no separate scatter launch
            const bool place = in_place && count_blocks(Q) <= 1;
            // rows read in place and few per-block totals: the metadata
            // scatter scans them itself
            const int local = in_place && local_scan_fits(Q, P.E) ? 1 : 0;
            e = launch_count_rank(ids, P.T, P.k, P.E, P.C, tile_bm, at<int32_t>(ws, L.rexp),
                                  at<int32_t>(ws, L.lrank), at<int32_t>(ws, L.partial), counts, offsets, mt,
                                  at<int32_t>(ws, L.ctrl), s, place ? route_dst : nullptr, row_src,
                                  r_max_of(P), local);
            if (e == hipSuccess) e = mark(m, MOE_STAGE_COUNT, s);
            if (e == hipSuccess && P.T > 0 && !place && local)
                e = launch_scatter_scan(P.T, P.k, P.E, P.C, tile_bm, r_max_of(P), at<int32_t>(ws, L.rexp),
                                        at<int32_t>(ws, L.lrank), at<int32_t>(ws, L.partial), counts, offsets,
                                        mt, route_dst, row_src, s);
            else if (e == hipSuccess && P.T > 0 && !place)
                e = launch_scatter(x, P.T, P.H, P.k, P.E, P.C, act_bytes(P), r_max_of(P),
                                   at<int32_t>(ws, L.rexp), at<int32_t>(ws, L.lrank),
                                   at<int32_t>(ws, L.partial), offsets, route_dst, row_src,
                                   in_place ? nullptr : x_disp, s);
        }
        if (e == hipSuccess) e = mark(m, MOE_STAGE_SCATTER, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    void* h = at<void>(ws, L.h);
    void* ybuf = at<void>(ws, L.ybuf);
    float* y_sh = P.n_shared ? at<float>(ws, L.y_shared) : nullptr;
    const bool work = P.T > 0 && r_max_of(P) > 0;
    if (dec && P.T > 0) {
        // slot-indexed expert GEMMs; routed and shared units share each launch
        void* h_sh = at<void>(ws, L.h_sh);
        const DecodeSeg r1 = routed_seg1(P, x, 1, offsets, mt, w13, s13, h);
        const DecodeSeg sh1 = P.n_shared ? shared_seg1(P, x, w13_sh, h_sh) : DecodeSeg{};
        // rows per group <= T: the dispatch keeps at most one route of a token per
        // expert (a repeated expert is a malformed route), shared groups hold T
        DecodeFused fz = {};
        if (fused) {
            fz.logits = logits;
            fz.ids_in = pre ? ids_in : nullptr;
            fz.bias = score_bias;
            fz.sigmoid = P.score_func == MOE_SIGMOID;
            fz.T = P.T;
            fz.k = P.k;
            fz.E = P.E;
            while ((1 << fz.ebits) < P.E) ++fz.ebits;
            fz.C = P.C;
            fz.renorm = P.renormalize;
            fz.scale = route_scale_of(P);
            fz.ids = ids_out;
            fz.w = w_out;
            fz.counts = counts;
            fz.offsets = offsets;
            fz.mt = mt;
            fz.row_src = row_src;
            fz.route_dst = route_dst;
            fz.ctrl = at<int32_t>(ws, L.ctrl);
            fz.r_max = r_max_of(P);
        }
        e = run_decode(&r1, P.n_shared ? &sh1 : nullptr, row_src, r_max_of(P), P.k, w, P.w_dtype, (int64_t)P.T * P.k, P.T, s,
                       fused ? &fz : nullptr);
        if (e == hipSuccess) e = mark(m, MOE_STAGE_GEMM1, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
        const DecodeSeg r2 = routed_seg2(P, h, offsets, mt, w2, s2, EPI_COMBINE, ybuf);
        const DecodeSeg sh2 = P.n_shared ? shared_seg2(P, h_sh, w2_sh, y_sh) : DecodeSeg{};
        e = run_decode(&r2, P.n_shared ? &sh2 : nullptr, row_src, r_max_of(P), P.k, w, P.w_dtype, (int64_t)P.T * P.k, P.T, s);
        if (e == hipSuccess) e = mark(m, MOE_STAGE_GEMM2, s);
        if (e == hipSuccess) e = mark(m, MOE_STAGE_SHARED, s);
        if (e == hipSuccess)
            e = launch_combine(ybuf, 0, route_dst, nullptr, y_sh, out, P.T, P.k, P.H, P.act_dtype, s);
        if (e == hipSuccess) e = mark(m, MOE_STAGE_COMBINE, s);
        return hip_status(e);
    }
    if (work)
        e = in_place ? run_gemm1(P, x, offsets, mt, w13, s13, h, s, row_src)
                     : run_gemm1(P, x_disp, offsets, mt, w13, s13, h, s);
    if (e == hipSuccess) e = mark(m, MOE_STAGE_GEMM1, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (work) e = run_gemm2(P, h, offsets, mt, w2, s2, EPI_COMBINE, ybuf, w, row_src, s);
    if (e == hipSuccess) e = mark(m, MOE_STAGE_GEMM2, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (P.T > 0 && P.n_shared) e = run_shared(P, x, w13_sh, w2_sh, at<void>(ws, L.h_sh), y_sh, s);
    if (e == hipSuccess) e = mark(m, MOE_STAGE_SHARED, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (P.T > 0) e = launch_combine(ybuf, 0, route_dst, nullptr, y_sh, out, P.T, P.k, P.H, P.act_dtype, s);
    if (e == hipSuccess) e = mark(m, MOE_STAGE_COMBINE, s);
    return hip_status(e);
}

}  // extern "C"

// ---- moe_forward_static: the layer without a caller workspace ---------------
// Its workspace is a file-scope device array (one copy per GPU, alive until
// the process ends).  In host code `scratch` only names the symbol: its
// device address is looked up once per device with hipGetSymbolAddress and
// that address is what the kernels get.
namespace rde {

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's array.  The first call on a device looks
// it up and clears the control words (malformed-route counter, the count
// kernel's arrival ticket) with a fill kernel on `s`, ahead of that call's
// own kernels; the count kernel leaves its ticket at zero after every launch.
moe_status static_scratch(hipStream_t s, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        if (((uintptr_t)ptr & 255) != 0) return MOE_ERR_HIP;
        if (launch_fill_i32((int32_t*)ptr, CTRL_WORDS, 0, s) != hipSuccess) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace
}  // namespace rde

extern "C" {

moe_status moe_forward_static(const moe_problem* p, const void* x, const float* logits,
                              const float* score_bias, const int32_t* ids_in, const float* w_in,
                              const void* w13, const void* w2, const float* s13, const float* s2,
                              const void* w13_sh, const void* w2_sh, void* out,
                              const moe_meta* meta, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (layout_of(*p).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = static_scratch((hipStream_t)stream, &ws)) != MOE_OK) return st;
    return moe_forward(p, x, logits, score_bias, ids_in, w_in, w13, w2, s13, s2, w13_sh, w2_sh, out,
                       meta, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

moe_status moe_error(void* ws, size_t ws_bytes, void* stream, int32_t* n_invalid_routes) {
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < sizeof(int32_t) * CTRL_WORDS) return MOE_ERR_WORKSPACE;
    if (!n_invalid_routes) return MOE_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    int32_t v = 0;
    if (hipMemcpyAsync(&v, (int32_t*)ws + CTRL_BAD_ROUTES, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    if (launch_fill_i32((int32_t*)ws + CTRL_BAD_ROUTES, 1, 0, s) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    *n_invalid_routes = v;
    return MOE_OK;
}

}  // extern "C"
