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
// m-tiles; the m-tile prefix over experts (mt_off, built on the device by the
// dispatch) maps a tile index to its expert with a binary search in LDS.
// Empty experts own no tiles; an overflowing expert owns ceil(C / BM).  The
// grid is persistent: each workgroup strides over tile indices, so the grid
// never depends on the routing and no host synchronisation is needed.
//
// bf16 kernel: 512 threads = 8 waves, block tile BM x BN x BK =
// 256 x 256 x 64, wave tile 128 x 64 = 4 x 2 MFMA v_mfma_f32_32x32x16_bf16
// blocks, one workgroup per CU (two LDS stages of A and B, ~147 KB of the
// 160 KB LDS).  Operands are staged global -> registers -> LDS (rows padded
// to 72 elements, so the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks); the next k-tile's global loads are in flight while the
// current one is multiplied, with one barrier per k-tile.  A wave skips the
// MFMAs of 32-row blocks that lie past the end of its expert's rows.
//
// SwiGLU needs gate and up of the same output column in the same lane: the
// B tile of a wave column holds 32 gate rows then the 32 matching up rows,
// so acc[.][0] and acc[.][1] hold g and u of identical (row, column); a
// 256-row B tile yields 128 output columns.
//
// e4m3 weights are widened to bf16 exactly while being staged into LDS (the
// hardware converts OCP e4m3 to float32; every e4m3 value is a bf16 value)
// and the per-row scale multiplies the float32 accumulator.
#include "common.h"

namespace rde {
namespace {

constexpr int BM = kGemmBM, BN = 256, BK = 64, LDK = BK + 8;
constexpr int kThreads = 512;   // 8 waves: 2 (M) x 4 (N)
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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// 4 e4m3 codes (one dword) -> 4 bf16 (two dwords), exact.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
    typedef float __attribute__((ext_vector_type(2))) f2;
    const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return make_uint2(pack_bf16x2(lo.x, lo.y), pack_bf16x2(hi.x, hi.y));
}

// 16 e4m3 codes -> 16 bf16 written to LDS (two 16-byte stores).
__device__ __forceinline__ void stage_e4m3(__bf16* dst, uint4 v) {
    const uint2 p0 = e4m3x4_to_bf16x4(v.x), p1 = e4m3x4_to_bf16x4(v.y);
    const uint2 p2 = e4m3x4_to_bf16x4(v.z), p3 = e4m3x4_to_bf16x4(v.w);
    *(uint4*)dst = make_uint4(p0.x, p0.y, p1.x, p1.y);
    *(uint4*)(dst + 8) = make_uint4(p2.x, p2.y, p3.x, p3.y);
}

// Block tile BM x BN x BK = 256 x 256 x 64, 8 waves.  Wave (wm, wn) owns
// the 32-row blocks wm, wm+2, wm+4, wm+6 (interleaved, so a half-filled
// tile keeps both M-waves busy) and B rows wn*64 .. wn*64+63.  The MFMA is
// issued as B x A^T so each lane ends with 4 consecutive output columns of
// one row (vector stores in the epilogue): for acc register r of a 32x32
// block, row = lane % 32, column = 8*(r/4) + 4*(lane/32) + r%4.
// LDS: two stages of A and B tiles, rows padded to 72 elements.
template <int EPI, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 sB[2][BN * LDK];
    __shared__ int32_t s_mt[kMaxGroupsLds + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const bool uniform = a.mt_off == nullptr;
    int total_mt, tiles_per_group = 0;
    if (uniform) {
        tiles_per_group = (a.uniform_rows + BM - 1) / BM;
        total_mt = tiles_per_group * a.n_groups;
    } else {
        for (int i = tid; i <= a.n_groups; i += kThreads) s_mt[i] = a.mt_off[i];
        __syncthreads();
        total_mt = s_mt[a.n_groups];
    }
    const int ntl = a.n_tiles;
    const int64_t total = (int64_t)total_mt * ntl;

    // Tiles are ordered (group, n-tile, m-tile) with the m-tile fastest, and
    // consecutive tile indices go to workgroups of one XCD (workgroups are
    // dealt round-robin over the 8 XCDs): the m-tiles sharing a weight tile
    // and the n-tiles sharing activation rows meet in the same L2.
    const int G = gridDim.x;
    const int vid = ((G & 7) == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;

    const __bf16* A = (const __bf16*)a.A;
    const char* Bb = (const char*)a.B;
    const int nk = a.K / BK;
    // global -> register staging plan: A 256 rows x 8 chunks of 16 B (4 per
    // thread); B bf16 likewise, B e4m3 256 rows x 4 chunks (2 per thread)
    const int ac = tid & 7, ar = tid >> 3;          // A: rows ar + 64*i
    const int bc = FP8 ? (tid & 3) : (tid & 7);
    const int br = FP8 ? (tid >> 2) : (tid >> 3);   // B: rows br + (FP8 ? 128 : 64)*i
    constexpr int BRS = FP8 ? 128 : 64;

    for (int64_t L = vid; L < total; L += G) {
        int g, cnt, ml, nt;
        if (uniform) {
            g = (int)(L / ((int64_t)tiles_per_group * ntl));
            const int loc = (int)(L - (int64_t)g * tiles_per_group * ntl);
            cnt = tiles_per_group;
            nt = loc / cnt;
            ml = loc - nt * cnt;
        } else {
            g = find_group(s_mt, a.n_groups, L, ntl);
            cnt = s_mt[g + 1] - s_mt[g];
            const int loc = (int)(L - (int64_t)s_mt[g] * ntl);
            nt = loc / cnt;
            ml = loc - nt * cnt;
        }
        int a_row0, rows;
        if (uniform) {
            a_row0 = ml * BM;
            rows = min(BM, a.uniform_rows - a_row0);
        } else {
            const int e0 = a.offsets[g], e1 = a.offsets[g + 1];
            a_row0 = e0 + ml * BM;
            rows = min(BM, e1 - a_row0);
        }

        const __bf16* ap0 = A + (int64_t)(a_row0 + min(ar, rows - 1)) * a.lda + ac * 8;
        const __bf16* ap1 = A + (int64_t)(a_row0 + min(ar + 64, rows - 1)) * a.lda + ac * 8;
        const __bf16* ap2 = A + (int64_t)(a_row0 + min(ar + 128, rows - 1)) * a.lda + ac * 8;
        const __bf16* ap3 = A + (int64_t)(a_row0 + min(ar + 192, rows - 1)) * a.lda + ac * 8;
        // byte offsets of this thread's B rows (bf16: 4 rows, e4m3: 2 rows)
        auto brow_of = [&](int r) {
            if (EPI == EPI_SWIGLU) {
                const int w2 = r >> 6, rr = r & 63;
                return (rr < 32) ? (nt * 128 + w2 * 32 + rr) : (a.I + nt * 128 + w2 * 32 + rr - 32);
            }
            return min(nt * BN + r, a.N_w - 1);   // rows past N (ragged last tile): clamped
        };
        const int64_t gbase = (int64_t)g * a.b_group_stride;
        const int esz = FP8 ? 1 : 2;
        const int64_t boff0 = (gbase + (int64_t)brow_of(br) * a.k_seg) * esz + bc * 16;
        const int64_t boff1 = (gbase + (int64_t)brow_of(br + BRS) * a.k_seg) * esz + bc * 16;
        const int64_t boff2 = FP8 ? 0 : (gbase + (int64_t)brow_of(br + 2 * BRS) * a.k_seg) * esz + bc * 16;
        const int64_t boff3 = FP8 ? 0 : (gbase + (int64_t)brow_of(br + 3 * BRS) * a.k_seg) * esz + bc * 16;

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        // waves whose 64 B rows lie past N (ragged last n-tile) do no work
        const bool col_ok = EPI == EPI_SWIGLU || nt * BN + wn * 64 < a.N_w;
        bool act[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) act[mb] = col_ok && 32 * (wm + 2 * mb) < rows;

        uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define RDE_LOAD(kt)                                                                     \
    do {                                                                                 \
        const int k0_ = (kt) * BK;                                                       \
        ra0 = *(const uint4*)(ap0 + k0_);                                                \
        ra1 = *(const uint4*)(ap1 + k0_);                                                \
        ra2 = *(const uint4*)(ap2 + k0_);                                                \
        ra3 = *(const uint4*)(ap3 + k0_);                                                \
        const int seg_ = k0_ / a.k_seg;                                                  \
        const int64_t so_ = ((int64_t)seg_ * a.b_seg_stride + (k0_ - seg_ * a.k_seg)) *  \
                            (FP8 ? 1 : 2);                                               \
        rb0 = *(const uint4*)(Bb + boff0 + so_);                                         \
        rb1 = *(const uint4*)(Bb + boff1 + so_);                                         \
        if (!FP8) {                                                                      \
            rb2 = *(const uint4*)(Bb + boff2 + so_);                                     \
            rb3 = *(const uint4*)(Bb + boff3 + so_);                                     \
        }                                                                                \
    } while (0)
#define RDE_STORE(buf)                                                                   \
    do {                                                                                 \
        __bf16* sa_ = sA[buf];                                                           \
        *(uint4*)&sa_[(ar)*LDK + ac * 8] = ra0;                                          \
        *(uint4*)&sa_[(ar + 64) * LDK + ac * 8] = ra1;                                   \
        *(uint4*)&sa_[(ar + 128) * LDK + ac * 8] = ra2;                                  \
        *(uint4*)&sa_[(ar + 192) * LDK + ac * 8] = ra3;                                  \
        __bf16* sb_ = sB[buf];                                                           \
        if (FP8) {                                                                       \
            stage_e4m3(sb_ + br * LDK + bc * 16, rb0);                                   \
            stage_e4m3(sb_ + (br + BRS) * LDK + bc * 16, rb1);                           \
        } else {                                                                         \
            *(uint4*)&sb_[br * LDK + bc * 8] = rb0;                                      \
            *(uint4*)&sb_[(br + BRS) * LDK + bc * 8] = rb1;                              \
            *(uint4*)&sb_[(br + 2 * BRS) * LDK + bc * 8] = rb2;                          \
            *(uint4*)&sb_[(br + 3 * BRS) * LDK + bc * 8] = rb3;                          \
        }                                                                                \
    } while (0)

        RDE_LOAD(0);
        RDE_STORE(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) RDE_LOAD(kt + 1);
            const __bf16* sa = sA[cur];
            const __bf16* sb = sB[cur];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int kof = ks * 16 + (lane >> 5) * 8;
                const bf16x8 b0 = *(const bf16x8*)&sb[(wn * 64 + (lane & 31)) * LDK + kof];
                const bf16x8 b1 = *(const bf16x8*)&sb[(wn * 64 + 32 + (lane & 31)) * LDK + kof];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    if (!act[mb]) continue;
                    const bf16x8 av =
                        *(const bf16x8*)&sa[((wm + 2 * mb) * 32 + (lane & 31)) * LDK + kof];
                    acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, av, acc[mb][0], 0, 0, 0);
                    acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, av, acc[mb][1], 0, 0, 0);
                }
            }
            if (kt + 1 < nk) RDE_STORE(cur ^ 1);
            __syncthreads();
        }
#undef RDE_LOAD
#undef RDE_STORE

        // ---- epilogue: lane owns row (lane % 32) of each active row block and
        // columns 8*i + 4*(lane/32) + 0..3 of each 32-column block ----
        const int c4 = 4 * (lane >> 5);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (!act[mb]) continue;
            const int row = (wm + 2 * mb) * 32 + (lane & 31);
            if (row >= rows) continue;
            const int64_t orow = (int64_t)a_row0 + row;
            if (EPI == EPI_SWIGLU) {
                const float* sc = FP8 ? a.bscale + (int64_t)g * a.N_w : nullptr;
                __bf16* o = (__bf16*)a.out + orow * a.ldo + (int64_t)g * a.out_col_per_group;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = nt * 128 + wn * 32 + 8 * i + c4;
                    float h[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float gv = acc[mb][0][4 * i + j], uv = acc[mb][1][4 * i + j];
                        if (FP8) {
                            gv *= sc[col + j];
                            uv *= sc[a.I + col + j];
                        }
                        h[j] = silu_mul(gv, uv);
                    }
                    *(uint2*)(o + col) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                }
            } else {
                float cw = 1.0f;
                int64_t drow = orow;
                if (EPI == EPI_COMBINE) {
                    const int32_t q = a.row_src[orow];
                    cw = a.route_w[q];
                    drow = q;
                }
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int col = nt * BN + wn * 64 + nb * 32 + 8 * i + c4;
                        float v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            v[j] = acc[mb][nb][4 * i + j];
                            if (FP8) v[j] *= a.bscale[(int64_t)g * a.N_w + col + j];
                            if (EPI == EPI_RELU2) v[j] = v[j] > 0.0f ? v[j] * v[j] : 0.0f;
                            if (EPI == EPI_COMBINE) v[j] *= cw;
                        }
                        if (EPI == EPI_F32) {
                            *(float4*)((float*)a.out + drow * a.ldo + col) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
                            const int64_t oc = EPI == EPI_RELU2 ? (int64_t)g * a.out_col_per_group + col : col;
                            *(uint2*)((__bf16*)a.out + drow * a.ldo + oc) =
                                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                        }
                    }
                }
            }
        }
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
#define RDE_GEMM_CASE(E)                                                                      \
    case E:                                                                                   \
        if (fp8) hipLaunchKernelGGL((gemm_bf16_kernel<E, true>), dim3(grid), dim3(kThreads), 0, s, a); \
        else hipLaunchKernelGGL((gemm_bf16_kernel<E, false>), dim3(grid), dim3(kThreads), 0, s, a);   \
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
