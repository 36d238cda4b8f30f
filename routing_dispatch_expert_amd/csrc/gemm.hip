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
// bf16 kernel: 256 threads = 4 waves in a 2 x 2 grid, block tile
// BM x BN x BK = 128 x 128 x 64, wave tile 64 x 64 = 2 x 2 MFMA
// v_mfma_f32_32x32x16_bf16 blocks.  Operands are staged global -> registers
// -> LDS (rows padded to 72 elements, so the 16-byte fragment reads of 8
// consecutive rows hit distinct banks); the next k-tile's global loads are
// in flight while the current one is multiplied.  A wave skips the MFMAs of
// 32-row blocks that lie past the end of its expert's rows.
//
// SwiGLU needs gate and up of the same output column in the same lane: the
// B tile of a wave column holds 32 gate rows then the 32 matching up rows,
// so acc[.][0] and acc[.][1] hold g and u of identical (row, column).
//
// e4m3 weights are widened to bf16 exactly while being staged into LDS (the
// hardware converts OCP e4m3 to float32; every e4m3 value is a bf16 value)
// and the per-row scale multiplies the float32 accumulator.
#include "common.h"

namespace rde {
namespace {

constexpr int BM = kGemmBM, BN = 128, BK = 64, LDK = BK + 8;
constexpr int kMaxGroupsLds = 1024;

__device__ __forceinline__ int find_group(const int32_t* s_mt, int n_groups, int mt) {
    // largest g with s_mt[g] <= mt (s_mt non-decreasing, s_mt[0] = 0)
    int lo = 0, hi = n_groups - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_mt[mid] <= mt) lo = mid;
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

template <int EPI, bool FP8>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 sA[BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 sB[BN * LDK];
    __shared__ int32_t s_mt[kMaxGroupsLds + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool uniform = a.mt_off == nullptr;
    int total_mt;
    int tiles_per_group = 0;
    if (uniform) {
        tiles_per_group = (a.uniform_rows + BM - 1) / BM;
        total_mt = tiles_per_group * a.n_groups;
    } else {
        for (int i = tid; i <= a.n_groups; i += blockDim.x) s_mt[i] = a.mt_off[i];
        __syncthreads();
        total_mt = s_mt[a.n_groups];
    }
    const int64_t total = (int64_t)total_mt * a.n_tiles;

    // XCD-aware order: workgroups are dealt round-robin over 8 XCDs; give
    // consecutive tile indices (same m-tile, neighbouring n-tiles, shared A
    // rows) to workgroups of one XCD so they meet in its L2.
    const int G = gridDim.x;
    int vid = blockIdx.x;
    if ((G & 7) == 0) vid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    const __bf16* A = (const __bf16*)a.A;
    const int nk = a.K / BK;

    for (int64_t tile = vid; tile < total; tile += G) {
        const int mt = (int)(tile / a.n_tiles);
        const int nt = (int)(tile - (int64_t)mt * a.n_tiles);
        int g, rows, a_row0, out_row0;
        if (uniform) {
            g = mt / tiles_per_group;
            const int ml = mt - g * tiles_per_group;
            a_row0 = ml * BM;
            out_row0 = a_row0;
            rows = min(BM, a.uniform_rows - a_row0);
        } else {
            g = find_group(s_mt, a.n_groups, mt);
            const int ml = mt - s_mt[g];
            const int e0 = a.offsets[g], e1 = a.offsets[g + 1];
            a_row0 = e0 + ml * BM;
            out_row0 = a_row0;
            rows = min(BM, e1 - a_row0);
        }

        // ---- per-thread global load plan ----
        // A: 128 rows x 8 chunks of 16 B; thread handles rows r = tid/8 + 32*i
        const int ac = tid & 7;
        const __bf16* a_ptr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            const int rr = r < rows ? r : rows - 1;
            a_ptr[i] = A + (int64_t)(a_row0 + rr) * a.lda + ac * 8;
        }
        // B rows of this tile
        const char* b_base = (const char*)a.B;
        const int esz = FP8 ? 1 : 2;
        int64_t b_row_off[4];  // element offset of the B row (within group, excluding K segments)
        constexpr int kBLoads = FP8 ? 2 : 4;
        const int bc = FP8 ? (tid & 3) : (tid & 7);
#pragma unroll
        for (int i = 0; i < kBLoads; ++i) {
            const int r = FP8 ? ((tid >> 2) + 64 * i) : ((tid >> 3) + 32 * i);
            int brow;
            if (EPI == EPI_SWIGLU) {
                const int w2 = r >> 6, rr = r & 63;
                brow = (rr < 32) ? (nt * 64 + w2 * 32 + rr) : (a.I + nt * 64 + w2 * 32 + rr - 32);
            } else {
                brow = nt * BN + r;
            }
            b_row_off[i] = (int64_t)g * a.b_group_stride + (int64_t)brow * a.k_seg;
        }

        uint4 ra[4], rb[4];
        auto load_tile = [&](int kt) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = *(const uint4*)(a_ptr[i] + k0);
            const int seg = k0 / a.k_seg;
            const int kl = k0 - seg * a.k_seg;
            const int64_t soff = (int64_t)seg * a.b_seg_stride + kl;
#pragma unroll
            for (int i = 0; i < kBLoads; ++i)
                rb[i] = *(const uint4*)(b_base + (b_row_off[i] + soff + (FP8 ? bc * 16 : bc * 8)) * esz);
        };
        auto store_tile = [&]() {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 3) + 32 * i;
                *(uint4*)&sA[r * LDK + ac * 8] = ra[i];
            }
            if (FP8) {
#pragma unroll
                for (int i = 0; i < kBLoads; ++i) {
                    const int r = (tid >> 2) + 64 * i;
                    const uint2 p0 = e4m3x4_to_bf16x4(rb[i].x), p1 = e4m3x4_to_bf16x4(rb[i].y);
                    const uint2 p2 = e4m3x4_to_bf16x4(rb[i].z), p3 = e4m3x4_to_bf16x4(rb[i].w);
                    *(uint4*)&sB[r * LDK + bc * 16] = make_uint4(p0.x, p0.y, p1.x, p1.y);
                    *(uint4*)&sB[r * LDK + bc * 16 + 8] = make_uint4(p2.x, p2.y, p3.x, p3.y);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kBLoads; ++i) {
                    const int r = (tid >> 3) + 32 * i;
                    *(uint4*)&sB[r * LDK + bc * 8] = rb[i];
                }
            }
        };

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        const bool act0 = wm * 64 < rows, act1 = wm * 64 + 32 < rows;

        load_tile(0);
        store_tile();
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) load_tile(kt + 1);
            if (act0) {
#pragma unroll
                for (int ks = 0; ks < BK / 16; ++ks) {
                    const int kof = ks * 16 + (lane >> 5) * 8;
                    const bf16x8 a0 = *(const bf16x8*)&sA[(wm * 64 + (lane & 31)) * LDK + kof];
                    const bf16x8 a1 = *(const bf16x8*)&sA[(wm * 64 + 32 + (lane & 31)) * LDK + kof];
                    const bf16x8 b0 = *(const bf16x8*)&sB[(wn * 64 + (lane & 31)) * LDK + kof];
                    const bf16x8 b1 = *(const bf16x8*)&sB[(wn * 64 + 32 + (lane & 31)) * LDK + kof];
                    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
                    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
                    if (act1) {
                        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
                        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
                    }
                }
            }
            __syncthreads();
            if (kt + 1 < nk) {
                store_tile();
                __syncthreads();
            }
        }

        // ---- epilogue ----
        const int cl = lane & 31;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            if (!(mb == 0 ? act0 : act1)) continue;
            if (EPI == EPI_SWIGLU) {
                const int col = nt * 64 + wn * 32 + cl;
                float sg = 1.0f, su = 1.0f;
                if (FP8) {
                    const float* sc = a.bscale + (int64_t)g * a.N_w;
                    sg = sc[col];
                    su = sc[a.I + col];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < rows) {
                        const float h = silu_mul(acc[mb][0][r] * sg, acc[mb][1][r] * su);
                        __bf16* o = (__bf16*)a.out + (int64_t)(out_row0 + row) * a.ldo +
                                    (int64_t)g * a.out_col_per_group + col;
                        *o = (__bf16)h;
                    }
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int col = nt * BN + wn * 64 + nb * 32 + cl;
                    const float sc = FP8 ? a.bscale[(int64_t)g * a.N_w + col] : 1.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (row >= rows) continue;
                        const float v = acc[mb][nb][r] * sc;
                        const int64_t orow = out_row0 + row;
                        if (EPI == EPI_RELU2) {
                            const float p = v > 0.0f ? v * v : 0.0f;
                            ((__bf16*)a.out)[orow * a.ldo + (int64_t)g * a.out_col_per_group + col] = (__bf16)p;
                        } else if (EPI == EPI_STORE) {
                            ((__bf16*)a.out)[orow * a.ldo + col] = (__bf16)v;
                        } else if (EPI == EPI_COMBINE) {
                            const int32_t q = a.row_src[orow];
                            ((__bf16*)a.out)[(int64_t)q * a.ldo + col] = (__bf16)(a.route_w[q] * v);
                        } else {  // EPI_F32
                            ((float*)a.out)[orow * a.ldo + col] = v;
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
            g = find_group(s_mt, a.n_groups, mt);
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
        if (fp8) hipLaunchKernelGGL((gemm_bf16_kernel<E, true>), dim3(grid), dim3(256), 0, s, a); \
        else hipLaunchKernelGGL((gemm_bf16_kernel<E, false>), dim3(grid), dim3(256), 0, s, a);   \
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
