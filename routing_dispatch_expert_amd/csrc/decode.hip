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
// For launches with few units, a workgroup of 4 wavefronts works on one unit
// at a time, each wavefront on a quarter of K; the four partial sums are
// added in LDS in wavefront order.
//
// Loads: each wavefront owns a private ring of kDStages LDS stages (8 KB:
// 32 activation rows and 32 weight rows of 128 bytes) filled by direct
// global -> LDS loads; it waits only on its own vector-memory counter (no
// workgroup barrier), so each wavefront keeps (kDStages - 1) x 8 KB in
// flight.  Within a 64-wide K group, lane half h supplies K elements
// [32h + 8j, 32h + 8j + 8) to MFMA step j (the same permutation of K for both
// operands leaves the product unchanged), so each lane's bytes for a group
// are one 64-byte run.  16-byte chunk c of row r sits at chunk slot
// c ^ ((r ^ r >> 3) & 7): the fragment reads are free of bank conflicts.
#include "common.h"

namespace rde {
namespace {

constexpr int kDWaves = 4;          // wavefronts per workgroup
constexpr int kDStages = 4;         // LDS ring stages per wavefront
constexpr int kDStage = 8192;       // bytes per stage: A 4 KB + B 4 KB
constexpr int kDGroupK = 64;        // K elements per stage

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

// Wait until at most n of this wavefront's vector-memory operations are
// outstanding (n = 8 x stages issued after the one needed).
__device__ __forceinline__ void wait_own(int stages_after) {
    if (stages_after >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (stages_after == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ int dswz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ float silu_mul_d(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint2 v) {
    typedef float __attribute__((ext_vector_type(2))) f2;
    const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
    const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
    const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
    const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
    const uint4 u = make_uint4(pack2(a.x, a.y), pack2(b.x, b.y), pack2(c.x, c.y), pack2(d.x, d.y));
    return __builtin_bit_cast(bf16x8, u);
}

// One unit segment of a launch (routed experts, or shared experts).
template <int EPI, bool FP8, bool SPLIT>
__device__ void run_unit(const DecodeSeg& s, const DecodeArgs& d, int group, int blk, int m0,
                         int rows, int row_base, unsigned char* ring, int lane, int wave,
                         float* red) {
    // SPLIT: this wavefront's share of the K groups (split-K over the
    // workgroup); otherwise the wavefront runs the whole unit alone
    const int nKall = s.K / kDGroupK;
    const int kq = SPLIT ? (nKall + kDWaves - 1) / kDWaves : nKall;
    const int g0 = SPLIT ? min(nKall, wave * kq) : 0, g1 = min(nKall, g0 + kq);
    const int nK = g1 - g0;
    const int mrows = min(32, rows - m0);
    const int r32 = lane & 31, h = lane >> 5;
    // ---- DMA plan: instruction i covers rows 8i + lane/8, chunk slot lane%8
    const int dr = lane >> 3, dsl = lane & 7;
    const char* asrc[4];
    const char* bsrc[4];
    const int esz_b = FP8 ? 1 : 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + dr;                 // row within the 32-row block
        const int c = dsl ^ dswz(r);              // logical chunk loaded into slot dsl
        // activation row
        const int m = min(r, mrows - 1);
        int64_t arow;
        if (s.offsets == nullptr) arow = (int64_t)(m0 + m);                        // uniform rows
        else if (s.gather) arow = (int64_t)(d.row_src[row_base + m0 + m] / d.k_top);  // token of the route
        else arow = (int64_t)(row_base + m0 + m);
        asrc[i] = (const char*)s.A + (arow * s.lda) * 2 + c * 16;
        // weight row
        int n;
        if (EPI == EPI_SWIGLU) n = r < 16 ? blk * 16 + r : s.I + blk * 16 + (r - 16);
        else n = min(blk * 32 + r, s.N_w - 1);
        // e4m3 rows hold 64 bytes per K group: chunk c < 4 only (slots >= 4 unused)
        bsrc[i] = (const char*)s.B + ((int64_t)group * s.b_group_stride + (int64_t)n * s.k_seg) * esz_b +
                  (FP8 ? (c & 3) * 16 : c * 16);
    }
    const uint32_t ring0 = __builtin_amdgcn_readfirstlane(lds_addr_d(ring));
    auto issue = [&](int gk) {
        const int k0 = (g0 + gk) * kDGroupK;
        const int seg = k0 / s.k_seg;
        const int64_t kb = (int64_t)seg * s.b_seg_stride + (k0 - seg * s.k_seg);
        const uint32_t st = ring0 + (gk % kDStages) * kDStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_d(asrc[i] + (int64_t)k0 * 2, __builtin_amdgcn_readfirstlane(st + i * 1024));
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_d(bsrc[i] + kb * esz_b, __builtin_amdgcn_readfirstlane(st + 4096 + i * 1024));
    };
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the ring are done
#pragma unroll
    for (int st = 0; st < kDStages - 1; ++st)
        if (st < nK) issue(st);
    for (int gk = 0; gk < nK; ++gk) {
        wait_own(min(kDStages - 2, nK - 1 - gk));
        const unsigned char* sa = ring + (gk % kDStages) * kDStage;
        const unsigned char* sb = sa + 4096;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * h + j;
            af[j] = *(const bf16x8*)(sa + r32 * 128 + ((c ^ dswz(r32)) * 16));
            if (FP8) {
                // 8 e4m3 codes at byte (32h + 8j) of the 64-byte row group
                const int byte = 32 * h + 8 * j;
                const int cc = byte >> 4;
                bfr[j] = e4m3x8_bf16(*(const uint2*)(sb + r32 * 128 + ((cc ^ dswz(r32)) * 16) + (byte & 15)));
            } else {
                bfr[j] = *(const bf16x8*)(sb + r32 * 128 + ((c ^ dswz(r32)) * 16));
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage read before it is refilled
        if (gk + kDStages - 1 < nK) issue(gk + kDStages - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[j], acc, 0, 0, 0);
    }

    // ---- sum the wavefronts' K shares in a fixed order (wave 0 first) ----
    if (SPLIT) {
    if (wave > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave - 1) * 16 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (wave != 0) {
        __syncthreads();  // wave 0 has read the partials
        return;
    }
#pragma unroll
    for (int w = 1; w < kDWaves; ++w)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += red[((w - 1) * 16 + r) * 64 + lane];
    __syncthreads();
    }

    // ---- epilogue: lane holds activation row m = lane % 32 ----
    const int m = r32;
    if (m >= mrows) return;
    const int64_t orow = (s.offsets == nullptr) ? (int64_t)(m0 + m) : (int64_t)(row_base + m0 + m);
    const int c4 = 4 * h;
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
            *(uint2*)(o + col) = make_uint2(pack2(hv[0], hv[1]), pack2(hv[2], hv[3]));
        }
        return;
    }
    float cw = 1.0f;
    int64_t drow = orow;
    if (EPI == EPI_COMBINE) {
        const int32_t q = d.row_src[orow];
        cw = d.route_w[q];
        drow = q;
    }
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
            *(uint2*)((__bf16*)s.out + drow * s.ldo + oc) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
        }
    }
}

// Units are numbered segment by segment; within a segment, group-major with
// the 32-row weight blocks fastest.  SPLIT: a workgroup takes one unit at a
// time and its wavefronts split the unit's K range (each streams a quarter of
// the weight rows through its own ring; the partial sums meet in LDS), for
// launches with fewer units than wavefronts.  Otherwise every wavefront takes
// units on its own (neighbouring wavefronts of a workgroup take neighbouring
// blocks of one expert and share its activation rows).  Units of experts
// without rows end at once.
template <int EPI0, int EPI1, bool FP8, bool SPLIT>
__global__ __launch_bounds__(kDWaves * 64, 1) void decode_gemm_kernel(DecodeArgs d) {
    __shared__ __attribute__((aligned(1024))) unsigned char rings[kDWaves][kDStages * kDStage];
    __shared__ float red[SPLIT ? (kDWaves - 1) * 16 * 64 : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)d.seg[0].n_groups * d.seg[0].blocks;
    const int64_t n1 = d.n_seg > 1 ? (int64_t)d.seg[1].n_groups * d.seg[1].blocks : 0;
    const int64_t first = SPLIT ? blockIdx.x : (int64_t)blockIdx.x * kDWaves + wave;
    const int64_t stride = SPLIT ? gridDim.x : (int64_t)gridDim.x * kDWaves;
    for (int64_t u = first; u < n0 + n1; u += stride) {
        const int si = u < n0 ? 0 : 1;
        const DecodeSeg& s = d.seg[si];
        const int64_t lu = si == 0 ? u : u - n0;
        const int group = (int)(lu / s.blocks), blk = (int)(lu - (int64_t)group * s.blocks);
        int rows, base;
        if (s.offsets) {
            base = s.offsets[group];
            rows = s.offsets[group + 1] - base;
        } else {
            base = 0;
            rows = s.uniform_rows;
        }
        if (rows <= 0) continue;  // uniform over the unit's wavefronts
        for (int m0 = 0; m0 < rows; m0 += 32) {
            if (si == 0) run_unit<EPI0, FP8, SPLIT>(s, d, group, blk, m0, rows, base, rings[wave], lane, wave, red);
            else run_unit<EPI1, false, SPLIT>(s, d, group, blk, m0, rows, base, rings[wave], lane, wave, red);
        }
    }
}

}  // namespace

hipError_t launch_decode_gemm(const DecodeArgs& d, int w_dtype, int split, int grid, hipStream_t st) {
    const bool fp8 = w_dtype == MOE_E4M3;
    const int e0 = d.seg[0].epi;
    const int e1 = d.n_seg > 1 ? d.seg[1].epi : ((e0 == EPI_SWIGLU || e0 == EPI_RELU2) ? EPI_SWIGLU : EPI_F32);
    dim3 g(grid), b(kDWaves * 64);
#define RDE_DEC(A, B)                                                                              \
    if (e0 == A && e1 == B) {                                                                      \
        if (fp8 && split) hipLaunchKernelGGL((decode_gemm_kernel<A, B, true, true>), g, b, 0, st, d);   \
        else if (fp8) hipLaunchKernelGGL((decode_gemm_kernel<A, B, true, false>), g, b, 0, st, d);      \
        else if (split) hipLaunchKernelGGL((decode_gemm_kernel<A, B, false, true>), g, b, 0, st, d);    \
        else hipLaunchKernelGGL((decode_gemm_kernel<A, B, false, false>), g, b, 0, st, d);              \
        return hipGetLastError();                                                                  \
    }
    RDE_DEC(EPI_SWIGLU, EPI_SWIGLU)
    RDE_DEC(EPI_RELU2, EPI_SWIGLU)
    RDE_DEC(EPI_COMBINE, EPI_F32)
    RDE_DEC(EPI_STORE, EPI_F32)
    RDE_DEC(EPI_F32, EPI_F32)
#undef RDE_DEC
    return hipErrorInvalidValue;
}

}  // namespace rde
