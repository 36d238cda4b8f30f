// Weighted combine back to token order (onnxruntime PR 33963 "Description":
// FP32 final routing/reduction; the fleet megakernel report's MOE_COMBINE
// step: weighted sum of the expert outputs of a token).
//
// One workgroup per token, 8 output columns per thread and step (16-byte
// loads of bf16 rows).  The k contributions are added in slot order in
// float32, then the shared-expert sum, and the result is rounded once.
//   gather form: contribution j = w[t,j] * y_disp[route_dst[t,j]]
//   slot form:   contribution j = ybuf[t*k + j] (weight applied upstream)
// Dropped routes (route_dst = -1) contribute nothing; a token holding a
// malformed route (route_dst = -2) gets a NaN row.
#include "common.h"

namespace rde {
namespace {

__device__ __forceinline__ void load8(const __bf16* p, float* v) {
    const uint4 u = *(const uint4*)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(__bf16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    }
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store8(float* p, const float* v) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T_>
__global__ __launch_bounds__(256) void combine_kernel(const T_* __restrict__ y, int gather,
                                                      const int32_t* __restrict__ route_dst,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ y_shared,
                                                      T_* __restrict__ out, int k, int H) {
    __shared__ int64_t s_src[32];
    __shared__ float s_coef[32];
    __shared__ int s_bad;
    const int t = blockIdx.x, tid = threadIdx.x;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (tid < k) {
        const int64_t q = (int64_t)t * k + tid;
        const int32_t rd = route_dst[q];
        if (rd == -2) atomicOr(&s_bad, 1);
        s_src[tid] = rd >= 0 ? (gather ? (int64_t)rd : q) : -1;
        s_coef[tid] = gather ? w[q] : 1.0f;
    }
    __syncthreads();
    const bool bad = s_bad != 0;
    for (int c = tid * 8; c < H; c += blockDim.x * 8) {
        float acc[8] = {};
        for (int j = 0; j < k; ++j) {
            const int64_t src = s_src[j];
            if (src < 0) continue;
            float v[8];
            load8(y + src * H + c, v);
            const float cf = s_coef[j];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(cf, v[i], acc[i]);
        }
        if (y_shared) {
            float v[8];
            load8(y_shared + (int64_t)t * H + c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
        if (bad) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_nanf("");
        }
        store8(out + (int64_t)t * H + c, acc);
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int gather, const int32_t* route_dst, const float* w,
                          const float* y_shared, void* out, int T, int k, int H, int act_dtype,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int threads = H / 8 >= 256 ? 256 : ((H / 8 + 63) / 64) * 64;
    if (act_dtype == MOE_F32)
        hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(threads), 0, s, (const float*)y, gather,
                           route_dst, w, y_shared, (float*)out, k, H);
    else
        hipLaunchKernelGGL(combine_kernel<__bf16>, dim3(T), dim3(threads), 0, s, (const __bf16*)y,
                           gather, route_dst, w, y_shared, (__bf16*)out, k, H);
    return hipGetLastError();
}

}  // namespace rde
