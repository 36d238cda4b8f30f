// Weighted combine back to token order (onnxruntime PR 33963 "Description":
// FP32 final routing/reduction; the fleet megakernel report's MOE_COMBINE
// step: weighted sum of the expert outputs of a token).
//
// One workgroup per token, 8 output columns per thread and step (16-byte
// loads of bf16 rows, the rows of up to 8 slots in flight together).  The k contributions are added in slot order in
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

// 8 consecutive elements of a row as loaded (one 16-byte load of bf16, two of float32)
template <typename T_>
struct Row8;
template <>
struct Row8<__bf16> {
    uint4 u;
};
template <>
struct Row8<float> {
    float4 a, b;
};
__device__ __forceinline__ Row8<__bf16> ld8(const __bf16* p) { return {*(const uint4*)p}; }
__device__ __forceinline__ Row8<float> ld8(const float* p) {
    return {*(const float4*)p, *(const float4*)(p + 4)};
}
template <typename T_>
__device__ __forceinline__ Row8<T_> zero8();
template <>
__device__ __forceinline__ Row8<__bf16> zero8<__bf16>() { return {make_uint4(0, 0, 0, 0)}; }
template <>
__device__ __forceinline__ Row8<float> zero8<float>() {
    return {make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)};
}
__device__ __forceinline__ void unpack8(const Row8<__bf16>& r, float* v) { load8((const __bf16*)&r.u, v); }
__device__ __forceinline__ void unpack8(const Row8<float>& r, float* v) { load8((const float*)&r.a, v); }

// Rows of up to this many slots are loaded before any of them is summed, so
// that a token's k rows cost one memory round trip instead of k.
constexpr int kCombineBatch = 8;

template <typename T_>
__global__ __launch_bounds__(256) void combine_kernel(const T_* __restrict__ y, int gather,
                                                      const int32_t* __restrict__ route_dst,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ y_shared,
                                                      T_* __restrict__ out, int k, int H) {
    __shared__ int64_t s_src[32];
    __shared__ float s_coef[32];
    const int t = blockIdx.x, tid = threadIdx.x;
    int my_bad = 0;
    if (tid < k) {
        const int64_t q = (int64_t)t * k + tid;
        // both loads in flight before either is used
        const int32_t rd = route_dst[q];
        const float cw = gather ? w[q] : 1.0f;
        my_bad = rd == -2;
        s_src[tid] = rd >= 0 ? (gather ? (int64_t)rd : q) : -1;
        s_coef[tid] = cw;
    }
    const bool bad = __syncthreads_or(my_bad) != 0;
    for (int c = tid * 8; c < H; c += blockDim.x * 8) {
        float acc[8] = {};
        Row8<float> sh;
        if (y_shared) sh = ld8(y_shared + (int64_t)t * H + c);
        for (int j0 = 0; j0 < k; j0 += kCombineBatch) {   // j0 <= 24: indexes below 32
            Row8<T_> r[kCombineBatch];
            bool ok[kCombineBatch];
#pragma unroll
            for (int jj = 0; jj < kCombineBatch; ++jj) {
                const int j = j0 + jj;
                const int64_t src = j < k ? s_src[j] : -1;
                ok[jj] = src >= 0;
                r[jj] = zero8<T_>();
                if (ok[jj]) r[jj] = ld8(y + src * H + c);
            }
            // summed in slot order; a slot without a row adds 0 * 0, which
            // leaves acc unchanged bit for bit (acc starts at +0 and is never -0)
#pragma unroll
            for (int jj = 0; jj < kCombineBatch; ++jj) {
                float v[8];
                unpack8(r[jj], v);
                const float cf = ok[jj] ? s_coef[j0 + jj] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(cf, v[i], acc[i]);
            }
        }
        if (y_shared) {
            float v[8];
            unpack8(sh, v);
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
