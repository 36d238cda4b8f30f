// Softmax top-k router: one wavefront per token.
//
// Operation (onnxruntime PR 33963 "Extend MoEPacked for Bolt ReLU-square
// routing and BF16 IQ2 precision", "Measured CUDA kernel latency": internal
// softmax routing; the fleet megakernel report's MOE_TOPK step: top-k as k
// rounds of a wave-wide maximum over the 64 lanes).
//
// Each lane holds E/64 logits (lane l holds experts l, l+64, ...: coalesced
// row loads).  The softmax max and sum are wave reductions.  Top-k is k rounds
// of a wave arg-max over a 64-bit key (order-preserving image of the float32
// logit) << 32 | ~expert, so a larger logit wins and equal logits resolve to
// the lower expert index; -0 is folded onto +0 and NaN maps to the lowest key.
#include "common.h"

namespace rde {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Order-preserving map float -> uint32 (larger float -> larger key), with -0
// folded onto +0 and NaN mapped to 0 (below -inf, whose key is 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 0u;
    uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t o) {
    return (o & 0x80000000u) ? __uint_as_float(o & 0x7FFFFFFFu) : __uint_as_float(~o);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int renorm, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;  // wave-uniform
    const float* row = logits + (int64_t)t * E;
    float v[EPL];
    uint64_t key[EPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? row[e] : -INFINITY;
        if (e < E) m = fmaxf(m, v[i]);  // fmaxf skips NaN
        key[i] = e < E ? (((uint64_t)order_key(v[i]) << 32) | (uint32_t)(~e)) : 0ull;
    }
    m = wave_max(m);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) s += expf(v[i] - m);
    s = wave_sum(s);

    int my_id = 0;
    float my_num = 0.0f, ssel = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (key[i] == best) key[i] = 0ull;  // taken: keys are unique
        const int e = (int)(~(uint32_t)best);
        const float num = expf(key_value((uint32_t)(best >> 32)) - m);
        ssel += num;
        if (lane == j) {
            my_id = e;
            my_num = num;
        }
    }
    if (lane < k) {
        ids[(int64_t)t * k + lane] = my_id;
        w[(int64_t)t * k + lane] = my_num / (renorm ? ssel : s);
    }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                        float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int waves = 4;
    dim3 grid((T + waves - 1) / waves), block(waves * kWave);
    if (E <= 64) hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (E <= 128) hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (E <= 256) hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (E <= 512) hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

}  // namespace rde
