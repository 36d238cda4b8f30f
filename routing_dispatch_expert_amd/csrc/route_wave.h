// Per-wavefront top-k routing of one token, shared by the router kernel and
// the single-block dispatch of small batches.
//
// Operation (onnxruntime PR 33963 "Extend MoEPacked for Bolt ReLU-square
// routing and BF16 IQ2 precision", "Measured CUDA kernel latency": internal
// softmax routing, and the commit adding projected sigmoid routing with an
// FP32 selection-only correction bias; the fleet megakernel report's
// MOE_TOPK step: top-k as k rounds of a wave-wide maximum over the 64 lanes).
//
// Lane l holds experts l, l+64, ... of the token (coalesced row loads).  Top-k
// is k rounds of a wave arg-max over a 64-bit key (order-preserving image of
// the float32 selection key) << 32 | ~expert, so a larger key wins and equal
// keys resolve to the lower expert index; -0 is folded onto +0 and NaN maps to
// the lowest key.
//   softmax: key = logit; the softmax max and sum are wave reductions and a
//            selected weight is recomputed from the key itself.
//   sigmoid: score = sigma(logit) evaluated in double and rounded once to
//            float32, key = score + bias in float32; the weight of a selected
//            expert is its unbiased score, fetched from the owning lane.
#pragma once

#include "common.h"

namespace rde {

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

// The token's logits into this lane's registers (-inf past E).
template <int EPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, int lane,
                                            float (&v)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        v[i] = e < E ? row[e] : -INFINITY;
    }
}

// Route the token whose logits are in v.  On return lane j < k holds the
// slot-j expert in id and its weight (times scale) in wt.
template <int EPL, bool SIG>
__device__ __forceinline__ void route_row(float (&v)[EPL], const float* __restrict__ bias, int E,
                                          int k, int renorm, float scale, int lane, int& id,
                                          float& wt) {
    uint64_t key[EPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        float kf = v[i];
        if (SIG) {
            // sigma in double, one rounding to float32; the key adds the bias in float32
            v[i] = (float)(1.0 / (1.0 + exp(-(double)v[i])));
            kf = (bias != nullptr && e < E) ? v[i] + bias[e] : v[i];
        } else if (e < E) {
            m = fmaxf(m, v[i]);  // fmaxf skips NaN
        }
        key[i] = e < E ? (((uint64_t)order_key(kf) << 32) | (uint32_t)(~e)) : 0ull;
    }
    float s = 0.0f;
    if (!SIG) {
        m = wave_max(m);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + kWave * i < E) s += expf(v[i] - m);
        s = wave_sum(s);
    }
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
        float num;
        if (SIG) {
            // the score of expert e lives in lane e % 64, slot e / 64
            float mine = v[0];
#pragma unroll
            for (int i = 1; i < EPL; ++i)
                if (i == (e >> 6)) mine = v[i];
            num = __shfl(mine, e & (kWave - 1), kWave);
        } else {
            num = expf(key_value((uint32_t)(best >> 32)) - m);
        }
        ssel += num;
        if (lane == j) {
            my_id = e;
            my_num = num;
        }
    }
    const float den = renorm ? ssel : (SIG ? 1.0f : s);
    id = my_id;
    wt = my_num / den * scale;
}

}  // namespace rde
