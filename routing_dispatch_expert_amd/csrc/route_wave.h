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
// is k rounds of: the wave maximum of the order-preserving 32-bit image of
// the float32 selection key over the experts not yet taken, then the lowest
// expert index holding that key (ballot, first set bit), so a larger key wins
// and equal keys resolve to the lower expert index; -0 is folded onto +0 and
// NaN maps to the lowest key.
//   softmax: key = logit; the softmax max and sum are wave reductions and a
//            selected weight is recomputed from the key itself.
//   sigmoid: score = sigma(logit) evaluated in double and rounded once to
//            float32, key = score + bias in float32; the weight of a selected
//            expert is its unbiased score, fetched from the owning lane.
#pragma once

#include "common.h"

namespace rde {

// Cross-lane exchange without the LDS: the value of lane (l ^ d) for the
// pairings a wave reduction needs.  Within a row of 16 lanes DPP moves pair
// lanes l ^ 1 and l ^ 2 (quad permutations), then the other half of each
// 8-lane group (row_half_mirror, i <-> 7 - i) and the other half of the row
// (row_mirror, i <-> 15 - i); gfx950's permlane swaps pair rows (l ^ 16) and
// halves (l ^ 32).  After the six steps every lane has combined all 64 lanes,
// and each step adds or compares a lane with one partner, so all lanes end
// with identical bits.
enum XStep { X_Q1 = 0xB1, X_Q2 = 0x4E, X_HALF = 0x141, X_ROW = 0x140, X_16 = 16, X_32 = 32 };
template <int S>
__device__ __forceinline__ uint32_t xlane(uint32_t v, int lane) {
    if (S == X_16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else if (S == X_32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    } else {
        return __builtin_amdgcn_update_dpp(0u, v, S, 0xf, 0xf, false);
    }
}

template <int S>
__device__ __forceinline__ float xmax_step(float v, int lane) {
    return fmaxf(v, __uint_as_float(xlane<S>(__float_as_uint(v), lane)));
}
template <int S>
__device__ __forceinline__ float xsum_step(float v, int lane) {
    return v + __uint_as_float(xlane<S>(__float_as_uint(v), lane));
}
__device__ __forceinline__ float wave_max(float v) {
    const int lane = threadIdx.x & (kWave - 1);
    v = xmax_step<X_Q1>(v, lane);
    v = xmax_step<X_Q2>(v, lane);
    v = xmax_step<X_HALF>(v, lane);
    v = xmax_step<X_ROW>(v, lane);
    v = xmax_step<X_16>(v, lane);
    return xmax_step<X_32>(v, lane);
}

__device__ __forceinline__ float wave_sum(float v) {
    const int lane = threadIdx.x & (kWave - 1);
    v = xsum_step<X_Q1>(v, lane);
    v = xsum_step<X_Q2>(v, lane);
    v = xsum_step<X_HALF>(v, lane);
    v = xsum_step<X_ROW>(v, lane);
    v = xsum_step<X_16>(v, lane);
    return xsum_step<X_32>(v, lane);
}

__device__ __forceinline__ int wave_sum_i32(int v) {
    const int lane = threadIdx.x & (kWave - 1);
    v += (int)xlane<X_Q1>((uint32_t)v, lane);
    v += (int)xlane<X_Q2>((uint32_t)v, lane);
    v += (int)xlane<X_HALF>((uint32_t)v, lane);
    v += (int)xlane<X_ROW>((uint32_t)v, lane);
    v += (int)xlane<X_16>((uint32_t)v, lane);
    return v + (int)xlane<X_32>((uint32_t)v, lane);
}

template <int S>
__device__ __forceinline__ uint32_t xmaxu_step(uint32_t v, int lane) {
    const uint32_t o = xlane<S>(v, lane);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    const int lane = threadIdx.x & (kWave - 1);
    v = xmaxu_step<X_Q1>(v, lane);
    v = xmaxu_step<X_Q2>(v, lane);
    v = xmaxu_step<X_HALF>(v, lane);
    v = xmaxu_step<X_ROW>(v, lane);
    v = xmaxu_step<X_16>(v, lane);
    return xmaxu_step<X_32>(v, lane);
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
    uint32_t key[EPL];
    uint32_t avail = 0;   // bit i: expert lane + 64 i exists and is not yet taken
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
        key[i] = order_key(kf);
        if (e < E) avail |= 1u << i;
    }
    float s = 0.0f;
    if (!SIG) {
        m = wave_max(m);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + kWave * i < E) s += expf(v[i] - m);
        s = wave_sum(s);
    }
    // lane j keeps slot j: its expert and either its score (sigmoid) or its
    // selection key, whose exponential is taken once after the k rounds
    int my_id = 0;
    uint32_t my_key = 0;
    float my_num = 0.0f;
    for (int j = 0; j < k; ++j) {
        // the largest key among the available experts, then the lowest
        // expert index holding it (wave-uniform: ballot and first set bit)
        uint32_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if ((avail >> i) & 1) best = key[i] > best ? key[i] : best;
        best = wave_max_u32(best);
        int e = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const uint64_t b = __ballot(((avail >> i) & 1) && key[i] == best);
            if (b) {
                e = kWave * i + __builtin_ctzll(b);
                break;
            }
        }
        if (lane == (e & (kWave - 1))) avail &= ~(1u << (e >> 6));   // taken
        if (SIG) {
            // the score of expert e lives in lane e % 64, slot e / 64
            float mine = v[0];
#pragma unroll
            for (int i = 1; i < EPL; ++i)
                if (i == (e >> 6)) mine = v[i];
            const float num = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & (kWave - 1)));
            if (lane == j) my_num = num;
        } else if (lane == j) {
            my_key = best;
        }
        if (lane == j) my_id = e;
    }
    if (!SIG) my_num = expf(key_value(my_key) - m);   // meaningful on lanes < k
    // the selected weights summed in slot order
    float ssel = 0.0f;
    if (renorm)
        for (int j = 0; j < k; ++j) ssel += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_num), j));
    const float den = renorm ? ssel : (SIG ? 1.0f : s);
    id = my_id;
    wt = my_num / den * scale;
}

}  // namespace rde
