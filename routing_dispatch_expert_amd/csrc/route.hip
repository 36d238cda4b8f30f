// Top-k router: one wavefront per token (the routing itself is route_row in
// route_wave.h).
#include <type_traits>

#include "route_wave.h"

namespace rde {
namespace {

template <int EPL, bool SIG>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int renorm, float scale,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;  // wave-uniform
    float v[EPL];
    load_logits<EPL>(logits + (int64_t)t * E, E, lane, v);
    int id;
    float wt;
    route_row<EPL, SIG>(v, bias, E, k, renorm, scale, lane, id, wt);
    if (lane < k) {
        ids[(int64_t)t * k + lane] = id;
        w[(int64_t)t * k + lane] = wt;
    }
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int score_func, int renorm, float scale, int32_t* ids, float* w,
                        hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int waves = 4;
    dim3 grid((T + waves - 1) / waves), block(waves * kWave);
    auto go = [&](auto epl) {
        constexpr int EPL = decltype(epl)::value;
        if (score_func == MOE_SIGMOID)
            hipLaunchKernelGGL((route_kernel<EPL, true>), grid, block, 0, s, logits, bias, T, E, k,
                               renorm, scale, ids, w);
        else
            hipLaunchKernelGGL((route_kernel<EPL, false>), grid, block, 0, s, logits, bias, T, E,
                               k, renorm, scale, ids, w);
    };
    if (E <= 64) go(std::integral_constant<int, 1>{});
    else if (E <= 128) go(std::integral_constant<int, 2>{});
    else if (E <= 256) go(std::integral_constant<int, 4>{});
    else if (E <= 512) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
    return hipGetLastError();
}

}  // namespace rde
