// Top-K routing with renormalised softmax gates.
//
// Per token ("Anatomy of a high-performance EP kernel", section "What we
// have to do", router figure): the K largest of E logits, largest first,
// equal logits in ascending expert id; gates = softmax over the K picks.
//
// One wave per token.  Lane l keeps logits l, l+64, ... in registers as
// order-preserving 64-bit keys (value in the high word, inverted expert id
// in the low word), so one unsigned max selects the largest logit with the
// lowest id.  K rounds of "local max -> wave max (DPP row reductions, then
// one lane per row) -> owner clears its key" produce the picks in order; gates come from the selected
// values with fp32 expf, written coalesced at the end.  With a placement map
// (Moreh report, load balancing between GPUs: the router emits the renumbered
// expert ids) the chosen ids are written through it; selection and gates are
// unchanged.  With n_shared always-on experts (Moreh report, "Overview": a
// shared expert runs for every token regardless of routing) each output row
// gets n_shared more slots, ids E, E+1, ... with gate 1.
#include "device_common.hpp"
#include "launch.hpp"

namespace moeep {
namespace {

constexpr int kRouteWaves = 4;

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);     // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// 64-bit key of the lane that DPP control CTRL names within this lane's row
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave, the same in every lane: within each 16-lane DPP row
// by cross-lane moves in the VALU (partners lane ^ 1, lane ^ 2, then the
// half-row and row mirrors, as in row16_max), then across the four rows by
// reading one lane of each.  No LDS traffic, unlike a shuffle.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0xB1>(v));
    v = max_u64(v, dpp_u64<0x4E>(v));
    v = max_u64(v, dpp_u64<0x141>(v));
    v = max_u64(v, dpp_u64<0x140>(v));
    return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                   max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

template <int EPL>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const float* __restrict__ logits, int B, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ w, const int32_t* __restrict__ map, int n_shared) {
    // dynamic LDS: per wave K gate numerators, then per wave K ids
    extern __shared__ char smem[];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    float* s_val = reinterpret_cast<float*>(smem) + wave * K;
    int* s_id = reinterpret_cast<int*>(smem) + kRouteWaves * K + wave * K;
    const int t = blockIdx.x * kRouteWaves + wave;
    if (t >= B) return;                       // whole wave leaves together

    const float* row = logits + (size_t)t * E;
    uint64_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        int e = lane + j * kWave;
        key[j] = (e < E) ? (((uint64_t)order_key(row[e]) << 32) | (uint32_t)(0xffffffffu - e)) : 0ull;
    }

    float top = 0.0f, sum = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xffffffffu - (uint32_t)best);
        const float v = key_value((uint32_t)(best >> 32));
        if (k == 0) top = v;
        const float ex = expf(v - top);
        sum += ex;
        if (lane == (e & (kWave - 1))) {
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (j == (e >> 6)) key[j] = 0ull;
        }
        if (lane == 0) {
            s_val[k] = ex;
            s_id[k] = e;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const float inv = 1.0f / sum;
    const int ld = K + n_shared;                       // output row length
    for (int k = lane; k < ld; k += kWave) {
        const bool routed = k < K;
        ids[(size_t)t * ld + k] = routed ? (map != nullptr ? map[s_id[k]] : s_id[k]) : E + (k - K);
        w[(size_t)t * ld + k] = routed ? s_val[k] * inv : 1.0f;
    }
}

template <int EPL>
hipError_t launch_epl(const float* logits, int B, int E, int K, int32_t* ids, float* w,
                      const int32_t* map, int n_shared, hipStream_t stream) {
    dim3 grid((B + kRouteWaves - 1) / kRouteWaves), block(kRouteWaves * kWave);
    const size_t lds = (size_t)kRouteWaves * K * (sizeof(float) + sizeof(int));
    hipLaunchKernelGGL(route_kernel<EPL>, grid, block, lds, stream, logits, B, E, K, ids, w, map,
                       n_shared);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int B, int E, int K, int32_t* ids, float* w,
                        const int32_t* map, int n_shared, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1) return launch_epl<1>(logits, B, E, K, ids, w, map, n_shared, stream);
    if (epl <= 2) return launch_epl<2>(logits, B, E, K, ids, w, map, n_shared, stream);
    if (epl <= 4) return launch_epl<4>(logits, B, E, K, ids, w, map, n_shared, stream);
    if (epl <= 8) return launch_epl<8>(logits, B, E, K, ids, w, map, n_shared, stream);
    return launch_epl<16>(logits, B, E, K, ids, w, map, n_shared, stream);
}

}  // namespace moeep
