// Combine: gate-weighted gather-reduce of the K expert outputs per token.
//
// "Anatomy of a high-performance EP kernel", the paragraph after the router
// figure: the expert GEMM runs where the activations landed and the results
// return to their tokens; SGLang "Expert Parallelism", "Framework Overview":
// post-permute, then combine.  out[t] = sum_k w[t,k] * y[row_of[t,k]] over
// the local slots, fp32 accumulation in ascending k, one rounding at the end.
//
// One block per (token, slice of 256 8-element vectors of the output row);
// each thread owns one vector and issues the loads of up to eight source
// rows before summing them, so a decode-sized batch spreads over the chip.
// Expert outputs are read once, with the non-temporal hint (measured faster
// than plain loads right after the down GEMM has written them; larger
// blocks were slower).
#include "device_common.hpp"
#include "launch.hpp"

namespace moeep {
namespace {

constexpr int kCombThreads = 256;
constexpr int kMaxKRegs = 8;       // slots whose rows are loaded together

__device__ __forceinline__ void load8(const void* y, int kind, size_t row, int c, int H, float* f) {
    if (kind == 0) {            // f32: two 16-byte vectors per 8 elements
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(y) + row * H) + 2 * c;
        const uint4 a = load_stream16(p), b = load_stream16(p + 1);
        f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z);
        f[3] = __uint_as_float(a.w); f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
        f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
    } else {                    // bf16
        const uint4 v = load_stream16(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y) + row * H) + c);
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
}

// kind: 0 = f32 -> f32, 1 = bf16 -> bf16, 2 = bf16 -> f32
template <int KIND>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const void* __restrict__ y, const int32_t* __restrict__ row_of, const float* __restrict__ w,
    int K, int H, int cap, void* __restrict__ out) {
    const int t = blockIdx.x;
    const int nvec = H / 8;
    const int c = blockIdx.y * blockDim.x + threadIdx.x;
    if (c >= nvec) return;
    const int32_t* rows = row_of + (size_t)t * K;
    const float* gates = w + (size_t)t * K;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k0 = 0; k0 < K; k0 += kMaxKRegs) {
        float v[kMaxKRegs][8];
        float g[kMaxKRegs];
        bool use[kMaxKRegs];
#pragma unroll
        for (int j = 0; j < kMaxKRegs; ++j) {
            const int k = k0 + j;
            const int r = k < K ? rows[k] : -1;
            use[j] = r >= 0 && r < cap;
            g[j] = use[j] ? gates[k] : 0.0f;
            if (use[j]) load8(y, KIND == 0 ? 0 : 1, (size_t)r, c, H, v[j]);
        }
#pragma unroll
        for (int j = 0; j < kMaxKRegs; ++j) {
            if (use[j]) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], v[j][i], acc[i]);
            }
        }
    }
    if (KIND == 1) {
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (size_t)t * H)[c] = o;
    } else {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H) + 2 * c;
        p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int kind, const int32_t* row_of, const float* w, int B,
                          int K, int H, void* out, int cap, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    // slices of at most kCombThreads vectors, balanced (a 360-vector row is two
    // slices of 180, not 256 + 104), in whole waves
    const int nvec = H / 8;
    const int nslice = (nvec + kCombThreads - 1) / kCombThreads;
    const int per = (nvec + nslice - 1) / nslice;
    const int nt = (per + kWave - 1) / kWave * kWave;
    dim3 grid(B, (nvec + nt - 1) / nt), block(nt);
    if (kind == 0)
        hipLaunchKernelGGL(combine_kernel<0>, grid, block, 0, stream, y, row_of, w, K, H, cap, out);
    else if (kind == 1)
        hipLaunchKernelGGL(combine_kernel<1>, grid, block, 0, stream, y, row_of, w, K, H, cap, out);
    else
        hipLaunchKernelGGL(combine_kernel<2>, grid, block, 0, stream, y, row_of, w, K, H, cap, out);
    return hipGetLastError();
}

}  // namespace moeep
