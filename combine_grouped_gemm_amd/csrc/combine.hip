// Combine: gate-weighted gather-reduce of the K expert outputs per token.
//
// "Anatomy of a high-performance EP kernel", the paragraph after the router
// figure: the expert GEMM runs where the activations landed and the results
// return to their tokens; SGLang "Expert Parallelism", "Framework Overview":
// post-permute, then combine.  out[t] = sum_k w[t,k] * y[row_of[t,k]] over
// the local slots, fp32 accumulation in ascending k, one rounding at the end.
//
// One block per (token, slice of at most 256 8-element vectors of the
// output row); each thread owns one vector.  The token's slots are read 64 at
// a time with one vector load per wave (lane l holds slot l's row and gate),
// so the expert-output loads of the local slots are issued back to back, four
// at a time, before they are summed; a chain of one scalar load per slot
// ahead of each row load was measured 6-13% slower at every size but decode.
// Four rows at a time keep the kernel under 50 VGPRs: eight (80-90 VGPRs,
// fewer waves per SIMD) was slower.  Expert outputs are read once, with the
// non-temporal hint (measured faster than plain loads right after the down
// GEMM has written them).
#include "device_common.hpp"
#include "launch.hpp"

namespace moeep {
namespace {

constexpr int kCombThreads = 256;
constexpr int kMaxKRegs = 4;       // slots whose rows are loaded together

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

// Sum of the local slots' weighted rows for this thread's vector c, slots
// taken 64 at a time (lane l of the wave holds slot k0 + l's row, -1 when not
// local, and its gate: one vector load each), the rows of up to kMaxKRegs
// slots loaded back to back before they are summed, in ascending k.
// ALL_LANES: the masks need every lane of the wave (more than 64 slots);
// otherwise lanes past the row may leave once the first mask is taken.
template <int KIND, bool ALL_LANES>
__device__ __forceinline__ void combine_token(const void* __restrict__ y, const int32_t* __restrict__ row_of,
                                              const float* __restrict__ w, int t, int K, int H, int cap,
                                              int c, bool live, int lane, void* __restrict__ out) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k0 = 0; k0 < K; k0 += kWave) {
        int my = -1;
        float myg = 0.0f;
        const int kl = k0 + lane;
        if (kl < K) {
            const int r = row_of[(size_t)t * K + kl];
            if (r >= 0 && r < cap) {
                my = r;
                myg = w[(size_t)t * K + kl];
            }
        }
        uint64_t m = ballot64(my >= 0);
        if (!ALL_LANES && !live) return;
        while (m != 0) {
            float v[kMaxKRegs][8];
            float g[kMaxKRegs];
            int n = 0;
#pragma unroll
            for (int j = 0; j < kMaxKRegs; ++j) {
                if (m != 0) {                            // wave-uniform
                    const int k = __builtin_ctzll(m);
                    m &= m - 1;
                    const int r = __builtin_amdgcn_readlane(my, k);
                    g[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myg), k));
                    if (!ALL_LANES || live) load8(y, KIND == 0 ? 0 : 1, (size_t)r, c, H, v[j]);
                    n = j + 1;
                }
            }
            if (!ALL_LANES || live) {
#pragma unroll
                for (int j = 0; j < kMaxKRegs; ++j) {
                    if (j < n) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], v[j][i], acc[i]);
                    }
                }
            }
        }
    }
    if (!live) return;
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

// kind: 0 = f32 -> f32, 1 = bf16 -> bf16, 2 = bf16 -> f32
template <int KIND, bool ALL_LANES>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const void* __restrict__ y, const int32_t* __restrict__ row_of, const float* __restrict__ w,
    int K, int H, int cap, void* __restrict__ out) {
    const int c = blockIdx.y * blockDim.x + threadIdx.x;
    combine_token<KIND, ALL_LANES>(y, row_of, w, blockIdx.x, K, H, cap, c, c < H / 8, threadIdx.x % kWave, out);
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
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, stream, y, row_of, w, K, H, cap, out); };
    const bool small = K <= kWave;
    if (kind == 0) small ? go(combine_kernel<0, false>) : go(combine_kernel<0, true>);
    else if (kind == 1) small ? go(combine_kernel<1, false>) : go(combine_kernel<1, true>);
    else small ? go(combine_kernel<2, false>) : go(combine_kernel<2, true>);
    return hipGetLastError();
}

}  // namespace moeep
