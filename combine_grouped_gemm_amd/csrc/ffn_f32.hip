// Grouped SwiGLU expert FFN in fp32 (the toy EP layer of "Anatomy of a
// high-performance EP kernel", section "What we have to do": E = 16 experts,
// K = 2, small hidden sizes, everything fp32).
//
// The sizes are tiny, so this is a plain FMA kernel: one block per (local
// expert, 64-column slice); thread (c, g) owns column c of the slice and the
// rows g, g + 4, ... of the expert, each a dot product over the contraction
// dimension.  Same semantics as the MFMA kernels (fp32 accumulation, h and y
// stored as fp32).
#include "grouped_tiles.hpp"

namespace moeep {
namespace {

constexpr int kCols = 64, kRowGroups = 4;

template <bool GATED>
__global__ __launch_bounds__(kCols * kRowGroups) void grouped_ffn_f32_kernel(FfnArgs p) {
    const int j = blockIdx.x;
    const int col = blockIdx.y * kCols + threadIdx.x % kCols;
    const int g = threadIdx.x / kCols;
    if (col >= p.N) return;
    int r0, r1;
    expert_rows(p, j, r0, r1);
    const float* A = static_cast<const float*>(p.a);
    const float* w0 = static_cast<const float*>(p.w0) + ((size_t)j * p.N + col) * p.Kdim;
    const float* w1 = GATED ? static_cast<const float*>(p.w1) + ((size_t)j * p.N + col) * p.Kdim : nullptr;
    float* Out = static_cast<float*>(p.out);
    for (int r = r0 + g; r < r1; r += kRowGroups) {
        const float* a = A + (size_t)r * p.Kdim;
        float s0 = 0.f, s1 = 0.f;
        for (int k = 0; k < p.Kdim; ++k) {
            s0 = fmaf(a[k], w0[k], s0);
            if (GATED) s1 = fmaf(a[k], w1[k], s1);
        }
        Out[(size_t)r * p.N + col] = GATED ? silu(s0) * s1 : s0;
    }
}

}  // namespace

hipError_t launch_ffn_f32(const FfnArgs& a, bool gated, hipStream_t stream) {
    dim3 grid(a.E_loc, (a.N + kCols - 1) / kCols), block(kCols * kRowGroups);
    if (gated)
        hipLaunchKernelGGL(grouped_ffn_f32_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(grouped_ffn_f32_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace moeep
