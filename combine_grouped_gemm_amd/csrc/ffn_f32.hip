// Grouped SwiGLU expert FFN in fp32 (the toy EP layer of "Anatomy of a
// high-performance EP kernel", section "What we have to do": E = 16 experts,
// K = 2, small hidden sizes, everything fp32).
//
// The sizes are tiny, so this is an FMA kernel with LDS tiles: one block per
// (local expert, 64-column slice).  Per 64-wide k-chunk the block loads the
// slice's weight rows and up to 32 of the expert's rows into LDS with
// coalesced 16-byte loads; thread (c, g) then owns column c and the rows
// g, g + 4, ... of the row block and accumulates in ascending k.  Same
// semantics as the MFMA kernels (fp32 accumulation, h and y stored as fp32).
// The contraction dimension is a multiple of 8 (checked by the C ABI); the
// 16-byte chunks past it in the last k-chunk are read as zero.
#include "grouped_tiles.hpp"

namespace moeep {
namespace {

constexpr int kCols = 64;          // output columns per block
constexpr int kRowGroups = 4;      // threads per column
constexpr int kChunk = 64;         // k-chunk
constexpr int kRowBlock = 32;      // rows per pass
constexpr int kThreads = kCols * kRowGroups;
constexpr int kRowsPerThread = kRowBlock / kRowGroups;

template <bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_ffn_f32_kernel(FfnArgs p) {
    // weight rows padded to 65 floats: the 64 threads of a wave read 64 different
    // rows at the same k, which then fall into distinct banks
    __shared__ float sW0[kCols][kChunk + 1];
    __shared__ float sW1[GATED ? kCols : 1][kChunk + 1];
    __shared__ __align__(16) float sA[kRowBlock][kChunk];   // float4 stores

    const int j = blockIdx.x;
    const int col0 = blockIdx.y * kCols;
    const int tid = threadIdx.x, c = tid % kCols, g = tid / kCols;
    const int N = p.N, Kdim = p.Kdim, ldw = p.ldw;
    int r0, r1;
    expert_rows(p, j, r0, r1);
    const float* A = static_cast<const float*>(p.a);
    const float* W0 = static_cast<const float*>(p.w0) + (size_t)j * N * ldw;
    const float* W1 = GATED ? static_cast<const float*>(p.w1) + (size_t)j * N * ldw : nullptr;
    float* Out = static_cast<float*>(p.out);

    for (int rb = r0; rb < r1; rb += kRowBlock) {
        float acc0[kRowsPerThread], acc1[kRowsPerThread];
#pragma unroll
        for (int q = 0; q < kRowsPerThread; ++q) acc0[q] = acc1[q] = 0.f;
        for (int k0 = 0; k0 < Kdim; k0 += kChunk) {
            __syncthreads();      // the previous chunk's reads are done
            // weight tile: kCols rows x kChunk floats, 16 float4 per row
            for (int i = tid; i < kCols * kChunk / 4; i += kThreads) {
                const int cc = i / (kChunk / 4), k4 = (i % (kChunk / 4)) * 4;
                const int col = col0 + cc;
                float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
                if (col < N && k0 + k4 < Kdim) {      // chunks past K (a partial last chunk) are zero
                    v0 = *reinterpret_cast<const float4*>(W0 + (size_t)col * ldw + k0 + k4);
                    if (GATED) v1 = *reinterpret_cast<const float4*>(W1 + (size_t)col * ldw + k0 + k4);
                }
                sW0[cc][k4] = v0.x; sW0[cc][k4 + 1] = v0.y; sW0[cc][k4 + 2] = v0.z; sW0[cc][k4 + 3] = v0.w;
                if (GATED) {
                    sW1[cc][k4] = v1.x; sW1[cc][k4 + 1] = v1.y; sW1[cc][k4 + 2] = v1.z; sW1[cc][k4 + 3] = v1.w;
                }
            }
            // row block: kRowBlock rows x kChunk floats (rows past the expert's read as 0)
            for (int i = tid; i < kRowBlock * kChunk / 4; i += kThreads) {
                const int rr = i / (kChunk / 4), k4 = (i % (kChunk / 4)) * 4;
                const int r = rb + rr;
                const float4 v = r < r1 && k0 + k4 < Kdim
                                     ? *reinterpret_cast<const float4*>(A + (size_t)r * Kdim + k0 + k4)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4*>(&sA[rr][k4]) = v;
            }
            __syncthreads();
#pragma unroll 8
            for (int kk = 0; kk < kChunk; ++kk) {
                const float w0 = sW0[c][kk];
                const float w1 = GATED ? sW1[c][kk] : 0.f;
#pragma unroll
                for (int q = 0; q < kRowsPerThread; ++q) {
                    const float a = sA[g + kRowGroups * q][kk];     // same address across the wave
                    acc0[q] = fmaf(a, w0, acc0[q]);
                    if (GATED) acc1[q] = fmaf(a, w1, acc1[q]);
                }
            }
        }
        const int col = col0 + c;
        if (col < N) {
#pragma unroll
            for (int q = 0; q < kRowsPerThread; ++q) {
                const int r = rb + g + kRowGroups * q;
                if (r < r1) Out[(size_t)r * N + col] = GATED ? silu(acc0[q]) * acc1[q] : acc0[q];
            }
        }
    }
}

}  // namespace

hipError_t launch_ffn_f32(const FfnArgs& a, bool gated, hipStream_t stream) {
    dim3 grid(a.E_loc, (a.N + kCols - 1) / kCols), block(kThreads);
    if (gated)
        hipLaunchKernelGGL(grouped_ffn_f32_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(grouped_ffn_f32_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace moeep
