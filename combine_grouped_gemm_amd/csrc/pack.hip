// Weight packing: copies weight rows to a padded row pitch (the layout the
// FFN kernels read when the weight dtype carries MOE_W_PACKED).  A one-time
// layout transform of this library, outside the layer's arithmetic: rows of
// row_bytes bytes move unchanged, bytes [row_bytes, ld_bytes) of every
// packed row are zero.
#include "launch.hpp"

namespace moeep {
namespace {

// one 4-byte word of the packed tensor per thread and grid-stride step
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint32_t* __restrict__ src, long long n_rows,
                                                        int row_words, int ld_words, uint32_t* __restrict__ dst) {
    const long long total = n_rows * ld_words;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const long long r = i / ld_words;
        const int c = (int)(i - r * ld_words);
        dst[i] = c < row_words ? src[r * row_words + c] : 0u;
    }
}

}  // namespace

hipError_t launch_pack_rows(const void* src, long long n_rows, int row_bytes, int ld_bytes, void* dst,
                            hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    const long long words = n_rows * (ld_bytes / 4);
    const long long want = (words + 255) / 256;
    const int grid = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(pack_rows_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint32_t*>(src),
                       n_rows, row_bytes / 4, ld_bytes / 4, static_cast<uint32_t*>(dst));
    return hipGetLastError();
}

}  // namespace moeep
