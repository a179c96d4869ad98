// Dispatch: scatter token rows into the dense expert-contiguous buffer.
//
// "Anatomy of a high-performance EP kernel", section "Dispatch": the tokens
// bound for the local experts are packed into one dense buffer so the
// grouped GEMM consumes them in a single call.  Tokens live on simulated
// source ranks (segments), as in the data-parallel attention setting of the
// same post's "What we have to do".
//
// One block per (source token, slice of up to 448 16-byte vectors of its
// row; a row of at most 448 vectors is one block of whole waves): each
// thread reads one vector from HBM once and writes it to every local
// destination row of the token, so a decode-sized batch still spreads over
// the whole chip.  The token's destination rows are read with one vector
// load per wave (lane k holds slot k's row; a ballot gives the local slots)
// instead of a chain of dependent scalar loads ahead of the row load (EP
// share 28 -> 23 us).  A token with no slot on the local experts is not read
// at all.  Plain stores: the non-temporal hint made this kernel slower in the
// layer's sequence.  For fp8 storage the token is quantised once per
// 128-element block (the 16 lanes of a DPP row cover a block; amax by
// cross-lane moves inside the row) and every copy receives the same codes
// and scale.
#include "device_common.hpp"
#include "launch.hpp"

namespace moeep {
namespace {

constexpr int kDispThreads = 448;      // most threads per block (7 waves: a 7168-element bf16 row is two blocks)

// Threads per block for rows of nvec 16-byte vectors: whole waves, at most
// kDispThreads; a multiple of 16 lanes, so fp8 scale blocks never straddle blocks.
inline int dispatch_threads(int nvec) {
    const int w = (nvec + kWave - 1) / kWave * kWave;
    return w < kDispThreads ? w : kDispThreads;
}

// Slots [k0, k0 + 64) of a token, one per lane: lane l holds row_of[t, k0 + l]
// when that slot exists and its row is in this buffer, else -1.  One vector
// load per wave, so no chain of dependent scalar loads precedes the token row.
__device__ __forceinline__ int slot_row(const int32_t* rows, int K, int k0, int cap, int lane) {
    const int k = k0 + lane;
    if (k >= K) return -1;
    const int r = rows[k];
    return (r >= 0 && r < cap) ? r : -1;
}

// Rows of token t in the segment-major concatenation: its segment is the
// number of segment starts at or below t (independent compares, no early exit).
__device__ __forceinline__ const void* token_row(const SegTable& seg, int t, size_t row_bytes) {
    int i = 0;
    for (int s = 1; s < seg.n; ++s) i += t >= seg.start[s] ? 1 : 0;
    return static_cast<const char*>(seg.ptr[i]) + (size_t)(t - seg.start[i]) * row_bytes;
}

// Whether any slot of the token is local (uniform over the block), looking at
// 64 slots per vector load.
__device__ __forceinline__ bool any_local(const int32_t* rows, int K, int cap, int lane) {
    for (int k0 = 0; k0 < K; k0 += kWave)
        if (ballot64(slot_row(rows, K, k0, cap, lane) >= 0) != 0) return true;
    return false;
}

// 16-byte copies (f32 -> f32, bf16 -> bf16).
__global__ __launch_bounds__(kDispThreads) void dispatch_copy_kernel(
    SegTable seg, size_t row_bytes, const int32_t* __restrict__ row_of, int K, int cap,
    char* __restrict__ xd) {
    const int t = blockIdx.x;
    const int c = blockIdx.y * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x % kWave;
    const int nvec = (int)(row_bytes / 16);
    const int32_t* rows = row_of + (size_t)t * K;
    int my = slot_row(rows, K, 0, cap, lane);
    uint64_t m = ballot64(my >= 0);          // local slots among the first 64, the same in every wave
    if (m == 0 && (K <= kWave || !any_local(rows, K, cap, lane))) return;
    // lanes past the row stay: with more than 64 slots each later ballot needs
    // every lane of the wave (lane l holds slot k0 + l)
    const bool ok = c < nvec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = static_cast<const uint4*>(token_row(seg, t, row_bytes))[c];
    for (int k0 = 0;;) {
        while (m != 0) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int r = __builtin_amdgcn_readlane(my, k);
            if (ok) reinterpret_cast<uint4*>(xd + (size_t)r * row_bytes)[c] = v;
        }
        k0 += kWave;
        if (k0 >= K) break;
        my = slot_row(rows, K, k0, cap, lane);
        m = ballot64(my >= 0);
    }
}

// bf16 -> fp8 e4m3 with one fp32 scale per 128 elements.  A block's slice
// starts at a multiple of 16 vectors, so the 16 vectors of a scale block are
// the 16 lanes of one DPP row of a wave.
__global__ __launch_bounds__(kDispThreads) void dispatch_fp8_kernel(
    SegTable seg, int H, const int32_t* __restrict__ row_of, int K, int cap,
    uint8_t* __restrict__ xd, float* __restrict__ xd_scales) {
    const int t = blockIdx.x;
    const int c = blockIdx.y * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x % kWave;
    const int nvec = H / 8;                 // 8 bf16 per 16-byte vector
    const int nblk = (H + 127) / 128;
    const int32_t* rows = row_of + (size_t)t * K;
    int my = slot_row(rows, K, 0, cap, lane);
    uint64_t m = ballot64(my >= 0);
    // whole block: the DPP rows below stay complete
    if (m == 0 && (K <= kWave || !any_local(rows, K, cap, lane))) return;
    const bool ok = c < nvec;
    const uint4* src = static_cast<const uint4*>(token_row(seg, t, (size_t)H * 2));
    const uint4 v = ok ? src[c] : make_uint4(0, 0, 0, 0);
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = row16_max(amax);
    // lanes past the row stay for the later slot ballots (more than 64 slots)
    const float s = pow2_block_scale(amax);
    const float rs = 1.0f / s;               // exact: s is a power of two
    // |f * rs| <= amax / s <= 448, the range where the hardware conversion is exact RNE
    const uint32_t lo = e4m3_pair(f[0] * rs, f[1] * rs) | (e4m3_pair(f[2] * rs, f[3] * rs) << 16);
    const uint32_t hi = e4m3_pair(f[4] * rs, f[5] * rs) | (e4m3_pair(f[6] * rs, f[7] * rs) << 16);
    for (int k0 = 0;;) {
        while (m != 0) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int r = __builtin_amdgcn_readlane(my, k);
            if (ok) {
                reinterpret_cast<uint2*>(xd + (size_t)r * H)[c] = make_uint2(lo, hi);
                if ((c & 15) == 0) xd_scales[(size_t)r * nblk + c / 16] = s;
            }
        }
        k0 += kWave;
        if (k0 >= K) break;
        my = slot_row(rows, K, k0, cap, lane);
        m = ballot64(my >= 0);
    }
}

}  // namespace

hipError_t launch_dispatch(const SegTable& seg, int B, int H, int kind, const int32_t* row_of,
                           int K, void* xd, float* xd_scales, int cap, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    if (kind == 0 || kind == 1) {
        const size_t row_bytes = (size_t)H * (kind == 0 ? 4 : 2);
        const int nvec = (int)(row_bytes / 16);
        const int nt = dispatch_threads(nvec);
        dim3 grid(B, (nvec + nt - 1) / nt);
        hipLaunchKernelGGL(dispatch_copy_kernel, grid, dim3(nt), 0, stream, seg,
                           row_bytes, row_of, K, cap, static_cast<char*>(xd));
    } else {
        const int nt = dispatch_threads(H / 8);
        dim3 grid(B, (H / 8 + nt - 1) / nt);
        hipLaunchKernelGGL(dispatch_fp8_kernel, grid, dim3(nt), 0, stream, seg, H,
                           row_of, K, cap, static_cast<uint8_t*>(xd), xd_scales);
    }
    return hipGetLastError();
}

}  // namespace moeep
