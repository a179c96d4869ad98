// Expert-contiguous layout of the routed slots: histogram, exclusive scan,
// stable permutation.
//
// "Anatomy of a high-performance EP kernel", section "Dispatch": each expert
// receives its own number of rows and the grouped GEMM runs over one row set
// per expert; SGLang "Expert Parallelism", "Framework Overview": the
// pre-permute stage in front of the grouped GEMM.
//
// The flattened slots s = t*K + k are cut into chunks of kChunk.  Three
// kernels, all deterministic (no arrival-order dependence):
//   1. hist:  one wave per chunk walks it 64 slots at a time; lanes holding
//             the same expert find each other with a ballot per id bit
//             (match mask), the lowest such lane adds the group size to an
//             LDS histogram.  The chunk histogram goes to the workspace,
//             expert-major ([E][nchunk]).
//   2. scan:  one wave per expert scans that expert's chunk counts
//             (contiguous) with shuffles, so chunk c learns how many earlier
//             slots share the expert; the total becomes counts[e].
//   3. rank:  each chunk's wave scans the local experts' counts into the
//             offsets (chunk 0 writes `offsets`), adds its per-expert chunk
//             base, then repeats the walk of 1: a slot's row is the running
//             base of its expert plus the number of lower lanes holding the
//             same expert, which keeps rows of an expert in ascending slot
//             order.  Also fills src_of's padding rows with -1.
//
// A batch of at most kFusedMaxSlots slots (decode sizes), in either layout,
// takes one launch instead: a single 1024-thread workgroup counts every expert (match masks
// and LDS atomics, order-independent), scans the local counts into the
// offsets, then ranks the slots 1024 at a time -- a slot's row is its
// expert's running base plus the same-expert slots of the lower waves of
// its chunk plus the lower lanes of its own wave -- which gives the same
// stable rows as the three kernels without their launch gaps.
//
// The fixed-capacity ("masked") variant (SGLang "Expert Parallelism", the
// MoE-runner table: masked layout for decode) runs the same three kernels;
// local expert j owns rows [j*cap_e, (j+1)*cap_e), so the ranking needs no
// offsets: a slot's row is j*cap_e + its rank within the expert, slots with
// rank >= cap_e are dropped, and the scan also writes m[j] = min(count, cap_e).
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

// Library-held workspace of the layout kernels for callers that cannot
// allocate (moe_layout_noalloc): the chunk histograms of one call.  One copy
// per GPU, alive until the process ends.  Host code never passes this name to
// a kernel (on the host it is only a stand-in for the symbol): it uses the
// device address hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) unsigned char scratch[moeep::kLayoutScratchBytes];

namespace moeep {
namespace {

constexpr int kChunk = 256;         // slots per chunk (4 wave steps)

struct LayoutWs {
    int32_t* base;    // [E][nchunk]: chunk histogram, then each chunk's first rank per expert
};

__host__ __device__ inline int n_chunks(long long slots) {
    return (int)((slots + kChunk - 1) / kChunk);
}

inline LayoutWs carve(void* ws, int nchunk, int E) {
    LayoutWs w;
    w.base = static_cast<int32_t*>(ws);
    return w;
}

__device__ __forceinline__ int id_bits(int E) { return E <= 1 ? 1 : 32 - __clz(E - 1); }

__global__ __launch_bounds__(kWave) void layout_hist_kernel(const int32_t* __restrict__ ids,
                                                            int n_slots, int E,
                                                            int32_t* __restrict__ base) {
    extern __shared__ int32_t s_hist[];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) s_hist[e] = 0;
    __syncthreads();
    const int nbits = id_bits(E);
    const int s0 = blockIdx.x * kChunk;
    for (int step = 0; step < kChunk; step += kWave) {
        const int s = s0 + step + lane;
        int e = (s < n_slots) ? ids[s] : -1;
        const bool valid = e >= 0 && e < E;
        const uint64_t active = ballot64(valid);
        if (active != 0) {                           // wave-uniform
            const uint64_t m = match_mask((uint32_t)(valid ? e : 0), active, nbits);
            if (valid && (m & lanemask_lt()) == 0) s_hist[e] += popc64(m);
        }
        __syncthreads();
    }
    __syncthreads();
    for (int e = lane; e < E; e += kWave) base[(size_t)e * gridDim.x + blockIdx.x] = s_hist[e];
}

// One wave per expert: exclusive scan of the expert's chunk counts in place
// (the chunk's first rank among the expert's slots); the total is counts[e].
__global__ __launch_bounds__(kWave) void layout_scan_kernel(int nchunk, int32_t* __restrict__ base,
                                                            int32_t* __restrict__ counts, int e_begin,
                                                            int e_end, int32_t* __restrict__ m,
                                                            int cap_e) {
    const int lane = threadIdx.x, e = blockIdx.x;
    int32_t* row = base + (size_t)e * nchunk;
    int carry = 0;
    for (int c0 = 0; c0 < nchunk; c0 += kWave) {
        const int c = c0 + lane;
        const int v = c < nchunk ? row[c] : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(x, d, kWave);
            if (lane >= d) x += y;
        }
        if (c < nchunk) row[c] = carry + x - v;
        carry += __shfl(x, kWave - 1, kWave);
    }
    if (lane == 0) {
        counts[e] = carry;
        if (m != nullptr && e >= e_begin && e < e_end) m[e - e_begin] = carry < cap_e ? carry : cap_e;
    }
}

// MASKED: cap is cap_e (rows per expert block) and offsets is unused.  Blocks
// past the nchunk chunks only pad src_of.
template <bool MASKED>
__global__ __launch_bounds__(kWave) void layout_rank_kernel(
    const int32_t* __restrict__ ids, int n_slots, int nchunk, int E, int e_begin, int e_end, int cap,
    const int32_t* __restrict__ base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_of, int32_t* __restrict__ src_of) {
    extern __shared__ int32_t s_next[];
    const int lane = threadIdx.x;
    const int E_loc = e_end - e_begin;
    const int s0 = blockIdx.x * kChunk;
    const int steps = s0 < n_slots ? kChunk : 0;     // an empty input still pads src_of
    // MASKED: next rank per local expert = this chunk's base
    // else:   local offsets (exclusive scan of counts[e_begin, e_end)) + the chunk's base
    int carry = 0;
    if (MASKED) {
        for (int j = lane; j < E_loc; j += kWave)
            s_next[j] = steps > 0 ? base[(size_t)(e_begin + j) * nchunk + blockIdx.x] : 0;
    }
    for (int j0 = 0; !MASKED && j0 < E_loc; j0 += kWave) {
        const int j = j0 + lane;
        const int v = j < E_loc ? counts[e_begin + j] : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(x, d, kWave);
            if (lane >= d) x += y;
        }
        if (j < E_loc) {
            const int off = carry + x - v;
            if (blockIdx.x == 0) offsets[j] = off;
            s_next[j] = off + (steps > 0 ? base[(size_t)(e_begin + j) * nchunk + blockIdx.x] : 0);
        }
        carry += __shfl(x, kWave - 1, kWave);
    }
    const int R = carry;                             // local rows (contiguous layout)
    if (!MASKED && blockIdx.x == 0 && lane == 0) offsets[E_loc] = R;
    __syncthreads();
    const int nbits = id_bits(E);
    for (int step = 0; step < steps; step += kWave) {
        const int s = s0 + step + lane;
        const bool in = s < n_slots;
        const int e = in ? ids[s] : -1;
        const bool local = e >= e_begin && e < e_end;
        const uint64_t active = ballot64(local);
        int row = -1;
        if (active != 0) {                            // wave-uniform
            const uint64_t m = match_mask((uint32_t)(local ? e - e_begin : 0), active, nbits);
            if (local) {
                const int rank = popc64(m & lanemask_lt());
                const int r = s_next[e - e_begin] + rank;
                if (MASKED)
                    row = r < cap ? (e - e_begin) * cap + r : -1;
                else
                    row = r < cap ? r : -1;
                if (row >= 0) src_of[row] = s;
                if (rank == 0) s_next[e - e_begin] = r + popc64(m);
            }
        }
        if (in) row_of[s] = row;
        __syncthreads();
    }
    // padding rows of src_of
    if (MASKED) {
        for (int r = blockIdx.x * kWave + lane; r < E_loc * cap; r += gridDim.x * kWave) {
            const int j = r / cap, q = r - j * cap;
            const int n = counts[e_begin + j];
            if (q >= n) src_of[r] = -1;
        }
    } else {
        for (int r = R + blockIdx.x * kWave + lane; r < cap; r += gridDim.x * kWave) src_of[r] = -1;
    }
}

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedMaxSlots = 4096;
constexpr int kFusedMaxE = 1024;

// MASKED: cap is cap_e (rows per expert block), `offsets` receives m (valid
// rows per local expert) and local expert j's rows start at j * cap_e.
template <bool MASKED>
__global__ __launch_bounds__(kFusedThreads) void layout_fused_kernel(
    const int32_t* __restrict__ ids, int n_slots, int E, int e_begin, int e_end, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_of) {
    __shared__ int s_cnt[kFusedMaxE];                  // all experts
    __shared__ int s_next[kFusedMaxE];                 // local experts: next free row
    __shared__ int s_wc[kFusedWaves * kFusedMaxE];     // [wave][local expert] slots in this chunk
    __shared__ int s_tmp[kFusedWaves];
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int E_loc = e_end - e_begin;
    const int nbits = id_bits(E);

    for (int e = tid; e < E; e += kFusedThreads) s_cnt[e] = 0;
    __syncthreads();
    // counts over all experts
    for (int s0 = 0; s0 < n_slots; s0 += kFusedThreads) {
        const int s = s0 + tid;
        const int e = s < n_slots ? ids[s] : -1;
        const bool valid = e >= 0 && e < E;
        const uint64_t active = ballot64(valid);
        if (active != 0) {                             // wave-uniform
            const uint64_t m = match_mask((uint32_t)(valid ? e : 0), active, nbits);
            if (valid && (m & lanemask_lt()) == 0) atomicAdd(&s_cnt[e], popc64(m));
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kFusedThreads) counts[e] = s_cnt[e];
    // contiguous: offsets = exclusive scan of the local counts, one expert per thread;
    // masked: m = counts clamped to the block, ranks start at 0 in every block
    const int v = tid < E_loc ? s_cnt[e_begin + tid] : 0;
    int x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) s_tmp[wv] = x;
    __syncthreads();
    int wsum = 0, R = 0;
#pragma unroll
    for (int w = 0; w < kFusedWaves; ++w) {
        wsum += w < wv ? s_tmp[w] : 0;
        R += s_tmp[w];
    }
    if (tid < E_loc) {
        const int off = wsum + x - v;
        offsets[tid] = MASKED ? (v < cap ? v : cap) : off;
        s_next[tid] = MASKED ? 0 : off;
    }
    if (!MASKED && tid == 0) offsets[E_loc] = R;
    // stable ranks, one chunk of kFusedThreads slots at a time
    for (int s0 = 0; s0 < n_slots; s0 += kFusedThreads) {
        for (int i = tid; i < kFusedWaves * E_loc; i += kFusedThreads) s_wc[i] = 0;
        __syncthreads();
        const int s = s0 + tid;
        const int e = s < n_slots ? ids[s] : -1;
        const bool local = e >= e_begin && e < e_end;
        const uint64_t active = ballot64(local);
        uint64_t m = 0;
        if (active != 0) {                             // wave-uniform
            m = match_mask((uint32_t)(local ? e - e_begin : 0), active, nbits);
            if (local && (m & lanemask_lt()) == 0) s_wc[wv * E_loc + (e - e_begin)] = popc64(m);
        }
        __syncthreads();
        int row = -1;
        if (local) {
            const int j = e - e_begin;
            int r = s_next[j] + popc64(m & lanemask_lt());
            for (int w = 0; w < wv; ++w) r += s_wc[w * E_loc + j];
            if (MASKED)
                row = r < cap ? j * cap + r : -1;
            else
                row = r < cap ? r : -1;
            if (row >= 0) src_of[row] = s;
        }
        if (s < n_slots) row_of[s] = row;
        __syncthreads();
        for (int j = tid; j < E_loc; j += kFusedThreads) {
            int add = 0;
#pragma unroll
            for (int w = 0; w < kFusedWaves; ++w) add += s_wc[w * E_loc + j];
            s_next[j] += add;
        }
        __syncthreads();                               // s_wc is read above before the next chunk clears it
    }
    // padding rows of src_of
    if (MASKED) {
        for (int r = tid; r < E_loc * cap; r += kFusedThreads) {
            const int j = r / cap, q = r - j * cap;
            if (q >= s_cnt[e_begin + j]) src_of[r] = -1;
        }
    } else {
        for (int r = R + tid; r < cap; r += kFusedThreads) src_of[r] = -1;
    }
}

}  // namespace

hipError_t layout_scratch_ptr(void** out) {
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

size_t layout_workspace_bytes(int B, int K, int E) {
    const int nchunk = n_chunks((long long)B * K);
    size_t bytes = ((size_t)nchunk * E + 1) * sizeof(int32_t);      // never empty
    return (bytes + 255) / 256 * 256;
}

hipError_t launch_layout(const int32_t* ids, int B, int K, int E, int e_begin, int e_end,
                         int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                         int cap, void* ws, hipStream_t stream) {
    const int n_slots = B * K;
    if (n_slots <= kFusedMaxSlots && E <= kFusedMaxE) {
        hipLaunchKernelGGL(layout_fused_kernel<false>, dim3(1), dim3(kFusedThreads), 0, stream, ids, n_slots,
                           E, e_begin, e_end, cap, counts, offsets, row_of, src_of);
        return hipGetLastError();
    }
    const int nchunk = n_chunks(n_slots);
    LayoutWs w = carve(ws, nchunk, E);
    if (nchunk > 0) {
        hipLaunchKernelGGL(layout_hist_kernel, dim3(nchunk), dim3(kWave), E * sizeof(int32_t),
                           stream, ids, n_slots, E, w.base);
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(E), dim3(kWave), 0, stream, nchunk, w.base, counts,
                       e_begin, e_end, (int32_t*)nullptr, 0);
    hipLaunchKernelGGL(layout_rank_kernel<false>, dim3(nchunk > 0 ? nchunk : 1), dim3(kWave),
                       (e_end - e_begin) * sizeof(int32_t), stream, ids, n_slots, nchunk, E,
                       e_begin, e_end, cap, w.base, counts, offsets, row_of, src_of);
    return hipGetLastError();
}

hipError_t launch_layout_masked(const int32_t* ids, int B, int K, int E, int e_begin, int e_end,
                                int32_t* counts, int32_t* m, int32_t* row_of, int32_t* src_of,
                                int cap_e, void* ws, hipStream_t stream) {
    const int n_slots = B * K;
    if (n_slots <= kFusedMaxSlots && E <= kFusedMaxE) {
        hipLaunchKernelGGL(layout_fused_kernel<true>, dim3(1), dim3(kFusedThreads), 0, stream, ids, n_slots,
                           E, e_begin, e_end, cap_e, counts, m, row_of, src_of);
        return hipGetLastError();
    }
    const int nchunk = n_chunks(n_slots);
    LayoutWs w = carve(ws, nchunk, E);
    if (nchunk > 0) {
        hipLaunchKernelGGL(layout_hist_kernel, dim3(nchunk), dim3(kWave), E * sizeof(int32_t),
                           stream, ids, n_slots, E, w.base);
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(E), dim3(kWave), 0, stream, nchunk, w.base, counts,
                       e_begin, e_end, m, cap_e);
    // enough blocks that the padding pass over E_local * cap_e rows is short
    const long long rows = (long long)(e_end - e_begin) * cap_e;
    const int pad_blocks = (int)((rows + 16 * kWave - 1) / (16 * kWave));
    const int grid = nchunk > pad_blocks ? nchunk : (pad_blocks > 0 ? pad_blocks : 1);
    hipLaunchKernelGGL(layout_rank_kernel<true>, dim3(grid), dim3(kWave),
                       (e_end - e_begin) * sizeof(int32_t), stream, ids, n_slots, nchunk, E,
                       e_begin, e_end, cap_e, w.base, counts, (int32_t*)nullptr, row_of, src_of);
    return hipGetLastError();
}

}  // namespace moeep
