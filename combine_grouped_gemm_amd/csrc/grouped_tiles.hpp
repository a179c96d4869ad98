// Ragged tile scheduling shared by the grouped GEMM kernels.
//
// The per-expert row counts exist only on the device (offsets of the
// contiguous layout, or the valid-row counts of the masked layout), so a
// persistent grid derives its work list there: every block builds the
// prefix sum over local experts (in id order, or most rows first) of
// ceil(rows / BM) m-tiles in LDS and maps a linear tile index tau to
// (expert j, n-tile, m-tile) by binary search, with the m-tile index fastest
// so that tiles sharing one weight tile are consecutive.  An expert's rows
// are split evenly over its m-tiles.  Blocks are renumbered XCD-major
// (hardware dispatch places block b on XCD b % 8), so consecutive tile
// indices run on one XCD and share its L2.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace moeep {

constexpr int kMaxExperts = 1024;
constexpr int kXcd = 8;

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Rows [r0, r1) of local expert j: a range of the contiguous layout, or the
// first m_counts[j] rows of the expert's fixed block in the masked layout;
// both clamped to the buffer.
__device__ __forceinline__ void expert_rows(const FfnArgs& p, int j, int& r0, int& r1) {
    if (p.offsets != nullptr) {
        r0 = clampi(p.offsets[j], 0, p.cap);
        r1 = clampi(p.offsets[j + 1], r0, p.cap);
    } else {
        r0 = j * p.cap_e;
        r1 = r0 + clampi(p.m_counts[j], 0, p.cap_e);
    }
}

// Block-wide exclusive prefix into s_pre[0..n] of count(i), i in [0, n).
// s_tmp needs NT / 64 ints.  Ends with a barrier.
template <int NT, typename Count>
__device__ void scan_tile_counts(int n, Count count, int* s_pre, int* s_tmp) {
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    constexpr int NW = NT / kWave;
    int carry = 0;
    if (tid == 0) s_pre[0] = 0;
    for (int base = 0; base < n; base += NT) {
        const int j = base + tid;
        const int v = j < n ? count(j) : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            int y = __shfl_up(x, d, kWave);
            if (lane >= d) x += y;
        }
        if (lane == kWave - 1) s_tmp[wv] = x;
        __syncthreads();
        int wsum = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            wsum += (w < wv) ? s_tmp[w] : 0;
            total += s_tmp[w];
        }
        if (j < n) s_pre[j + 1] = carry + wsum + x;
        carry += total;
        __syncthreads();
    }
    __syncthreads();
}

// Block-wide exclusive prefix of m-tile counts per expert into s_pre[0..E_loc],
// experts in id order.  s_tmp needs NT / 64 ints.  Ends with a barrier.
template <int NT, int BM>
__device__ void build_tile_prefix(const FfnArgs& p, int* s_pre, int* s_tmp) {
    scan_tile_counts<NT>(p.E_loc, [&](int j) {
        int r0, r1;
        expert_rows(p, j, r0, r1);
        return (r1 - r0 + BM - 1) / BM;
    }, s_pre, s_tmp);
}

// The same prefix with the experts in decreasing row count (ties: lower id
// first): s_ord[pos] is the expert at position pos, s_pre the prefix in that
// order.  A persistent grid walks tiles in this order, so its last, partly
// filled round holds the smallest experts' tiles instead of whichever
// experts have the highest ids (longest tiles first).  s_rows is E_loc ints
// of scratch that is free at this point.  Ends with a barrier.
template <int NT, int BM>
__device__ void build_tile_prefix_sorted(const FfnArgs& p, int* s_pre, uint16_t* s_ord, int* s_rows,
                                         int* s_tmp) {
    const int E_loc = p.E_loc, tid = threadIdx.x;
    for (int j = tid; j < E_loc; j += NT) {
        int r0, r1;
        expert_rows(p, j, r0, r1);
        s_rows[j] = r1 - r0;
    }
    __syncthreads();
    for (int j = tid; j < E_loc; j += NT) {
        const int r = s_rows[j];
        int rank = 0;
        for (int i = 0; i < E_loc; ++i) {
            const int q = s_rows[i];
            rank += (q > r || (q == r && i < j)) ? 1 : 0;
        }
        s_ord[rank] = (uint16_t)j;
    }
    __syncthreads();
    scan_tile_counts<NT>(E_loc, [&](int pos) { return (s_rows[s_ord[pos]] + BM - 1) / BM; }, s_pre,
                         s_tmp);
}

struct TileCoord {
    int j;        // local expert
    int nt;       // n-tile
    int row0;     // first row of the tile
    int nvalid;   // valid rows in the tile (<= BM)
};

// s_ord: expert at each prefix position (build_tile_prefix_sorted), or nullptr
// for id order.
template <int BM>
__device__ __forceinline__ TileCoord decode_tile(int tau, int n_tiles_n, const int* s_pre,
                                                 const FfnArgs& p, const uint16_t* s_ord = nullptr) {
    int lo = 0, hi = p.E_loc;     // largest position j with n_tiles_n * s_pre[j] <= tau
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (n_tiles_n * s_pre[mid] <= tau) lo = mid; else hi = mid;
    }
    TileCoord t;
    t.j = s_ord != nullptr ? (int)s_ord[lo] : lo;
    const int mt_j = s_pre[lo + 1] - s_pre[lo];
    const int local = tau - n_tiles_n * s_pre[lo];
    t.nt = local / mt_j;
    const int mt = local % mt_j;
    int r0, r1;
    expert_rows(p, t.j, r0, r1);
    // balanced split: m-tile mt of mt_j takes rows [n*mt/mt_j, n*(mt+1)/mt_j) of the
    // expert, at most ceil(n/mt_j) <= BM of them
    const int n = r1 - r0;
    t.row0 = r0 + (int)(((long long)n * mt) / mt_j);
    t.nvalid = r0 + (int)(((long long)n * (mt + 1)) / mt_j) - t.row0;
    // every lane computed the same values: keep them in scalar registers, so
    // tile base addresses are scalar and stores can use 32-bit lane offsets
    t.j = __builtin_amdgcn_readfirstlane(t.j);
    t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
    t.nvalid = __builtin_amdgcn_readfirstlane(t.nvalid);
    return t;
}

// Tile of round r for the block with XCD-major position v and hardware
// index b in a grid of G, or -1 when it has none.  Rounds go in XCD-major
// order (tiles that run together are neighbours in memory and share L2),
// except a last round that fills less than half the grid: in XCD-major
// order it would run on the first few XCDs alone, so it goes in hardware
// order, spread over all of them.  (Measured on the decode-sized FFN with
// several blocks per CU: spreading a 45%-full last round 5% faster overall,
// a 78%-full one 2.7% slower.)
__device__ __forceinline__ int round_tile(int r, int v, int b, int G, int total) {
    const long long base = (long long)r * G;
    if (base >= total) return -1;
    const long long rem = total - base;
    const int tau = (int)base + (2 * rem >= G ? v : b);
    return tau < total ? tau : -1;
}

// XCD-major renumbering of the block index (identity when G % 8 != 0).
__device__ __forceinline__ int xcd_block_order() {
    const int G = gridDim.x, b = blockIdx.x;
    return (G % kXcd == 0) ? (b % kXcd) * (G / kXcd) + b / kXcd : b;
}

template <typename Kern>
hipError_t launch_persistent(Kern kern, int threads, const FfnArgs& a, hipStream_t stream,
                             int* per_cu_cache) {
    if (*per_cu_cache == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess || n < 1)
            n = 1;
        *per_cu_cache = n;
    }
    const int grid = device_cu_count() * *per_cu_cache;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moeep
