// Wide bf16 grouped GEMM tile for prefill-sized row counts (SwiGLU gate/up
// or plain down projection), used by ffn_bf16.hip.
//
// A tile is up to BM rows of one expert (an expert with more rows is split
// evenly over several tiles) by 256 weight rows (gate/up: 128 gate + 128 up
// rows of the same output columns, so the SwiGLU epilogue has g and u of a
// column in one wave).  With BM = 320 every expert of a DeepSeek-shaped
// prefill batch (256 rows on average, a few past 300) fits one m-tile, so
// each weight tile is streamed from HBM once and feeds all of its rows.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4:
// each lane's 16 bytes land at the wave's LDS base + 16 * lane) through two
// k-step buffers.  Each buffer is its own __shared__ object and the k loop is
// unrolled by two so every LDS access names its buffer statically: the
// compiler can then see that reads of one stage do not alias the loads in
// flight into the other and does not drain the loads before every LDS read.
// The 16-byte chunks of a row are XOR-swizzled by (row & 7) so the 16 rows
// one MFMA operand read touches fall into distinct LDS banks; the direct
// loads permute which global chunk each lane fetches to produce that layout.
//
// Measured limits on MI355X that shaped this: the kernel is bound by its load
// pipeline, not by MFMA or LDS bandwidth; deeper direct-load rings (32-wide
// k-steps in 4 or 5 stages, or a separate weight ring loaded by dedicated
// waves) did not help, and a wave with a dozen or more strided direct loads
// outstanding slows down sharply.
#pragma once

#include <type_traits>

#include "grouped_tiles.hpp"

namespace moeep {
namespace wide {

constexpr int BN = 256;
constexpr int BK = 64;              // bf16 per k-step: 128 bytes per row
constexpr int CPR = 8;              // 16-byte chunks per row
constexpr int ROWB = 128;           // bytes per LDS row

template <int N>
using ic = std::integral_constant<int, N>;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt at
// their maxima so they do not wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}
// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every load in flight (the direct-to-LDS loads count as
// LDS stores), which would drain the next stage's loads at every k-step.  The
// memory clobber keeps the compiler from moving memory accesses across it;
// the explicit s_waitcnt calls around it order the LDS traffic.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS at
// lds_wave_base + 16 * lane.  The builtin only exists in the device pass; the
// host pass of a kernel template that names it directly drops the kernel's
// launch stub, hence the wrapper.  CPOL is the cache-policy operand: 0 for
// plain loads, kNonTemporal for data a tile reads once.
constexpr int kNonTemporal = 2;

template <int CPOL>
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, CPOL);
#endif
}

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

// 8 waves laid out 2 (rows) x 4 (weight rows).  A wave owns the interleaved
// 16-row fragments {wm, wm + 2, ...} (so a short tile still spreads its valid
// rows over both row-waves) and 64 weight rows.
template <int BM, bool GATED>
__global__ __launch_bounds__(512, 1) void grouped_gemm_bf16_wide_kernel(FfnArgs p) {
    constexpr int WMW = 2, WNW = 4, NT = 512, NW = 8;
    constexpr int A_BLOCKS = BM * CPR / 64;          // 1 KiB blocks of a row stage
    constexpr int BLOCKS = (BM + BN) * CPR / 64;
    constexpr int LPS = BLOCKS / NW;                 // direct loads per wave per stage
    constexpr int FM = BM / 16 / WMW;                // 16-row fragments per wave
    constexpr int WN = BN / WNW;                     // 64 weight rows per wave
    constexpr int FN = WN / 16;                      // 4
    constexpr int BNO = GATED ? BN / 2 : BN;         // output columns per tile
    static_assert(BM % 32 == 0 && BLOCKS % NW == 0 && (!GATED || FN % 2 == 0), "tile shape");
    // block q = i * NW + wave: whether it is a row block and which weight half it
    // covers depends only on i, so both are compile-time after unrolling
    static_assert(A_BLOCKS % NW == 0 && (BN / 16) % NW == 0, "block split");
    constexpr int A_ITERS = A_BLOCKS / NW;           // i < A_ITERS: row blocks
    constexpr int G_ITERS = (BN / 16) / NW;          // next G_ITERS: gate (or first) weight half

    __shared__ uint4 sa0[BM * CPR];
    __shared__ uint4 sb0[BN * CPR];
    __shared__ uint4 sa1[BM * CPR];
    __shared__ uint4 sb1[BN * CPR];
    __shared__ int s_pre[kMaxExperts + 1];
    __shared__ uint16_t s_ord[kMaxExperts];          // experts, most rows first
    static_assert(sizeof(sa0) >= kMaxExperts * sizeof(int), "row counts fit in the first row stage");
    __shared__ int s_tmp[NT / kWave];

    auto a_base = [&](auto I) -> char* {
        if constexpr (decltype(I)::value == 0) return reinterpret_cast<char*>(sa0);
        else return reinterpret_cast<char*>(sa1);
    };
    auto b_base = [&](auto I) -> char* {
        if constexpr (decltype(I)::value == 0) return reinterpret_cast<char*>(sb0);
        else return reinterpret_cast<char*>(sb1);
    };

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: keeps LDS bases scalar
    const int wm = wave / WNW, wn = wave % WNW;
    const int Kdim = p.Kdim, N = p.N, cap = p.cap;
    const int nk = Kdim / BK;

    // largest experts' tiles first; the first row stage is free scratch until the first load
    build_tile_prefix_sorted<NT, BM>(p, s_pre, s_ord, reinterpret_cast<int*>(sa0), s_tmp);
    const int n_tiles_n = (N + BNO - 1) / BNO;
    const int total = n_tiles_n * s_pre[p.E_loc];
    const int G = gridDim.x;
    const int v = xcd_block_order();

    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(p.a);
    const uint16_t* __restrict__ W0 = static_cast<const uint16_t*>(p.w0);
    const uint16_t* __restrict__ W1 = static_cast<const uint16_t*>(p.w1);
    uint16_t* __restrict__ Out = static_cast<uint16_t*>(p.out);

    for (int tau = v; tau < total; tau += G) {
        const TileCoord tc = decode_tile<BM>(tau, n_tiles_n, s_pre, p, s_ord);
        const int j = tc.j, row0 = tc.row0, nvalid = tc.nvalid;
        const int col0 = tc.nt * BNO;
        const uint16_t* wg = W0 + (size_t)j * N * Kdim;
        const uint16_t* wu = GATED ? W1 + (size_t)j * N * Kdim : nullptr;

        // per-lane source offsets of this wave's direct loads (fixed for the tile),
        // 32-bit, relative to the row tensor or to the expert's weight matrices;
        // lanes past the valid rows / columns re-read row 0 so every stage is
        // exactly LPS vector-memory instructions per wave
        const char* abase = reinterpret_cast<const char*>(A + (size_t)row0 * Kdim);
        const char* gbase = reinterpret_cast<const char*>(wg);
        const char* ubase = reinterpret_cast<const char*>(wu);
        uint32_t off[LPS];
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const bool is_a = i < A_ITERS;
            const int r = (is_a ? i * NW : (i - A_ITERS) * NW) * 8 + wave * 8 + lane / 8;
            const uint32_t c16 = (uint32_t)swz(r, lane % 8) * 16;   // logical chunk this lane fetches
            if (is_a) {
                off[i] = (uint32_t)(r < nvalid ? r : 0) * (uint32_t)(Kdim * 2) + c16;
            } else {
                const int rr = (GATED && r >= BN / 2) ? r - BN / 2 : r;
                const int col = col0 + rr;
                off[i] = (uint32_t)(col < N ? col : 0) * (uint32_t)(Kdim * 2) + c16;
            }
        }
        auto issue = [&](auto I, int kstep) {
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const bool is_a = i < A_ITERS;
                const bool up = GATED && i >= A_ITERS + G_ITERS;
                const char* b = is_a ? abase : (up ? ubase : gbase);
                char* dst = is_a ? a_base(I) + (i * NW + wave) * 1024
                                 : b_base(I) + ((i - A_ITERS) * NW + wave) * 1024;
                // weight tiles are read by one or two m-tiles of an expert, all
                // close together in tile order; the row block is re-read by
                // every n-tile, so only the weights stream.  Row blocks wholly
                // past the valid rows are not loaded (wave-uniform): their
                // stale LDS rows feed only outputs that are never stored.
                if (is_a) {
                    if ((i * NW + wave) * 8 < nvalid) lds_dma16<0>(b + off[i] + (size_t)kstep * BK * 2, dst);
                } else
                    lds_dma16<kNonTemporal>(b + off[i] + (size_t)kstep * BK * 2, dst);
            }
        };

        floatx4 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

        auto brow = [&](int f) {      // B-tile row of this lane for n-fragment f
            if (GATED) {
                const int half = f < FN / 2 ? 0 : BN / 2;
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return half + wn * (WN / 2) + ff * 16 + (lane & 15);
            }
            return wn * WN + f * 16 + (lane & 15);
        };
        auto fcol = [&](int f) {      // output column of fragment f's first lane column
            if (GATED) {
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return col0 + wn * (WN / 2) + ff * 16;
            }
            return col0 + wn * WN + f * 16;
        };

        // v_mfma_f32_16x16x32_bf16: lane l feeds row (l % 16) with k-chunk (l / 16)
        // of the 32-wide step for both operands and receives rows 4*(l/16)+e,
        // column l % 16 of the 16x16 result
        auto compute = [&](auto I) {
            const char* ab = a_base(I);
            const char* bb = b_base(I);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c = kk * 4 + (lane >> 4);
                bf16x8 bfr[FN];
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    const int r = brow(f);
                    bfr[f] = *reinterpret_cast<const bf16x8*>(bb + r * ROWB + swz(r, c) * 16);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int mrow = (wm + WMW * i) * 16;
                    if (mrow < nvalid) {
                        const int r = mrow + (lane & 15);
                        const bf16x8 afr = *reinterpret_cast<const bf16x8*>(ab + r * ROWB + swz(r, c) * 16);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[f], acc[i][f], 0, 0, 0);
                    }
                }
            }
        };

        // the previous tile's reads of both stages must be complete before new loads land
        wait_lgkm0();
        block_barrier();
        issue(ic<0>{}, 0);

        // step k: wait for stage k (nothing else is in flight), then load k+1
        // into the other buffer while computing k
        auto step = [&](auto I, int k) {
            constexpr int s = decltype(I)::value;
            wait_vmcnt<0>();
            wait_lgkm0();
            block_barrier();
            if (k + 1 < nk) issue(ic<1 - s>{}, k + 1);
            compute(I);
        };
        for (int k = 0; k < nk; k += 2) {
            step(ic<0>{}, k);
            if (k + 1 < nk) step(ic<1>{}, k + 1);
        }

        // ---- epilogue
        constexpr int FO = GATED ? FN / 2 : FN;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int mrow = (wm + WMW * i) * 16;
            if (mrow >= nvalid) continue;
#pragma unroll
            for (int f = 0; f < FO; ++f) {
                const int col = fcol(f) + (lane & 15);
                if (col >= N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = mrow + (lane >> 4) * 4 + e;
                    if (r < nvalid) {
                        const float val = GATED ? silu(acc[i][f][e]) * acc[i][f + FN / 2][e] : acc[i][f][e];
                        Out[(size_t)(row0 + r) * N + col] = (uint16_t)f32_to_bf16_bits(val);
                    }
                }
            }
        }
    }
}

}  // namespace wide
}  // namespace moeep
