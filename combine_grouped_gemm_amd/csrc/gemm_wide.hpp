// Wide bf16 grouped GEMM tile for prefill-sized row counts (SwiGLU gate/up
// or plain down projection), used by ffn_bf16.hip.
//
// A tile is 256 rows of one expert (an expert with more rows is split evenly
// over several tiles) by 256 weight rows (gate/up: 128 gate + 128 up rows of
// the same output columns, so the SwiGLU epilogue has g and u of a column in
// one wave).  Almost every expert of a prefill batch fits one m-tile, so each
// weight tile is streamed from HBM once and reused for all of its rows.
//
// Operands go from global memory straight into LDS (global_load_lds_dwordx4:
// each lane's 16 bytes land at the wave's LDS base + 16 * lane), through a
// ring of STAGES k-step buffers.  Each buffer is its own __shared__ object
// and the ring is unrolled so every LDS access names its buffer statically:
// the compiler can then see that reads of stage s do not alias the loads in
// flight into the other stages and only waits for stage s (vmcnt counting).
// The 16-byte chunks of a row are XOR-swizzled so that the 16 rows one MFMA
// operand read touches fall into distinct LDS banks; the direct loads permute
// which global chunk each lane fetches to produce that layout.
#pragma once

#include <type_traits>

#include "grouped_tiles.hpp"

namespace moeep {
namespace wide {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int kObjUint4 = 2048;     // 32 KiB per LDS object

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
// LDS stores), which would drain the load ring at every k-step.  The memory
// clobber keeps the compiler from moving memory accesses across it; the
// explicit s_waitcnt calls around it order the LDS traffic.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS at
// lds_wave_base + 16 * lane.  The builtin only exists in the device pass; the
// host pass of a kernel template that names it directly drops the kernel's
// launch stub, hence the wrapper.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
#endif
}

template <int BK, int WMW, int WNW, bool GATED, int S_ = (BK == 32 ? 4 : 2)>
struct Cfg {
    static constexpr int NT = 64 * WMW * WNW;
    static constexpr int NW = WMW * WNW;
    static constexpr int CPR = BK / 8;                    // 16-byte chunks per row
    static constexpr int STAGES = S_;                     // BK 32: one 32 KiB object per stage; BK 64: two
    static constexpr int A_BLOCKS = BM * CPR / 64;         // 1 KiB blocks per stage for A
    static constexpr int BLOCKS = (BM + BN) * CPR / 64;
    static constexpr int LPS = BLOCKS / NW;                // direct loads per wave per stage
    static constexpr int FM = BM / 16 / WMW;               // 16-row fragments per wave
    static constexpr int WN = BN / WNW;                    // B rows per wave
    static constexpr int FN = WN / 16;
    static constexpr int BNO = GATED ? BN / 2 : BN;        // output columns per tile
    static_assert(BLOCKS % NW == 0 && FN >= 1 && (!GATED || FN % 2 == 0), "tile shape");
    static_assert(BK == 32 || BK == 64, "k-step");
    static_assert((BK == 32 && STAGES == 4) || (BK == 64 && STAGES == 2), "ring");
};

__device__ __forceinline__ int swz(int row, int c, int cpr) {
    return cpr == 8 ? (c ^ (row & 7)) : (c ^ ((row >> 1) & 3));
}

template <int BK, int WMW, int WNW, bool GATED, int STAGES>
__global__ __launch_bounds__(64 * WMW * WNW, 1) void grouped_gemm_bf16_wide_kernel(FfnArgs p) {
    using C = Cfg<BK, WMW, WNW, GATED, STAGES>;
    constexpr int NT = C::NT, CPR = C::CPR, S = C::STAGES, LPS = C::LPS, FM = C::FM, FN = C::FN;
    constexpr int ROWB = CPR * 16;                         // bytes per LDS row

    __shared__ uint4 o0[kObjUint4];
    __shared__ uint4 o1[kObjUint4];
    __shared__ uint4 o2[kObjUint4];
    __shared__ uint4 o3[kObjUint4];
    __shared__ int s_pre[kMaxExperts + 1];
    __shared__ int s_tmp[NT / kWave];

    // stage s: A region and B region (byte pointers)
    auto a_base = [&](auto I) -> char* {
        constexpr int s = decltype(I)::value;
        if constexpr (BK == 32) {
            if constexpr (s == 0) return reinterpret_cast<char*>(o0);
            else if constexpr (s == 1) return reinterpret_cast<char*>(o1);
            else if constexpr (s == 2) return reinterpret_cast<char*>(o2);
            else return reinterpret_cast<char*>(o3);
        } else {
            if constexpr (s == 0) return reinterpret_cast<char*>(o0);
            else return reinterpret_cast<char*>(o2);
        }
    };
    auto b_base = [&](auto I) -> char* {
        constexpr int s = decltype(I)::value;
        if constexpr (BK == 32) {
            return a_base(I) + BM * ROWB;
        } else {
            if constexpr (s == 0) return reinterpret_cast<char*>(o1);
            else return reinterpret_cast<char*>(o3);
        }
    };

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WNW, wn = wave % WNW;
    const int Kdim = p.Kdim, N = p.N, cap = p.cap;
    const int nk = Kdim / BK;

    build_tile_prefix<NT, BM>(p.offsets, p.E_loc, cap, s_pre, s_tmp);
    const int n_tiles_n = (N + C::BNO - 1) / C::BNO;
    const int total = n_tiles_n * s_pre[p.E_loc];
    const int G = gridDim.x;
    const int v = xcd_block_order();

    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(p.a);
    const uint16_t* __restrict__ W0 = static_cast<const uint16_t*>(p.w0);
    const uint16_t* __restrict__ W1 = static_cast<const uint16_t*>(p.w1);
    uint16_t* __restrict__ Out = static_cast<uint16_t*>(p.out);

    for (int tau = v; tau < total; tau += G) {
        const TileCoord tc = decode_tile<BM>(tau, n_tiles_n, s_pre, p.E_loc, p.offsets, cap);
        const int j = tc.j, row0 = tc.row0, nvalid = tc.nvalid;
        const int col0 = tc.nt * C::BNO;
        const uint16_t* wg = W0 + (size_t)j * N * Kdim;
        const uint16_t* wu = GATED ? W1 + (size_t)j * N * Kdim : nullptr;

        // per-lane source rows of this wave's direct loads (fixed for the tile)
        const char* src[LPS];
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int q = i * C::NW + wave;                  // 1 KiB block of the stage
            const bool is_a = q < C::A_BLOCKS;
            const int qq = is_a ? q : q - C::A_BLOCKS;
            const int r = qq * (64 / CPR) + lane / CPR;     // row inside the A or B region
            const int c = swz(r, lane % CPR, CPR);           // logical chunk this lane fetches
            if (is_a) {
                src[i] = reinterpret_cast<const char*>(A + (size_t)(row0 + (r < nvalid ? r : 0)) * Kdim) + c * 16;
            } else {
                int col;
                const uint16_t* w;
                if (GATED) {
                    const bool up = r >= BN / 2;
                    col = col0 + (up ? r - BN / 2 : r);
                    w = up ? wu : wg;
                } else {
                    col = col0 + r;
                    w = wg;
                }
                src[i] = reinterpret_cast<const char*>(w + (size_t)(col < N ? col : 0) * Kdim) + c * 16;
            }
        }
        auto issue = [&](auto I, int kstep) {
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const int q = i * C::NW + wave;
                const bool is_a = q < C::A_BLOCKS;
                char* dst = is_a ? a_base(I) + q * 1024 : b_base(I) + (q - C::A_BLOCKS) * 1024;
                // issued by every lane, valid or not (invalid lanes re-read a valid row), so
                // that each stage is exactly LPS vector-memory instructions per wave, which
                // the vmcnt waits count on
                lds_dma16(src[i] + (size_t)kstep * BK * 2, dst);
            }
        };

        floatx4 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

        auto brow = [&](int f) {
            if (GATED) {
                const int half = f < FN / 2 ? 0 : BN / 2;
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return half + wn * (C::WN / 2) + ff * 16 + (lane & 15);
            }
            return wn * C::WN + f * 16 + (lane & 15);
        };
        auto fcol = [&](int f) {
            if (GATED) {
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return col0 + wn * (C::WN / 2) + ff * 16;
            }
            return col0 + wn * C::WN + f * 16;
        };

        auto compute = [&](auto I) {
            const char* ab = a_base(I);
            const char* bb = b_base(I);
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
                const int c = kk * 4 + (lane >> 4);
                bf16x8 bfr[FN];
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    const int r = brow(f);
                    bfr[f] = *reinterpret_cast<const bf16x8*>(bb + r * ROWB + swz(r, c, CPR) * 16);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int mrow = (wm + WMW * i) * 16;
                    if (mrow < nvalid) {
                        const int r = mrow + (lane & 15);
                        const bf16x8 afr = *reinterpret_cast<const bf16x8*>(ab + r * ROWB + swz(r, c, CPR) * 16);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[f], acc[i][f], 0, 0, 0);
                    }
                }
            }
        };

        // the previous tile's reads of every stage must be complete before new loads land
        wait_lgkm0();
        block_barrier();
        // prologue: stages 0 .. S-2
        issue(ic<0>{}, 0);
        if constexpr (S > 2) {
            if (1 < nk) issue(ic<1>{}, 1);
            if (2 < nk) issue(ic<2>{}, 2);
        }

        auto step = [&](auto I, int k) {
            constexpr int s = decltype(I)::value;
            // stages issued after k: min(k + S - 2, nk - 1) - k
            const int after = min(k + S - 2, nk - 1) - k;
            if constexpr (S == 4) {
                if (after >= 2) wait_vmcnt<2 * LPS>();
                else if (after == 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            } else {
                wait_vmcnt<0>();
            }
            wait_lgkm0();
            block_barrier();
            if (k + S - 1 < nk) issue(ic<(s + S - 1) % S>{}, k + S - 1);
            compute(I);
        };

        for (int k = 0; k < nk; k += S) {
            step(ic<0>{}, k);
            if (k + 1 < nk) step(ic<1>{}, k + 1);
            if constexpr (S >= 4) {
                if (k + 2 < nk) step(ic<2>{}, k + 2);
                if (k + 3 < nk) step(ic<3>{}, k + 3);
            }
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
