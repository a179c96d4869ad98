// Grouped SwiGLU expert FFN, bf16 operands, fp32 accumulation on MFMA.
//
// "Anatomy of a high-performance EP kernel", section "Dispatch": one grouped
// GEMM call multiplies a separate row set per expert, the row counts being
// whatever the routing produced; Moreh report, "Overview": each expert is a
// small FFN.  Two launches share one kernel template:
//   gate/up:  h = silu(Xd Wg^T) * (Xd Wu^T)      (GATED, bf16 h out)
//   down:     y = h Wd^T                          (bf16 y out)
//
// Work decomposition.  A tile is (local expert j, n-tile, m-tile).  The
// per-expert row counts live only on the device (offsets), so every block
// of a persistent grid first builds, in LDS, the prefix sum of m-tiles per
// expert and then walks tile indices tau = v, v + G, ... where v is the
// block's XCD-grouped position: blocks b and b + 8 run on the same XCD
// (dispatch is round-robin over the 8 XCDs), so consecutive tile indices --
// the m-tiles that share one weight tile, and the n-tiles that share one
// row block -- meet in the same L2.
//
// Inside a tile: K loop in steps of 64 bf16 (128 bytes per row).  Global
// 16-byte loads (non-temporal for the weights, which the m-tiles of one
// expert read close together in tile order) go to registers one step ahead, then to LDS with a XOR
// swizzle of the 16-byte chunk index by (row & 7), which spreads the 16
// rows that one MFMA operand read touches over distinct banks.  Waves are
// laid out WMW x WNW; a wave owns the 16-row fragments {wm, wm + WMW, ...}
// (interleaved, so a short last m-tile still spreads its valid rows over
// all waves) and skips fragments past the tile's valid rows.  MFMA is
// v_mfma_f32_16x16x32_bf16: lane l feeds row (l % 16) with k-chunk (l / 16)
// of the 32-wide step for both operands and receives rows 4*(l/16)+i,
// column l % 16 of the 16x16 result.
#include "gemm_wide.hpp"
#include "grouped_tiles.hpp"

namespace moeep {
namespace {

constexpr int BK = 64;            // bf16 per k-step

template <int BM, int BN, int WMW, int WNW, bool GATED>
__global__ __launch_bounds__(64 * WMW * WNW) void grouped_gemm_bf16_kernel(FfnArgs p) {
    constexpr int NT = 64 * WMW * WNW;
    constexpr int FM = BM / 16 / WMW;          // m-fragments per wave
    constexpr int WN = BN / WNW;               // B-tile rows per wave
    constexpr int FN = WN / 16;                // n-fragments per wave
    constexpr int BNO = GATED ? BN / 2 : BN;   // output columns per tile
    static_assert(FM >= 1 && FN >= 1 && (!GATED || FN % 2 == 0), "tile shape");
    constexpr int A_IT = (BM * 8 + NT - 1) / NT;
    constexpr int B_IT = (BN * 8 + NT - 1) / NT;

    __shared__ uint4 sA[BM * 8];
    __shared__ uint4 sB[BN * 8];
    __shared__ int s_pre[kMaxExperts + 1];
    __shared__ int s_tmp[NT / kWave];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WNW, wn = wave % WNW;
    const int Kdim = p.Kdim, N = p.N, cap = p.cap, ldw = p.ldw;

    build_tile_prefix<NT, BM>(p, s_pre, s_tmp);
    const int n_tiles_n = (N + BNO - 1) / BNO;
    const int total = n_tiles_n * s_pre[p.E_loc];

    const int G = gridDim.x;
    const int v = xcd_block_order();

    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(p.a);
    const uint16_t* __restrict__ W0 = static_cast<const uint16_t*>(p.w0);
    const uint16_t* __restrict__ W1 = static_cast<const uint16_t*>(p.w1);
    uint16_t* __restrict__ Out = static_cast<uint16_t*>(p.out);

    for (int rnd = 0;; ++rnd) {
        const int tau = round_tile(rnd, v, blockIdx.x, G, total);
        if (tau < 0) break;
        const TileCoord tc = decode_tile<BM>(tau, n_tiles_n, s_pre, p);
        const int j = tc.j, row0 = tc.row0, nvalid = tc.nvalid;
        const int col0 = tc.nt * BNO;

        const uint16_t* wg = W0 + (size_t)j * N * ldw;
        const uint16_t* wu = GATED ? W1 + (size_t)j * N * ldw : nullptr;

        // ---- global -> register staging
        uint4 ra[A_IT], rb[B_IT];
#pragma unroll
        for (int i = 0; i < A_IT; ++i) ra[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_IT; ++i) rb[i] = make_uint4(0, 0, 0, 0);
        auto load_step = [&](int k0) {
#pragma unroll
            for (int i = 0; i < A_IT; ++i) {
                const int q = tid + i * NT;
                const int r = q >> 3, c = q & 7;
                // chunks past K (a partial last step) are zero
                if (q < BM * 8 && r < nvalid)
                    ra[i] = k0 + c * 8 < Kdim
                                ? *reinterpret_cast<const uint4*>(A + (size_t)(row0 + r) * Kdim + k0 + c * 8)
                                : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < B_IT; ++i) {
                const int q = tid + i * NT;
                const int r = q >> 3, c = q & 7;
                if (q < BN * 8) {
                    const uint16_t* src;
                    int col;
                    if (GATED) {
                        const bool up = r >= BN / 2;
                        col = col0 + (up ? r - BN / 2 : r);
                        src = up ? wu : wg;
                    } else {
                        col = col0 + r;
                        src = wg;
                    }
                    if (col < N)
                        rb[i] = k0 + c * 8 < Kdim ? load_stream16(src + (size_t)col * ldw + k0 + c * 8)
                                                  : make_uint4(0, 0, 0, 0);
                }
            }
        };
        auto store_step = [&]() {
#pragma unroll
            for (int i = 0; i < A_IT; ++i) {
                const int q = tid + i * NT;
                const int r = q >> 3, c = q & 7;
                if (q < BM * 8 && r < nvalid) sA[r * 8 + (c ^ (r & 7))] = ra[i];
            }
#pragma unroll
            for (int i = 0; i < B_IT; ++i) {
                const int q = tid + i * NT;
                const int r = q >> 3, c = q & 7;
                if (q < BN * 8) sB[r * 8 + (c ^ (r & 7))] = rb[i];
            }
        };

        floatx4 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

        // B-tile row of this lane for n-fragment f
        auto brow = [&](int f) {
            if (GATED) {
                const int half = f < FN / 2 ? 0 : BN / 2;
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return half + wn * (WN / 2) + ff * 16 + (lane & 15);
            }
            return wn * WN + f * 16 + (lane & 15);
        };
        auto fcol = [&](int f) {    // output column of fragment f's first lane column
            if (GATED) {
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return col0 + wn * (WN / 2) + ff * 16;
            }
            return col0 + wn * WN + f * 16;
        };

        load_step(0);
        for (int k0 = 0; k0 < Kdim; k0 += BK) {
            __syncthreads();
            store_step();
            __syncthreads();
            if (k0 + BK < Kdim) load_step(k0 + BK);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int chunk = kk * 4 + (lane >> 4);
                bf16x8 bfr[FN];
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    const int r = brow(f);
                    uint4 t = sB[r * 8 + (chunk ^ (r & 7))];
                    bfr[f] = __builtin_bit_cast(bf16x8, t);
                }
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int mrow = (wm + WMW * i) * 16;
                    if (mrow < nvalid) {
                        const int r = mrow + (lane & 15);
                        uint4 t = sA[r * 8 + (chunk ^ (r & 7))];
                        const bf16x8 afr = __builtin_bit_cast(bf16x8, t);
#pragma unroll
                        for (int f = 0; f < FN; ++f) {
                            if (fcol(f) < N)
                                acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[f], acc[i][f], 0, 0, 0);
                        }
                    }
                }
            }
        }

        // ---- epilogue
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int mrow = (wm + WMW * i) * 16;
            if (mrow >= nvalid) continue;
            constexpr int FO = GATED ? FN / 2 : FN;
#pragma unroll
            for (int f = 0; f < FO; ++f) {
                const int col = fcol(f) + (lane & 15);
                if (col >= N) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = mrow + (lane >> 4) * 4 + e;
                    if (r < nvalid) {
                        float val = GATED ? silu(acc[i][f][e]) * acc[i][f + FN / 2][e] : acc[i][f][e];
                        Out[(size_t)(row0 + r) * N + col] = (uint16_t)f32_to_bf16_bits(val);
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WMW, int WNW, bool GATED>
hipError_t launch_cfg(const FfnArgs& a, hipStream_t stream) {
    static int per_cu = 0;
    return launch_persistent(grouped_gemm_bf16_kernel<BM, BN, WMW, WNW, GATED>, 64 * WMW * WNW, a,
                             stream, &per_cu);
}

template <int BM, bool GATED>
hipError_t launch_wide(const FfnArgs& a, hipStream_t stream) {
    static int per_cu = 0;
    return launch_persistent(wide::grouped_gemm_bf16_wide_kernel<BM, GATED>, 512, a, stream, &per_cu);
}

}  // namespace

hipError_t launch_ffn_bf16(const FfnArgs& a, bool gated, hipStream_t stream) {
    // the wide kernels address one expert's weight matrix with 32-bit offsets
    // and keep every resource extent (plus the k-step offset) below 2^31, so
    // that an out-of-range lane offset exists
    const bool wide_ok = (unsigned long long)a.N * a.ldw * 2 < (1ull << 31) &&
                         (unsigned long long)320 * (a.Kdim + 64) * 2 < (1ull << 31);
    if (wide_ok && a.rows_hint >= 192)   // ~256-row experts: one 320-row tile holds nearly all
        return gated ? launch_wide<320, true>(a, stream) : launch_wide<320, false>(a, stream);
    if (wide_ok && a.rows_hint >= 64)
        return gated ? launch_wide<256, true>(a, stream) : launch_wide<256, false>(a, stream);
    if (a.rows_hint < 24) {
        // decode-sized experts: 16-row tiles of two waves (more workgroups per
        // CU than four-wave ones: DeepSeek decode gate/up -1.6%, down -1%)
        return gated ? launch_cfg<16, 128, 1, 2, true>(a, stream)
                     : launch_cfg<16, 128, 1, 2, false>(a, stream);
    }
    return gated ? launch_cfg<128, 128, 2, 2, true>(a, stream)
                 : launch_cfg<128, 128, 2, 2, false>(a, stream);
}

}  // namespace moeep
