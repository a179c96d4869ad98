// Grouped SwiGLU expert FFN with fp8 e4m3 operands and fp32 1x128 block
// scales (SGLang "Expert Parallelism", MoE-runner backend table: block-wise
// fp8 quantisation for the grouped GEMM; the block geometry is this
// library's convention, one scale per 128 contraction elements).
//
// Two kernels: the wide one (gemm_wide_fp8.hpp: direct global-to-LDS ring,
// 192-row tiles, scales staged per tile) for expert row counts from a few
// dozen up and K <= 2944; the register-staged one below for decode-sized
// row counts or longer K.  The register-staged kernel uses the same ragged
// persistent tile walk as the bf16 kernel.  One k-step is one
// 128-wide scale block: v_mfma_f32_16x16x128_f8f6f4 (both operands OCP
// e4m3) produces the unscaled block product from a zero accumulator, which
// is folded into the fp32 accumulator as acc += partial * sa[row] * sb[col].
// Lane l feeds row (l % 16) with bytes [32*(l/16), 32*(l/16)+32) of the
// block for both operands.  A partial tail block (K = 2880 leaves 64 of
// 128; K is a multiple of 16) is zero-filled on both operands.
//
// gate/up writes h as fp8: each tile covers exactly one 128-column block of
// h per row, so the block amax is reduced inside the tile (the 16 lanes of a
// DPP row, then the waves of a row through LDS), s is the smallest power of
// two with amax <= 448 s, and the codes are written with the scale.
#include "gemm_wide_fp8.hpp"
#include "grouped_tiles.hpp"

namespace moeep {
namespace {

constexpr int BKB = 128;          // bytes (= fp8 elements) per k-step

constexpr int kTabKB = 32;        // scale blocks per row the E8M0 weight-scale table holds

// PO2W: the weight scales are powers of two.  Then a tile's weight-row scales
// for every k-block are staged once, as E8M0 bytes, in an LDS table
// (coalesced loads of the contiguous scale runs) instead of one scattered
// 4-byte load per weight row and k-step, and the scaled MFMA applies both
// scales and accumulates in place.
template <int BM, int BN, int WMW, int WNW, bool GATED, bool PO2W>
__global__ __launch_bounds__(64 * WMW * WNW) void grouped_gemm_fp8_kernel(FfnArgs p) {
    constexpr int NT = 64 * WMW * WNW;
    constexpr int FM = BM / 16 / WMW;
    constexpr int WN = BN / WNW;
    constexpr int FN = WN / 16;
    constexpr int BNO = GATED ? BN / 2 : BN;
    static_assert(FM >= 1 && FN >= 1 && (!GATED || (FN % 2 == 0 && BNO == 128)), "tile shape");
    static_assert(BM <= NT && BN <= NT, "one row scale and one column scale per thread and k-block");
    constexpr int A_IT = (BM * 8 + NT - 1) / NT;
    constexpr int B_IT = (BN * 8 + NT - 1) / NT;

    __shared__ uint4 sA[BM * 8];
    __shared__ uint4 sB[BN * 8];
    __shared__ float sAs[BM];
    __shared__ float sBs[BN];
    __shared__ uint8_t sBe[PO2W ? BN * kTabKB : 4];     // [weight row][k-block] E8M0
    __shared__ float s_amax[WNW][BM];
    __shared__ int s_pre[kMaxExperts + 1];
    __shared__ int s_tmp[NT / kWave];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / WNW, wn = wave % WNW;
    const int Kdim = p.Kdim, N = p.N, cap = p.cap, ldw = p.ldw;
    const int nbK = (Kdim + BKB - 1) / BKB;
    const int nbN = (N + 127) / 128;

    build_tile_prefix<NT, BM>(p, s_pre, s_tmp);
    const int n_tiles_n = (N + BNO - 1) / BNO;
    const int total = n_tiles_n * s_pre[p.E_loc];
    const int G = gridDim.x;
    const int v = xcd_block_order();

    const uint8_t* __restrict__ A = static_cast<const uint8_t*>(p.a);
    const uint8_t* __restrict__ W0 = static_cast<const uint8_t*>(p.w0);
    const uint8_t* __restrict__ W1 = static_cast<const uint8_t*>(p.w1);

    for (int rnd = 0;; ++rnd) {
        const int tau = round_tile(rnd, v, blockIdx.x, G, total);
        if (tau < 0) break;
        const TileCoord tc = decode_tile<BM>(tau, n_tiles_n, s_pre, p);
        const int j = tc.j, row0 = tc.row0, nvalid = tc.nvalid;
        const int col0 = tc.nt * BNO;
        const uint8_t* wg = W0 + (size_t)j * N * ldw;
        const uint8_t* wu = GATED ? W1 + (size_t)j * N * ldw : nullptr;
        const float* wgs = p.w0_scales + (size_t)j * N * nbK;
        const float* wus = GATED ? p.w1_scales + (size_t)j * N * nbK : nullptr;

        if constexpr (PO2W) {
            __syncthreads();                       // the previous tile's reads of sBe are done
            for (int e = tid; e < BN * nbK; e += NT) {
                const int c = e / nbK, k = e - c * nbK;
                const bool up = GATED && c >= BN / 2;
                const int col = col0 + (up ? c - BN / 2 : c);
                const float* sp = up ? wus : wgs;
                sBe[c * kTabKB + k] = (uint8_t)(col < N ? e8m0_of_pow2(sp[(size_t)col * nbK + k]) : 127);
            }
        }

        uint4 ra[A_IT], rb[B_IT];
        float ras = 0.f, rbs = 0.f;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) ra[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_IT; ++i) rb[i] = make_uint4(0, 0, 0, 0);

        auto load_step = [&](int kb) {
            const int k0 = kb * BKB;
#pragma unroll
            for (int i = 0; i < A_IT; ++i) {
                const int q = tid + i * NT;
                const int r = q >> 3, c = q & 7;
                if (q < BM * 8 && r < nvalid) {
                    ra[i] = (k0 + c * 16 < Kdim)
                                ? *reinterpret_cast<const uint4*>(A + (size_t)(row0 + r) * Kdim + k0 + c * 16)
                                : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < B_IT; ++i) {
                const int q = tid + i * NT;
                const int r = q >> 3, c = q & 7;
                if (q < BN * 8) {
                    int col;
                    const uint8_t* src;
                    if (GATED) {
                        const bool up = r >= BN / 2;
                        col = col0 + (up ? r - BN / 2 : r);
                        src = up ? wu : wg;
                    } else {
                        col = col0 + r;
                        src = wg;
                    }
                    rb[i] = (col < N && k0 + c * 16 < Kdim)
                                ? *reinterpret_cast<const uint4*>(src + (size_t)col * ldw + k0 + c * 16)
                                : make_uint4(0, 0, 0, 0);
                }
            }
            // scales of this k-block: thread tid < BM loads a row scale, BM <= tid < BM+BN a column scale
            if (tid < BM) {
                ras = (tid < nvalid) ? p.a_scales[(size_t)(row0 + tid) * nbK + kb] : 0.f;
            }
            const int bt = tid - (NT - BN);           // the last BN threads load column scales
            if (!PO2W && bt >= 0 && bt < BN) {
                int col;
                const float* sp;
                if (GATED) {
                    const bool up = bt >= BN / 2;
                    col = col0 + (up ? bt - BN / 2 : bt);
                    sp = up ? wus : wgs;
                } else {
                    col = col0 + bt;
                    sp = wgs;
                }
                rbs = (col < N) ? sp[(size_t)col * nbK + kb] : 0.f;
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
            if (tid < BM) sAs[tid] = ras;
            const int bt = tid - (NT - BN);
            if (!PO2W && bt >= 0 && bt < BN) sBs[bt] = rbs;
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
                return half + wn * (WN / 2) + ff * 16 + (lane & 15);
            }
            return wn * WN + f * 16 + (lane & 15);
        };
        auto fcol = [&](int f) {
            if (GATED) {
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return col0 + wn * (WN / 2) + ff * 16;
            }
            return col0 + wn * WN + f * 16;
        };

        load_step(0);
        for (int kb = 0; kb < nbK; ++kb) {
            __syncthreads();
            store_step();
            __syncthreads();
            if (kb + 1 < nbK) load_step(kb + 1);
            const int c0 = 2 * (lane >> 4);
            intx8 bfr[FN];
            float bsc[FN];
            int sb8[FN];
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                const int r = brow(f);
                const uint4 t0 = sB[r * 8 + (c0 ^ (r & 7))];
                const uint4 t1 = sB[r * 8 + ((c0 + 1) ^ (r & 7))];
                bfr[f] = intx8{(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w,
                               (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
                if constexpr (PO2W) sb8[f] = sBe[r * kTabKB + kb];
                else bsc[f] = sBs[r];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mrow = (wm + WMW * i) * 16;
                if (mrow < nvalid) {
                    const int r = mrow + (lane & 15);
                    const uint4 t0 = sA[r * 8 + (c0 ^ (r & 7))];
                    const uint4 t1 = sA[r * 8 + ((c0 + 1) ^ (r & 7))];
                    const intx8 afr = intx8{(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w,
                                            (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
                    if constexpr (PO2W) {
                        // the power-of-two scale of the row this lane feeds, and of
                        // each weight row, as E8M0 bytes: the matrix core applies both
                        const int sa8 = e8m0_of_pow2(sAs[r]);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            if (fcol(f) < N)
                                acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    afr, bfr[f], acc[i][f], 0, 0, 0, sa8, 0, sb8[f]);
                    } else {
                        float asc[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) asc[e] = sAs[mrow + (lane >> 4) * 4 + e];
#pragma unroll
                        for (int f = 0; f < FN; ++f) {
                            if (fcol(f) < N) {
                                const floatx4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    afr, bfr[f], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                                // lane l's outputs sit in column l % 16, whose scale bsc[f] holds
#pragma unroll
                                for (int e = 0; e < 4; ++e) acc[i][f][e] = fmaf(part[e], asc[e] * bsc[f], acc[i][f][e]);
                            }
                        }
                    }
                }
            }
        }

        // ---- epilogue
        if constexpr (GATED) {
            // h = silu(g) * u, then per-row amax over the tile's 128 columns
            constexpr int FO = FN / 2;
            float hv[FM][FO][4];
            float rmax[FM][4];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) rmax[i][e] = 0.f;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int f = 0; f < FO; ++f)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = fcol(f) + (lane & 15) < N;
                        const float h = ok ? silu(acc[i][f][e]) * acc[i][f + FO][e] : 0.f;
                        hv[i][f][e] = h;
                        rmax[i][e] = fmaxf(rmax[i][e], fabsf(h));
                    }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float m = row16_max(rmax[i][e]);
                    if ((lane & 15) == 0) s_amax[wn][(wm + WMW * i) * 16 + (lane >> 4) * 4 + e] = m;
                }
            __syncthreads();
            uint8_t* Out = static_cast<uint8_t*>(p.out);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mrow = (wm + WMW * i) * 16;
                if (mrow >= nvalid) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = mrow + (lane >> 4) * 4 + e;
                    if (r >= nvalid) continue;
                    float amax = 0.f;
#pragma unroll
                    for (int w = 0; w < WNW; ++w) amax = fmaxf(amax, s_amax[w][r]);
                    const float s = pow2_block_scale(amax);
                    const float rs = 1.0f / s;       // exact: s is a power of two
#pragma unroll
                    for (int f = 0; f < FO; ++f) {
                        const int col = fcol(f) + (lane & 15);
                        if (col < N) Out[(size_t)(row0 + r) * N + col] = (uint8_t)f32_to_e4m3_sat(hv[i][f][e] * rs);
                    }
                    if (wn == 0 && (lane & 15) == 0) p.out_scales[(size_t)(row0 + r) * nbN + tc.nt] = s;
                }
            }
            __syncthreads();
        } else {
            uint16_t* Out = static_cast<uint16_t*>(p.out);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mrow = (wm + WMW * i) * 16;
                if (mrow >= nvalid) continue;
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    const int col = fcol(f) + (lane & 15);
                    if (col >= N) continue;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = mrow + (lane >> 4) * 4 + e;
                        if (r < nvalid) Out[(size_t)(row0 + r) * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][f][e]);
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WMW, int WNW, bool GATED, bool PO2W>
hipError_t launch_cfg(const FfnArgs& a, hipStream_t stream) {
    static int per_cu = 0;
    return launch_persistent(grouped_gemm_fp8_kernel<BM, BN, WMW, WNW, GATED, PO2W>, 64 * WMW * WNW, a,
                             stream, &per_cu);
}

template <bool GATED, bool PO2W>
hipError_t launch_wide(const FfnArgs& a, hipStream_t stream) {
    static int per_cu = 0;
    return launch_persistent(widefp8::grouped_gemm_fp8_wide_kernel<192, 256, 2, 4, GATED, PO2W>, 512, a,
                             stream, &per_cu);
}

}  // namespace

hipError_t launch_ffn_fp8(const FfnArgs& a, bool gated, hipStream_t stream) {
    // the wide kernel keeps all of a tile's scale blocks in LDS, addresses an
    // expert's weight matrix with 32-bit offsets and takes a whole or a half
    // (64-byte) last block
    const int nbK = (a.Kdim + 127) / 128;
    const bool wide_ok = nbK <= widefp8::kMaxKBlocks && (a.Kdim % 128 == 0 || a.Kdim % 128 == 64) &&
                         (unsigned long long)a.N * a.ldw < (1ull << 32);
    if (wide_ok && a.rows_hint >= 48) {
        if (a.w_scales_pow2)
            return gated ? launch_wide<true, true>(a, stream) : launch_wide<false, true>(a, stream);
        return gated ? launch_wide<true, false>(a, stream) : launch_wide<false, false>(a, stream);
    }
    if (a.w_scales_pow2 && nbK <= kTabKB && a.rows_hint < 8) {
        // decode-sized experts (a few rows each): 16-row tiles of 256 threads,
        // small enough (LDS and registers) for several workgroups per CU, with
        // the weight-row scales staged once per tile (measured: +21% gate/up,
        // +9% down at 4 rows per expert; at 16 or more rows the 128-row tiles
        // below are faster)
        return gated ? launch_cfg<16, 256, 1, 4, true, true>(a, stream)
                     : launch_cfg<16, 128, 1, 4, false, true>(a, stream);
    }
    return gated ? launch_cfg<128, 256, 2, 4, true, false>(a, stream)
                 : launch_cfg<128, 128, 2, 2, false, false>(a, stream);
}

}  // namespace moeep
