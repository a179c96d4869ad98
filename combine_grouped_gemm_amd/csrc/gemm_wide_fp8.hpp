// Wide fp8 (OCP e4m3) grouped GEMM tile with fp32 1x128 block scales, for
// expert row counts of a few dozen to ~190 rows (GPT-OSS-shaped prefill),
// used by ffn_fp8.hip.
//
// Same ragged persistent tile walk and direct global-to-LDS two-stage ring as
// the wide bf16 kernel: a step's row loads go out one step ahead and its
// weight loads two steps ahead (a weight buffer is refilled as soon as every
// wave holds its fragments); one k-step is one 128-byte scale block, so the
// LDS row geometry (8 swizzled 16-byte chunks per row) is identical.  The
// next tile's scales and first k-step are loaded while the current tile's
// epilogue runs.  A tile is
// up to 192 rows of one expert by 256 weight rows (gate/up: 128 gate + 128
// up rows of the same output columns, so one tile owns exactly one
// 128-column block of h and can quantise it in its epilogue).  With 192 rows
// an expert of a GPT-OSS-shaped batch (128 rows on average) fits one m-tile,
// so each weight tile is streamed from HBM once.
//
// Scales: the tile's row scales and weight-column scales for every k-block
// are copied to LDS once per tile, row-major with a fixed row stride of 23
// blocks.  With exactly 23 blocks (K in (2816, 2944]) the stride equals the
// global one, so the tile's row scales and each 128-row weight half's scales
// are one contiguous run each, copied with 16-byte loads (≈ 6 per wave
// instead of ≈ 20 four-byte ones); other K use 4-byte loads over the flat
// index.  Row (activation) scales are powers of two, so the scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 applies them itself, exactly, as E8M0
// bytes (lane l gives the scale of the row it feeds, l % 16, for its 32-byte
// slice l / 16 of the block).  With arbitrary fp32 weight scales the block
// product from a zero accumulator is folded in as acc += part * s_col; with
// power-of-two weight scales (PO2W) the MFMA applies the column scale too and
// accumulates in place, so the k-loop has no per-output vector arithmetic.
// Lane l feeds row (l % 16) with bytes [32*(l/16), 32*(l/16)+32) of the
// block for both operands.
//
// K is a multiple of 128 or leaves a 64-byte tail block (K = 2880; other K
// go through the register-staged tiles): in the tail step the direct loads of
// chunks 4..7 read a 16-byte zero block instead, so both operands are zero
// there (a garbage fp8 code could be NaN).
#pragma once

#include "gemm_wide.hpp"

namespace moeep {
namespace widefp8 {

using wide::ic;

constexpr int CPR = 8;              // 16-byte chunks per 128-byte row step
constexpr int ROWB = 128;           // bytes per LDS row = fp8 elements per k-step
constexpr int kMaxKBlocks = 23;     // scale blocks a tile keeps in LDS (K <= 2944)
constexpr int SK = kMaxKBlocks;     // LDS row stride of the scale tables (odd: conflict-free)

// source of the tail block's missing chunks
__device__ __align__(16) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

// 4 bytes per lane from global memory straight into LDS at lds_wave_base + 4 * lane
__device__ __forceinline__ void lds_dma4(const void* g, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
#endif
}

// Copies the contiguous run [run, run + count) of a scale array ending at
// `end` into LDS at lds + sh, sh = the run's float offset from the 16-byte
// boundary at or below it (returned; uniform): 16-byte direct buffer loads
// spread over the waves, lanes past the run's last piece masked off, pieces
// past `end` landing zeros.  lds must hold count + 3 floats.
template <int NW>
__device__ __forceinline__ int stage_scale_run(const float* run, const float* end, int count, float* lds,
                                               int wave, int lane) {
    const int sh = __builtin_amdgcn_readfirstlane((int)((reinterpret_cast<uintptr_t>(run) & 15u) >> 2));
    const float* al = run - sh;
    const wide::rsrc_t r = wide::make_rsrc(al, (uint32_t)((end - al) * 4));
    const int n16 = (sh + count + 3) >> 2;
    for (int q = wave; q * kWave < n16; q += NW)
        if (q * kWave + lane < n16)
            wide::lds_buf16<0>(r, lds + q * kWave * 4, (uint32_t)(q * kWave + lane) * 16u, 0);
    return sh;
}

// Waves laid out WMW (rows) x WNW (weight rows); a wave owns the interleaved
// 16-row fragments {wm, wm + WMW, ...} and BN / WNW weight rows.
template <int BM, int BN, int WMW, int WNW, bool GATED, bool PO2W>
__global__ __launch_bounds__(64 * WMW * WNW, 1) void grouped_gemm_fp8_wide_kernel(FfnArgs p) {
    constexpr int NT = 64 * WMW * WNW, NW = WMW * WNW;
    constexpr int A_BLOCKS = BM * CPR / 64;          // 1 KiB blocks of a row stage
    constexpr int B_BLOCKS = BN * CPR / 64;
    constexpr int BLOCKS = A_BLOCKS + B_BLOCKS;
    constexpr int LPS = BLOCKS / NW;                 // direct loads per wave per stage
    constexpr int FM = BM / 16 / WMW;
    constexpr int WN = BN / WNW;
    constexpr int FN = WN / 16;
    constexpr int BNO = GATED ? BN / 2 : BN;
    static_assert(BM % (16 * WMW) == 0 && BN % (16 * WNW) == 0 && (!GATED || (FN % 2 == 0 && BNO == 128)),
                  "tile shape");
    static_assert(BLOCKS % NW == 0, "every wave issues LPS loads per stage");
    static_assert(A_BLOCKS % NW == 0, "a wave's first A_LPS loads of a stage are row loads, the rest weight loads");
    constexpr int A_LPS = A_BLOCKS / NW;
    constexpr int B_LPS = LPS - A_LPS;
    // with 8 waves, load i of a stage covers 64 consecutive operand rows and
    // a lane always fetches row (wave * 8 + lane / 8) of them
    static_assert(NW == 8, "one 64-row group per load");
    constexpr int B_OFFS = (GATED ? BN / 2 : BN) / 64;   // distinct weight-row groups (gate and up share)
    static_assert(BM * SK % kWave == 0 && BN * SK % kWave == 0 && BN / 2 * SK % kWave == 0,
                  "scale staging by 64-lane loads");

    __shared__ uint4 sa0[BM * CPR];
    __shared__ uint4 sb0[BN * CPR];
    __shared__ uint4 sa1[BM * CPR];
    __shared__ uint4 sb1[BN * CPR];
    // scales, row-major with row stride SK: [tile row][k-block], [tile weight row][k-block],
    // each table starting a_sh / b_sh[half] floats into its region (room for the shift)
    __shared__ float s_as[BM * SK + 4];
    __shared__ float s_bs[BN * SK + 8];
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
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / WNW, wn = wave % WNW;
    const int Kdim = p.Kdim, N = p.N, cap = p.cap;
    const int ldw = p.ldw;                          // weight row pitch (bytes = elements)
    const int nk = (Kdim + ROWB - 1) / ROWB;        // k-steps = scale blocks (<= kMaxKBlocks)
    const bool k_tail = nk * ROWB != Kdim;          // the last block holds 64 bytes (launcher: K % 128 is 0 or 64)
    const int nbN = (N + 127) / 128;

    // largest experts' tiles first; the first row stage is free scratch until the first load
    build_tile_prefix_sorted<NT, BM>(p, s_pre, s_ord, reinterpret_cast<int*>(sa0), s_tmp);
    const int n_tiles_n = (N + BNO - 1) / BNO;
    const int total = n_tiles_n * s_pre[p.E_loc];
    const int G = gridDim.x;
    const int v = xcd_block_order();

    const uint8_t* __restrict__ A = static_cast<const uint8_t*>(p.a);
    const uint8_t* __restrict__ W0 = static_cast<const uint8_t*>(p.w0);
    const uint8_t* __restrict__ W1 = static_cast<const uint8_t*>(p.w1);

    // logical chunk this lane fetches in every direct load: rows of a 1 KiB
    // block start at multiples of 8, so (row & 7) = lane / 8
    const int lchunk = wide::swz(lane / 8, lane % 8);

    // ---- load state: the tile whose operands the direct loads fetch.  The
    // next tile's scales and first k-step are issued as soon as every wave has
    // finished the current tile's k-loop, so their latency hides behind the
    // current tile's epilogue (which then works in the second stage's buffers).
    const bool w_lines = ldw % 128 == 0;
    const char* abase = nullptr;
    const char* gbase = nullptr;
    const char* ubase = nullptr;
    uint32_t off_a[A_LPS], off_b[B_OFFS];    // lane offsets of a stage's loads (k-step 0)
    int a_sh = 0, b_sh0 = 0, b_sh1 = 4;

    // decode tile t, copy its scales to LDS and set the load state.  Scales go
    // row-major with a fixed row stride of SK = kMaxKBlocks floats ([tile
    // row][k-block]; odd, so the 16 rows one MFMA operand touches fall into
    // distinct banks).  Global scales are [row][k-block] with nk per row, so
    // 4-byte direct loads over the flat index e = row * SK + k read one
    // contiguous run per tile (a few cache lines per load); lanes with k >= nk
    // or past the valid rows / columns re-read element 0, whose value no
    // output uses.  Operand offsets are 32-bit, relative to the tile's first
    // row or to the expert's weight matrices; wave w loads the 1 KiB blocks
    // w, w + NW, ... of a stage (8 rows each; row blocks first, then weight
    // blocks); rows / columns past the valid ones re-read row 0.
    auto stage_tile = [&](int t) -> TileCoord {
        const TileCoord tc = decode_tile<BM>(t, n_tiles_n, s_pre, p, s_ord);
        const int j = tc.j, row0 = tc.row0, nvalid = tc.nvalid;
        const int col0 = tc.nt * BNO;
        const float* wgs = p.w0_scales + (size_t)j * N * nk;
        const float* wus = GATED ? p.w1_scales + (size_t)j * N * nk : nullptr;
        const float* asrc = p.a_scales + (size_t)row0 * nk;
        if (nk == SK) {
            // K = 23 blocks: a run of rows' scales is the table itself, so each
            // table (the tile's rows; each 128-row weight half) is one
            // contiguous run, copied with 16-byte loads
            a_sh = stage_scale_run<NW>(asrc, p.a_scales + (size_t)cap * nk, nvalid * nk, s_as, wave, lane);
            const int c1 = GATED ? col0 : col0 + BN / 2;
            const int n0 = min(BN / 2, N - col0), n1 = min(BN / 2, N - c1);
            b_sh0 = stage_scale_run<NW>(wgs + (size_t)col0 * nk, wgs + (size_t)N * nk, n0 * nk, s_bs, wave, lane);
            if (n1 > 0) {
                const float* h1 = GATED ? wus : wgs;
                b_sh1 = 4 + stage_scale_run<NW>(h1 + (size_t)c1 * nk, h1 + (size_t)N * nk, n1 * nk,
                                                s_bs + BN / 2 * SK + 4, wave, lane);
            }
        } else {
            a_sh = 0;
            b_sh0 = 0;
            b_sh1 = 4;
            for (int q = wave; q < BM * SK / kWave; q += NW) {
                const int e = q * kWave + lane, r = e / SK, k = e - r * SK;
                lds_dma4(asrc + (r < nvalid && k < nk ? r * nk + k : 0), s_as + q * kWave);
            }
            for (int q = wave; q < BN * SK / kWave; q += NW) {
                const int e = q * kWave + lane, c = e / SK, k = e - c * SK;      // tile weight row c
                const bool up = GATED && c >= BN / 2;
                const int col = col0 + (up ? c - BN / 2 : c);
                const float* bsrc = up ? wus : wgs;
                // the second half's table starts 4 floats further on (a wave's 64
                // entries never straddle the halves, so the LDS base stays uniform)
                lds_dma4(bsrc + (col < N && k < nk ? (size_t)col * nk + k : 0),
                         s_bs + q * kWave + (q * kWave >= BN / 2 * SK ? 4 : 0));
            }
        }
        abase = reinterpret_cast<const char*>(A + (size_t)row0 * Kdim);
        gbase = reinterpret_cast<const char*>(W0 + (size_t)j * N * ldw);
        ubase = GATED ? reinterpret_cast<const char*>(W1 + (size_t)j * N * ldw) : nullptr;
        const int lrow = wave * 8 + lane / 8;
        const uint32_t c16 = (uint32_t)lchunk * 16;
#pragma unroll
        for (int i = 0; i < A_LPS; ++i) {
            const int r = i * 64 + lrow;
            off_a[i] = (uint32_t)(r < nvalid ? r : 0) * (uint32_t)Kdim + c16;
        }
#pragma unroll
        for (int i = 0; i < B_OFFS; ++i) {
            const int col = col0 + i * 64 + lrow;
            off_b[i] = (uint32_t)(col < N ? col : 0) * (uint32_t)ldw + c16;
        }
        return tc;
    };
    // Weight rows are streamed with the non-temporal hint only when they start
    // on 128-byte lines (a row pitch that is a multiple of 128, as packed
    // weights have): otherwise a k-step's 128 bytes straddle two lines and the
    // next k-step re-reads the second one, which must still be in L2.
    auto issue_p = [&](auto I, int kstep, auto WPOL, auto FIRST, auto LAST) {
        const uint32_t kb = (uint32_t)kstep * ROWB;
        // in a 64-byte last block, chunks 4..7 come from the zero block
        const bool zl = k_tail && kstep == nk - 1 && lchunk >= 4;
#pragma unroll
        for (int i = decltype(FIRST)::value; i < decltype(LAST)::value; ++i) {
            const int q = i * NW + wave;                 // < BLOCKS: LPS * NW == BLOCKS
            // operand, gate / up half and row group are known per unrolled load
            const bool is_a = i < A_LPS;
            const int ib = i - A_LPS;
            const bool up = GATED && !is_a && ib * 64 >= BN / 2;
            const char* b = is_a ? abase : (up ? ubase : gbase);
            const uint32_t o = is_a ? off_a[is_a ? i : 0] : off_b[is_a ? 0 : ib % B_OFFS];
            char* dst = is_a ? a_base(I) + q * 1024 : b_base(I) + (q - A_BLOCKS) * 1024;
            // 32-bit offset add: a uniform base plus one lane offset per load
            const char* src = zl ? reinterpret_cast<const char*>(kZeroChunk) : b + (uint32_t)(o + kb);
            if (is_a)
                wide::lds_dma16<0>(src, dst);
            else
                wide::lds_dma16<decltype(WPOL)::value>(src, dst);
        }
    };
    // a k-step's row loads, its weight loads, or both
    auto issue_a = [&](auto I, int kstep) { issue_p(I, kstep, ic<0>{}, ic<0>{}, ic<A_LPS>{}); };
    auto issue_b = [&](auto I, int kstep) {
        if (w_lines) issue_p(I, kstep, ic<wide::kNonTemporal>{}, ic<A_LPS>{}, ic<LPS>{});
        else issue_p(I, kstep, ic<0>{}, ic<A_LPS>{}, ic<LPS>{});
    };
    auto issue = [&](auto I, int kstep) {
        issue_a(I, kstep);
        issue_b(I, kstep);
    };

    TileCoord cur{};
    if (v < total) {
        cur = stage_tile(v);
        issue(ic<0>{}, 0);
    }
    for (int tau = v; tau < total; tau += G) {
        const int row0 = cur.row0, nvalid = cur.nvalid, nt = cur.nt;
        const int col0 = nt * BNO;

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

        const int c0 = 2 * (lane >> 4);                 // first logical chunk this lane feeds
        // a wave whose output columns all lie past N (the last n-tile of an
        // expert when N is not a multiple of the tile width) skips its MFMAs
        const bool wcols = fcol(0) < N;
        auto compute = [&](auto I, int kstep) {
            const char* ab = a_base(I);
            const char* bb = b_base(I);
            intx8 bfr[FN];
            float bsc[FN];
            static_assert(FN == 4, "weight fragment reads");
            {
                uint32_t ad[2 * FN];
                uint4 t[2 * FN];
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    const int r = brow(f);
                    ad[2 * f] = wide::lds_addr(bb + r * ROWB + wide::swz(r, c0) * 16);
                    ad[2 * f + 1] = wide::lds_addr(bb + r * ROWB + wide::swz(r, c0 + 1) * 16);
                }
                wide::lds_read16x8(t, ad);
#pragma unroll
                for (int f = 0; f < FN; ++f)
                    bfr[f] = intx8{(int)t[2 * f].x, (int)t[2 * f].y, (int)t[2 * f].z, (int)t[2 * f].w,
                                   (int)t[2 * f + 1].x, (int)t[2 * f + 1].y, (int)t[2 * f + 1].z, (int)t[2 * f + 1].w};
            }
            // (issued after this step's fragment reads, which therefore need
            // not wait for them) step 1's weights on a tile's first step, then
            // step kstep + 1's rows into the other row buffer
            if (kstep == 0 && nk > 1) issue_b(ic<1>{}, 1);
            if (kstep + 1 < nk) issue_a(ic<1 - decltype(I)::value>{}, kstep + 1);
            // every wave holds this step's weight fragments: their buffer
            // takes step kstep + 2's weights
            if (kstep + 2 < nk) {
                wide::wait_lgkm0();
                wide::block_barrier();
                issue_b(I, kstep + 2);
            }
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                const int r = brow(f);
                bsc[f] = s_bs[(r < BN / 2 ? b_sh0 : b_sh1) + r * SK + kstep];
            }
            int sb8[FN];        // weight-row scales as E8M0 bytes (power-of-two weight scales)
#pragma unroll
            for (int f = 0; f < FN; ++f) sb8[f] = PO2W ? e8m0_of_pow2(bsc[f]) : 127;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mrow = (wm + WMW * i) * 16;
                if (mrow < nvalid && wcols) {
                    const int r = mrow + (lane & 15);
                    const uint4 t0 = *reinterpret_cast<const uint4*>(ab + r * ROWB + wide::swz(r, c0) * 16);
                    const uint4 t1 = *reinterpret_cast<const uint4*>(ab + r * ROWB + wide::swz(r, c0 + 1) * 16);
                    const intx8 afr = intx8{(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w,
                                            (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
                    // the row scale (a power of two) of the A row this lane
                    // feeds, as an E8M0 byte: the matrix core applies it
                    const int sa8 = e8m0_of_pow2(s_as[a_sh + r * SK + kstep]);
                    if constexpr (PO2W) {
                        // both scales in the matrix core: accumulate in place
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                afr, bfr[f], acc[i][f], 0, 0, 0, sa8, 0, sb8[f]);
                    } else {
                        // all four products first, then their column scaling:
                        // the MFMAs do not wait for each other's consumers
                        floatx4 part[FN];
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            part[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                afr, bfr[f], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, sa8, 0, 127);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[i][f][e] = fmaf(part[f][e], bsc[f], acc[i][f][e]);
                    }
                }
            }
        };

        // step k: wait for stage k's rows and weights (step k + 1's weights,
        // issued during step k - 1, stay in flight) and compute it; the
        // compute loads step k + 1's rows into the other row buffer and, once
        // every wave holds step k's weight fragments in registers, step k +
        // 2's weights into their buffer, so the weight stream keeps one to two
        // k-steps in flight instead of draining at every step.
        auto step = [&](auto I, int k) {
            if (k > 0 && k + 1 < nk) wide::wait_vmcnt<B_LPS>();
            else wide::wait_vmcnt<0>();
            wide::wait_lgkm0();
            wide::block_barrier();
            compute(I, k);
        };
        for (int k = 0; k < nk; k += 2) {
            step(ic<0>{}, k);
            if (k + 1 < nk) step(ic<1>{}, k + 1);
        }

        // every wave is done with both stages and the scale tables: start the
        // next tile's loads into stage 0 and the scale tables
        wide::wait_lgkm0();
        wide::block_barrier();
        if (tau + G < total) {
            cur = stage_tile(tau + G);
            issue(ic<0>{}, 0);
        }

        // ---- epilogue (LDS: only the second stage's buffers; the barriers wait
        // for LDS traffic, not for the next tile's loads in flight)
        if constexpr (GATED) {
            // h = silu(g) * u; the tile's 128 columns are one scale block of h:
            // row amax over 16 lanes (DPP row) and the 4 column waves
            float* s_amax = reinterpret_cast<float*>(sb1);
            // the h tile (BM rows x 128 bytes) is assembled in the row buffer
            // and leaves as 16-byte row chunks; chunk c of row r sits at chunk
            // c ^ (r % 8), so the eight rows of one half-wave dword write fall
            // into distinct banks
            uint8_t* h_tile = reinterpret_cast<uint8_t*>(sa1);
            // row scales of h, stored with the tile (no global store inside the
            // loop above: a wait for one would also wait for the loads in flight)
            float* s_hscale = s_amax + WNW * BM;
            static_assert((WNW + 2) * BM * 4 <= BN * ROWB, "amax partials, row scales and reciprocals fit the weight buffer");
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
                        // computed for every column and zeroed past N (a select, not
                        // a branch per element, so the exponentials and reciprocals of
                        // different elements interleave); columns past N hold finite
                        // values, their weight rows having re-read row 0
                        const float hs = silu(acc[i][f][e]) * acc[i][f + FO][e];
                        const float h = fcol(f) < N ? hs : 0.f;
                        hv[i][f][e] = h;
                        rmax[i][e] = fmaxf(rmax[i][e], fabsf(h));
                    }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float m = row16_max(rmax[i][e]);
                    if ((lane & 15) == 0) s_amax[wn * BM + (wm + WMW * i) * 16 + (lane >> 4) * 4 + e] = m;
                }
            wide::wait_lgkm0();
            wide::block_barrier();
            // one thread per row: the row's scale and its reciprocal
            float* s_hrs = s_hscale + BM;
            for (int r = tid; r < BM; r += NT) {
                float amax = 0.f;
#pragma unroll
                for (int w = 0; w < WNW; ++w) amax = fmaxf(amax, s_amax[w * BM + r]);
                const float s = pow2_block_scale(amax);
                s_hscale[r] = s;
                s_hrs[r] = pow2_recip(s);
            }
            wide::wait_lgkm0();
            wide::block_barrier();
            static_assert(FO == 2 && WN / 2 == 32, "two 16-column chunks per wave and fragment row");
            // A lane holds the codes of one column in each of the wave's two
            // chunks for four rows; a 4 x 4 byte transpose inside each quad
            // (partners lane ^ 2, then lane ^ 1: a DPP move and a byte permute
            // each) leaves lane j of the quad with four consecutive columns of
            // row j, written as one dword per chunk.
            const int qj = lane & 3;
            const uint32_t selA = qj < 2 ? 0x05040100u : 0x03020706u;    // keep low / high half
            const uint32_t selB = (qj & 1) == 0 ? 0x06020400u : 0x03070105u;
            auto quad_transpose = [&](uint32_t v) {
                const uint32_t x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
                const uint32_t a2 = __builtin_amdgcn_perm(x, v, selA);
                const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a2, 0xB1, 0xF, 0xF, false);
                return __builtin_amdgcn_perm(y, a2, selB);
            };
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int mrow = (wm + WMW * i) * 16;
                if (mrow >= nvalid) continue;                            // wave-uniform
                const int rb = mrow + (lane >> 4) * 4;                   // this lane's first row
                const float4 rs = *reinterpret_cast<const float4*>(s_hrs + rb);
                // |h| <= amax <= 448 s: the hardware conversion needs no saturation
                uint32_t p0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hv[i][0][0] * rs.x, hv[i][0][1] * rs.y, 0, false);
                p0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hv[i][0][2] * rs.z, hv[i][0][3] * rs.w, (int)p0, true);
                uint32_t p1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hv[i][1][0] * rs.x, hv[i][1][1] * rs.y, 0, false);
                p1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hv[i][1][2] * rs.z, hv[i][1][3] * rs.w, (int)p1, true);
                const uint32_t t0 = quad_transpose(p0), t1 = quad_transpose(p1);
                const int r = rb + qj;
                uint8_t* row = h_tile + r * ROWB + (lane & 12);             // dword (lane % 16) / 4 of a chunk
                *reinterpret_cast<uint32_t*>(row + ((2 * wn) ^ (r & 7)) * 16) = t0;
                *reinterpret_cast<uint32_t*>(row + ((2 * wn + 1) ^ (r & 7)) * 16) = t1;
            }
            wide::wait_lgkm0();
            wide::block_barrier();
            // rows [0, nvalid) x the valid 16-byte chunks of the tile's columns
            uint8_t* Out = static_cast<uint8_t*>(p.out);
            const int nchunk = min(8, (N - col0) / 16);
            for (int t = tid; t < nvalid * 8; t += NT) {
                const int r = t >> 3, c = t & 7;
                if (c < nchunk) {
                    const uint4 v = *reinterpret_cast<const uint4*>(h_tile + r * ROWB + ((c ^ (r & 7)) * 16));
                    *reinterpret_cast<uint4*>(Out + (size_t)(row0 + r) * N + col0 + c * 16) = v;
                }
            }
            for (int r = tid; r < nvalid; r += NT) p.out_scales[(size_t)(row0 + r) * nbN + nt] = s_hscale[r];
        } else {
            // bf16 outputs: every wave stages its 64 columns in a private region
            // of the second stage's buffers (the first already receives the next
            // tile's loads) and stores whole 16-byte row chunks, 8 per 128-byte
            // output row piece, instead of one 2-byte store per element.  PF
            // fragments per pass; staged rows are padded by 16 bytes so that the
            // four row groups of one LDS write fall into different banks.  The
            // regions are private, so the passes need no barrier: one wave's LDS
            // accesses take effect in order.
            constexpr int OCOLS = FN * 16;                  // output columns of a wave
            constexpr int OCH = OCOLS * 2 / 16;             // 16-byte chunks per staged row
            constexpr int OPITCH = OCOLS * 2 + 16;          // staged row pitch (bytes)
            constexpr int PF = 2;                           // fragments per pass
            constexpr int RSZ = PF * 16 * OPITCH;           // bytes of a wave's region
            constexpr int NRA = (int)sizeof(sa1) / RSZ;     // regions in the row buffer
            static_assert(NRA + (int)sizeof(sb1) / RSZ >= NW, "a region per wave");
            char* region = wave < NRA ? reinterpret_cast<char*>(sa1) + wave * RSZ
                                      : reinterpret_cast<char*>(sb1) + (wave - NRA) * RSZ;
            const int colbase = fcol(0);                    // the wave's first output column
            char* out_bytes = static_cast<char*>(p.out);
#pragma unroll
            for (int p0 = 0; p0 < FM; p0 += PF) {
#pragma unroll
                for (int ii = 0; ii < PF; ++ii) {
                    const int i = p0 + ii;
                    if (i < FM) {
#pragma unroll
                        for (int f = 0; f < FN; ++f)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int lrow = ii * 16 + (lane >> 4) * 4 + e;
                                *reinterpret_cast<uint16_t*>(region + lrow * OPITCH + (f * 16 + (lane & 15)) * 2) =
                                    (uint16_t)f32_to_bf16_bits(acc[i][f][e]);
                            }
                    }
                }
                constexpr int RPI = 64 / OCH;               // staged rows per 64-lane read
#pragma unroll
                for (int q = 0; q < PF * 16 / RPI; ++q) {
                    const int lrow = q * RPI + lane / OCH, ch = lane % OCH;
                    const int i = p0 + lrow / 16;
                    const int trow = (wm + WMW * i) * 16 + lrow % 16;   // row within the tile
                    const int col = colbase + ch * 8;                   // N is a multiple of 16
                    if (i < FM && trow < nvalid && col < N) {
                        const uint4 v = *reinterpret_cast<const uint4*>(region + lrow * OPITCH + ch * 16);
                        *reinterpret_cast<uint4*>(out_bytes + ((size_t)(row0 + trow) * N + col) * 2) = v;
                    }
                }
            }
        }
    }
}

}  // namespace widefp8
}  // namespace moeep
