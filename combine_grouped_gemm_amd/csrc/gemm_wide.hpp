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
// Operands go from global memory straight into LDS by buffer loads
// (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at the wave's LDS
// base + 16 * lane) through two k-step buffers.  A scalar buffer resource per
// operand bounds its extent, so rows past the tile's valid rows (and weight
// rows past N) read no memory and land zeros, and every stage is the same
// LPS loads per wave.  Each buffer is its own __shared__ object and the k loop
// is unrolled by two so every LDS access names its buffer statically: the
// compiler can then see that reads of one stage do not alias the loads in
// flight into the other and does not drain the loads before every LDS read.
// The 16-byte chunks of a row are XOR-swizzled by (row & 7) so the 16 rows
// one MFMA operand read touches fall into distinct LDS banks; the loads
// permute which global chunk each lane fetches to produce that layout.
//
// A wave's valid row fragments are a prefix of its fragments, so the tile
// runs one of FM + 1 copies of the k loop, selected by that count: no branch
// inside a step, so the compiler keeps the accumulators in place, prefetches
// the next fragment's rows under the current fragment's MFMAs, and the next
// stage's loads go out one after each fragment's MFMA group (the order is
// pinned with scheduling fences).  Issued all at once, they stalled every
// wave of the workgroup on a full memory queue for 800-1400 cycles per step.
//
// Measured limits on MI355X that shaped this: per k-step the loads of the
// next stage (32 KB of weights from HBM, 32-40 KB of rows from L2) take about
// as long as the MFMA work of the current one, and the two waves that share a
// SIMD finish their MFMA groups about 1000 cycles apart.  The weight stream
// therefore runs two steps ahead: once every wave holds a step's weight
// fragments in registers (256-row tiles: both k-halves at the start of the
// step; 320-row tiles, which lack the registers: the second k-half), a
// barrier releases that weight buffer and step k + 2's weights go into it.
// Issuing a whole stage before waiting for the previous one, loads in the
// order weights first, and two loads per fragment were each measured slower;
// deeper rings do not fit in LDS.
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

// Buffer resource over [base, base + bytes): raw (stride 0), so an access
// at byte offset o >= bytes is out of range: it reads no memory and returns
// zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;      // 32-bit data format, no swizzle
// A lane offset no buffer resource here reaches: the launcher keeps every
// extent (and extent plus k-step offset) below 2^31.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16 bytes per lane through a buffer resource straight into LDS at
// lds_wave_base + 16 * lane (the device-pass-only wrapper of lds_dma16).
template <int CPOL>
__device__ __forceinline__ void lds_buf16(rsrc_t r, void* lds_wave_base, uint32_t voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                             (int)voff, soff, 0, CPOL);
#endif
}

// Eight 16-byte LDS reads in one block that also waits for them: operand
// fragments of a buffer whose loads for a later step are issued right
// after, kept out of the compiler's own wait placement (which, not knowing
// on every path which direct loads are still in flight, waits for all of
// them before the first read).
__device__ __forceinline__ void lds_read16x8(uint4 (&t)[8], const uint32_t (&ad)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
}

__device__ __forceinline__ void lds_read16x4(uint4 (&t)[4], const uint32_t (&ad)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
}

// 32-bit LDS address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) char*)reinterpret_cast<const char*>(p));
}

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
    constexpr int B_ITERS = LPS - A_ITERS;           // weight loads per wave per stage
    // Tiles of at most 256 rows keep both k-halves' weight fragments of a step
    // in registers, so the weight buffer of step k takes step k + 2's weights
    // as soon as every wave holds them (the weight stream keeps up to two
    // steps in flight); 320-row tiles have no registers to spare for that.
    constexpr bool LOOK = BM <= 256;
    // wider tiles release the weight buffer half-way: step k + 2's weights go
    // out during the second k-half, once every wave holds its fragments
    constexpr bool HALF = !LOOK;

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
    const int ldw = p.ldw;                          // weight row pitch (elements)
    const int nk = (Kdim + BK - 1) / BK;            // the last k-step may be partial (K % 64 != 0)
    // contraction offset, within a k-step, of the 16-byte chunk this lane
    // fetches in every direct load (rows of a load's 1 KiB block start at
    // multiples of 8, so a row's (row & 7) is lane / 8)
    const int lane_k = swz(lane / 8, lane % 8) * 8;

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
        const uint16_t* wg = W0 + (size_t)j * N * ldw;
        const uint16_t* wu = GATED ? W1 + (size_t)j * N * ldw : nullptr;

        // Operands come in by buffer loads straight into LDS: a scalar resource
        // per operand (base, byte extent) plus a 32-bit per-lane offset and the
        // k-step as scalar offset.  Rows past the tile's valid rows and weight
        // rows past N lie outside their resource's extent, so those lanes read
        // nothing from memory and land zeros.  Each lane's offset is fixed for
        // the tile.
        const char* abase = reinterpret_cast<const char*>(A + (size_t)row0 * Kdim);
        const uint32_t a_bytes = (uint32_t)nvalid * (uint32_t)(Kdim * 2);
        const uint32_t w_bytes = (uint32_t)N * (uint32_t)(ldw * 2);
        uint32_t off[LPS];
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const bool is_a = i < A_ITERS;
            const int r = (is_a ? i * NW : (i - A_ITERS) * NW) * 8 + wave * 8 + lane / 8;
            const uint32_t c16 = (uint32_t)swz(r, lane % 8) * 16;   // logical chunk this lane fetches
            const int rr = (!is_a && GATED && r >= BN / 2) ? r - BN / 2 : r;
            off[i] = (is_a ? (uint32_t)r * (uint32_t)(Kdim * 2) : (uint32_t)(col0 + rr) * (uint32_t)(ldw * 2)) + c16;
        }
        // direct load i of a stage; `live` false (the step after the last) reads
        // nothing, so every step issues the same LPS loads without a branch
        auto issue_one = [&](auto I, int i, int kstep, bool live) {
            const bool is_a = i < A_ITERS;
            const bool up = GATED && i >= A_ITERS + G_ITERS;
            char* dst = is_a ? a_base(I) + (i * NW + wave) * 1024
                             : b_base(I) + ((i - A_ITERS) * NW + wave) * 1024;
            // the step after the last gets an empty extent: every access out of range
            const rsrc_t r = make_rsrc(is_a ? (const void*)abase : (up ? (const void*)wu : (const void*)wg),
                                       live ? (is_a ? a_bytes : w_bytes) : 0u);
            // chunks past K (a partial last step) get an offset beyond every
            // extent, so they read nothing and land zeros in both operands
            const uint32_t vo = kstep * BK + lane_k < Kdim ? off[i] : kOutOfRange;
            // the row block is re-read by every n-tile of the expert (kept in
            // L2); weight tiles are read by one or two m-tiles close together in
            // tile order, so only the weights stream (non-temporal)
            if (is_a)
                lds_buf16<0>(r, dst, vo, kstep * BK * 2);
            else
                lds_buf16<kNonTemporal>(r, dst, vo, kstep * BK * 2);
        };

        // per-lane LDS byte offset of the 16-byte chunk this lane feeds to an
        // MFMA at half-step kk, for any operand row that is a multiple of 16
        // plus (lane & 15): the swizzle then depends on the lane alone
        int lds_lane[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            lds_lane[kk] = (lane & 15) * ROWB + (((kk * 4 + (lane >> 4)) ^ (lane & 7)) * 16);
        auto brow0 = [&](int f) {     // first B-tile row of n-fragment f
            if (GATED) {
                const int half = f < FN / 2 ? 0 : BN / 2;
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return half + wn * (WN / 2) + ff * 16;
            }
            return wn * WN + f * 16;
        };
        auto fcol = [&](int f) {      // output column of fragment f's first lane column
            if (GATED) {
                const int ff = f < FN / 2 ? f : f - FN / 2;
                return col0 + wn * (WN / 2) + ff * 16;
            }
            return col0 + wn * WN + f * 16;
        };

        // this wave's valid 16-row fragments are i < nf (rows (wm + 2 i) * 16 ...)
        const int nf = __builtin_amdgcn_readfirstlane(
            nvalid > wm * 16 ? min(FM, (nvalid - wm * 16 + 31) / 32) : 0);

        // the previous tile's reads of both stages must be complete before new loads land
        wait_lgkm0();
        block_barrier();
#pragma unroll
        for (int i = 0; i < LPS; ++i) issue_one(ic<0>{}, i, 0, true);
        if constexpr (LOOK || HALF) {
            // and step 1's weights (nothing read when there is no step 1)
            const bool l1 = __builtin_amdgcn_readfirstlane(nk > 1 ? 1 : 0) != 0;
#pragma unroll
            for (int i = A_ITERS; i < LPS; ++i) issue_one(ic<1>{}, i, 1, l1);
        }

        // The tile for NF valid fragments: no branch inside a step.
        // v_mfma_f32_16x16x32_bf16: lane l feeds row (l % 16) with k-chunk (l / 16)
        // of the 32-wide step for both operands and receives rows 4*(l/16)+e,
        // column l % 16 of the 16x16 result.
        auto tile = [&](auto NFc) {
            constexpr int NF = decltype(NFc)::value;
            floatx4 acc[NF > 0 ? NF : 1][FN];
#pragma unroll
            for (int i = 0; i < NF; ++i)
#pragma unroll
                for (int f = 0; f < FN; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

            // compute stage I while issuing the next stage's LPS loads, one
            // after each fragment's MFMA group (the rest, if there are fewer
            // groups than loads, at the end), so the waves do not all stall at
            // once on a full memory queue
            auto compute = [&](auto I, int knext, bool live) {
                const char* ab = a_base(I);
                const char* bb = b_base(I);
                constexpr auto nextbuf = ic<1 - decltype(I)::value>{};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 bfr[FN];
#pragma unroll
                    for (int f = 0; f < FN; ++f)
                        bfr[f] = *reinterpret_cast<const bf16x8*>(bb + lds_lane[kk] + brow0(f) * ROWB);
                    bf16x8 acur;
                    if (NF > 0) acur = *reinterpret_cast<const bf16x8*>(ab + lds_lane[kk] + wm * 16 * ROWB);
#pragma unroll
                    for (int i = 0; i < NF; ++i) {
                        bf16x8 anext;      // next fragment's rows, read under this one's MFMAs
                        if (i + 1 < NF)
                            anext = *reinterpret_cast<const bf16x8*>(
                                ab + lds_lane[kk] + (wm + WMW * (i + 1)) * 16 * ROWB);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur, bfr[f], acc[i][f], 0, 0, 0);
                        const int slot = kk * NF + i;
                        if (slot < LPS) issue_one(nextbuf, slot, knext, live);
                        if (i + 1 < NF) acur = anext;
                        // keep this order: the loads go out one per fragment, early
                        // in the step, between MFMA groups
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if (2 * NF < LPS) {
#pragma unroll
                    for (int q = 2 * NF; q < LPS; ++q) issue_one(nextbuf, q, knext, live);
                }
            };

            // LOOK: read both k-halves' weight fragments of step k, and once every
            // wave holds them issue, one after each fragment's MFMA group, step
            // k + 1's row loads into the other row buffer and then step k + 2's
            // weight loads into this step's weight buffer (loads past the last
            // step read nothing but count, so every step issues LPS loads)
            auto compute_look = [&](auto I, int k, bool liveA, bool liveB) {
                const char* ab = a_base(I);
                const char* bb = b_base(I);
                constexpr auto nextbuf = ic<1 - decltype(I)::value>{};
                static_assert(2 * FN == 8, "weight fragment reads");
                bf16x8 bfr[2][FN];
                {
                    uint32_t ad[8];
                    uint4 t[8];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int f = 0; f < FN; ++f) ad[kk * FN + f] = lds_addr(bb + lds_lane[kk] + brow0(f) * ROWB);
                    lds_read16x8(t, ad);
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int f = 0; f < FN; ++f) bfr[kk][f] = __builtin_bit_cast(bf16x8, t[kk * FN + f]);
                }
                block_barrier();
                auto issue_slot = [&](int q) {
                    if (q < A_ITERS) issue_one(nextbuf, q, k + 1, liveA);
                    else issue_one(I, q, k + 2, liveB);
                };
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 acur;
                    if (NF > 0) acur = *reinterpret_cast<const bf16x8*>(ab + lds_lane[kk] + wm * 16 * ROWB);
#pragma unroll
                    for (int i = 0; i < NF; ++i) {
                        bf16x8 anext;
                        if (i + 1 < NF)
                            anext = *reinterpret_cast<const bf16x8*>(
                                ab + lds_lane[kk] + (wm + WMW * (i + 1)) * 16 * ROWB);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur, bfr[kk][f], acc[i][f], 0, 0, 0);
                        const int slot = kk * NF + i;
                        if (slot < LPS) issue_slot(slot);
                        if (i + 1 < NF) acur = anext;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if (2 * NF < LPS) {
#pragma unroll
                    for (int q = 2 * NF; q < LPS; ++q) issue_slot(q);
                }
            };

            // HALF: as compute, but the first k-half issues step k + 1's row
            // loads and the second half, once every wave holds its weight
            // fragments, step k + 2's weight loads into this step's buffer
            auto compute_half = [&](auto I, int k, bool liveA, bool liveB) {
                const char* ab = a_base(I);
                const char* bb = b_base(I);
                constexpr auto nextbuf = ic<1 - decltype(I)::value>{};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 bfr[FN];
                    {
                        static_assert(FN == 4, "weight fragment reads");
                        uint32_t ad[4];
                        uint4 t[4];
#pragma unroll
                        for (int f = 0; f < FN; ++f) ad[f] = lds_addr(bb + lds_lane[kk] + brow0(f) * ROWB);
                        lds_read16x4(t, ad);
#pragma unroll
                        for (int f = 0; f < FN; ++f) bfr[f] = __builtin_bit_cast(bf16x8, t[f]);
                    }
                    if (kk == 1) block_barrier();      // every wave holds this step's weight fragments
                    bf16x8 acur;
                    if (NF > 0) acur = *reinterpret_cast<const bf16x8*>(ab + lds_lane[kk] + wm * 16 * ROWB);
#pragma unroll
                    for (int i = 0; i < NF; ++i) {
                        bf16x8 anext;
                        if (i + 1 < NF)
                            anext = *reinterpret_cast<const bf16x8*>(
                                ab + lds_lane[kk] + (wm + WMW * (i + 1)) * 16 * ROWB);
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur, bfr[f], acc[i][f], 0, 0, 0);
                        if (kk == 0 && i < A_ITERS) issue_one(nextbuf, i, k + 1, liveA);
                        if (kk == 1 && i < B_ITERS) issue_one(I, A_ITERS + i, k + 2, liveB);
                        if (i + 1 < NF) acur = anext;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (kk == 0 && NF < A_ITERS) {
#pragma unroll
                        for (int q = NF; q < A_ITERS; ++q) issue_one(nextbuf, q, k + 1, liveA);
                    }
                    if (kk == 1 && NF < B_ITERS) {
#pragma unroll
                        for (int q = NF; q < B_ITERS; ++q) issue_one(I, A_ITERS + q, k + 2, liveB);
                    }
                }
            };

            // step k: wait for stage k (nothing else is in flight; LOOK: step
            // k + 1's weights stay in flight), then compute k while stage k + 1
            // is loaded into the other buffer
            auto step = [&](auto I, int k) {
                if constexpr (LOOK || HALF) wait_vmcnt<B_ITERS>();
                else wait_vmcnt<0>();
                wait_lgkm0();
                block_barrier();
                // wave-uniform by construction; say so, so that the resource
                // select below stays scalar
                const bool live = __builtin_amdgcn_readfirstlane(k + 1 < nk ? 1 : 0) != 0;
                if constexpr (LOOK) {
                    const bool live2 = __builtin_amdgcn_readfirstlane(k + 2 < nk ? 1 : 0) != 0;
                    compute_look(I, k, live, live2);
                } else if constexpr (HALF) {
                    const bool live2 = __builtin_amdgcn_readfirstlane(k + 2 < nk ? 1 : 0) != 0;
                    compute_half(I, k, live, live2);
                } else {
                    compute(I, k + 1, live);
                }
            };
            for (int k = 0; k < nk; k += 2) {
                step(ic<0>{}, k);
                if (k + 1 < nk) step(ic<1>{}, k + 1);
            }
            // the loads issued by the last step read nothing but still count
            wait_vmcnt<0>();

            // ---- epilogue: every wave stages its bf16 outputs in a private LDS
            // region (both stages are free once every wave is past the k-loop)
            // and stores whole 16-byte row chunks: 8 per 128-byte output row
            // piece instead of one 2-byte store per element.  PF fragments
            // per pass; staged rows are padded by 16 bytes so that the four
            // row groups of one LDS write fall into different banks.
            constexpr int FO = GATED ? FN / 2 : FN;
            constexpr int OCOLS = FO * 16;                  // output columns of a wave
            constexpr int OCH = OCOLS * 2 / 16;             // 16-byte chunks per staged row
            constexpr int OPITCH = OCOLS * 2 + 16;          // staged row pitch (bytes)
            constexpr int PF = 5;                           // fragments per pass
            constexpr int RSZ = PF * 16 * OPITCH;           // bytes of a wave's region
            static_assert(2 * RSZ <= BN * ROWB && 2 * RSZ <= BM * ROWB, "two regions per stage buffer");
            wait_lgkm0();
            block_barrier();
            char* region = (wave < 2 ? reinterpret_cast<char*>(sa0) : wave < 4 ? reinterpret_cast<char*>(sb0)
                            : wave < 6 ? reinterpret_cast<char*>(sa1) : reinterpret_cast<char*>(sb1)) + (wave & 1) * RSZ;
            const int colbase = fcol(0);                    // the wave's first output column
            char* out_bytes = reinterpret_cast<char*>(Out);
#pragma unroll
            for (int p0 = 0; p0 < NF; p0 += PF) {
#pragma unroll
                for (int ii = 0; ii < PF; ++ii) {
                    const int i = p0 + ii;
                    if (i < NF) {
#pragma unroll
                        for (int f = 0; f < FO; ++f)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float val = GATED ? silu(acc[i][f][e]) * acc[i][f + FN / 2][e] : acc[i][f][e];
                                const int lrow = ii * 16 + (lane >> 4) * 4 + e;
                                *reinterpret_cast<uint16_t*>(region + lrow * OPITCH + (f * 16 + (lane & 15)) * 2) =
                                    (uint16_t)f32_to_bf16_bits(val);
                            }
                    }
                }
                constexpr int RPI = 64 / OCH;               // staged rows per 64-lane read
#pragma unroll
                for (int q = 0; q < PF * 16 / RPI; ++q) {
                    const int lrow = q * RPI + lane / OCH, ch = lane % OCH;
                    const int i = p0 + lrow / 16;
                    const int trow = (wm + WMW * i) * 16 + lrow % 16;   // row within the tile
                    const int col = colbase + ch * 8;
                    if (i < NF && trow < nvalid && col < N) {
                        const uint4 v = *reinterpret_cast<const uint4*>(region + lrow * OPITCH + ch * 16);
                        *reinterpret_cast<uint4*>(out_bytes + ((size_t)(row0 + trow) * N + col) * 2) = v;
                    }
                }
            }
        };
        // a switch, not a chain of ifs: with the chain the compiler no longer
        // treated the tile's scalars as uniform and wrapped every buffer load
        // in a readfirstlane loop
        static_assert(FM <= 10, "one case per fragment count");
        switch (nf) {
            case 0: if constexpr (0 <= FM) tile(ic<0>{}); break;
            case 1: if constexpr (1 <= FM) tile(ic<1>{}); break;
            case 2: if constexpr (2 <= FM) tile(ic<2>{}); break;
            case 3: if constexpr (3 <= FM) tile(ic<3>{}); break;
            case 4: if constexpr (4 <= FM) tile(ic<4>{}); break;
            case 5: if constexpr (5 <= FM) tile(ic<5>{}); break;
            case 6: if constexpr (6 <= FM) tile(ic<6>{}); break;
            case 7: if constexpr (7 <= FM) tile(ic<7>{}); break;
            case 8: if constexpr (8 <= FM) tile(ic<8>{}); break;
            case 9: if constexpr (9 <= FM) tile(ic<9>{}); break;
            case 10: if constexpr (10 <= FM) tile(ic<10>{}); break;
            default: break;
        }
    }
}

}  // namespace wide
}  // namespace moeep
