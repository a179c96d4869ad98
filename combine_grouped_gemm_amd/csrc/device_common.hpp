// Device helpers shared by the libmoeep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeep {

constexpr int kWave = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Streaming 16-byte loads: the non-temporal hint keeps data read once
// (weights streamed by a decode GEMM, expert outputs gathered by combine)
// from displacing reusable lines in L2 and the MALL.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even; NaN stays NaN, overflow becomes inf.
// f32 -> bf16, round to nearest even, by gfx950's packed conversion
// (v_cvt_pk_bf16_f32; bit-identical to the integer RNE
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 on every finite input, checked on the
// GPU across all exponents, denormals, ties and the overflow boundary).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t b = __builtin_convertvector(float2_t{lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// ---------------------------------------------------------------------------
// OCP fp8 e4m3fn: encode with round-to-nearest-even after saturating the
// magnitude to 448 (the largest finite code).  Subnormal quantum is 2^-9.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
    uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    float a = fabsf(v);
    if (!(a <= 448.0f)) a = 448.0f;
    uint32_t au = __float_as_uint(a);
    if (au < 0x3c800000u) {                       // a < 2^-6: subnormal codes 0..8
        return sign | (uint32_t)rintf(a * 512.0f);
    }
    uint32_t r = (au + 0x7ffffu + ((au >> 20) & 1u)) >> 20;   // keep 3 fraction bits
    return sign | (r - (120u << 3));              // rebias exponent 127 -> 7
}

// Activation block scale: the smallest power of two s = 2^e with
// amax <= 448 * s and e >= -127 (an E8M0 scale byte's range); 1 for amax = 0.
// With amax = m * 2^E, m in [0.5, 1) and 448 = 0.875 * 2^9: e = E - 9 when
// m <= 0.875 (fraction bits <= 0x600000 in [1, 2) form), else E - 8.  Any
// subnormal amax gets 2^-127.  The matrix cores apply such a scale exactly.
__device__ __forceinline__ float pow2_block_scale(float amax) {
    if (amax == 0.0f) return 1.0f;
    const uint32_t u = __float_as_uint(amax);
    if (u < 0x00800000u) return __uint_as_float(0x00400000u);     // 2^-127
    const int E = (int)((u >> 23) & 0xffu) - 126;
    int e = (u & 0x7fffffu) <= 0x600000u ? E - 9 : E - 8;
    if (e < -127) e = -127;
    return e == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(e + 127) << 23);
}

// E8M0 byte of a power-of-two scale from pow2_block_scale: its biased exponent.
__device__ __forceinline__ int e8m0_of_pow2(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }

// 1 / s for s = 2^e, e in [-127, 127], exactly: the bits of 2^-e are
// (127 - e) << 23 = 0x7f000000 - bits(s) for e in [-126, 126]; 2^-127 (the one
// subnormal) and 2^127 are each other's reciprocal.
__device__ __forceinline__ float pow2_recip(float s) {
    const uint32_t u = __float_as_uint(s);
    if (u < 0x00800000u) return __uint_as_float(0x7f000000u);
    if (u >= 0x7f000000u) return __uint_as_float(0x00400000u);
    return __uint_as_float(0x7f000000u - u);
}

// Two values with |v| <= 448 to OCP e4m3 codes (round to nearest even) by
// the hardware conversion, first value in bits 7:0, second in bits 15:8.
// Identical to f32_to_e4m3_sat on that range (checked exhaustively at every
// code, rounding tie and its neighbours on gfx950).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Maximum over the 16 lanes of a DPP row (lanes 16k .. 16k + 15), returned in
// every lane of the row, by cross-lane moves inside the VALU: quad permutes
// [1,0,3,2] and [2,3,0,1] (partners lane ^ 1 and lane ^ 2), then the half-row
// mirror (lane i <-> 7 - i: joins the two quads of each half) and the row
// mirror (lane i <-> 15 - i: joins the two halves).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Mask of the lanes whose `key` equals this lane's, among lanes in `active`.
// `nbits` bits of the key are compared (keys must be < 2^nbits).
__device__ __forceinline__ uint64_t match_mask(uint32_t key, uint64_t active, int nbits) {
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        bool bit = (key >> b) & 1u;
        uint64_t bal = ballot64(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// silu(z) = z / (1 + e^-z), with the hardware exponential and reciprocal
// (about 1 ulp each; the result is rounded to bf16 or fp8 afterwards).
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

}  // namespace moeep
