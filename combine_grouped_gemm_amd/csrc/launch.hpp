// Internal launchers behind the C ABI.  Arguments have been validated by the
// caller (api.hip); each launcher only enqueues kernels on `stream` and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeep {

// route.hip (map: optional (E) device table logical -> physical expert id; n_shared
// always-on slots appended to each output row, ids E.., gate 1)
hipError_t launch_route(const float* logits, int B, int E, int K, int32_t* ids, float* w,
                        const int32_t* map, int n_shared, hipStream_t stream);

// placement.hip (host): balanced equal-size expert groups, see the file header
bool place_experts(const int64_t* load, int E, int G, int32_t* phys_of_logical);

// layout.hip
size_t layout_workspace_bytes(int B, int K, int E);
// moe_layout_noalloc: the layout workspace held by the library, one
// kLayoutScratchBytes array per GPU; layout_scratch_ptr gives the current
// GPU's copy (its device address, looked up once per GPU and cached)
constexpr size_t kLayoutScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
hipError_t layout_scratch_ptr(void** out);
hipError_t launch_layout(const int32_t* ids, int B, int K, int E, int e_begin, int e_end,
                         int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                         int cap, void* ws, hipStream_t stream);
// fixed-capacity variant: local expert j owns rows [j*cap_e, (j+1)*cap_e); m (E_loc) gets
// min(count, cap_e)
hipError_t launch_layout_masked(const int32_t* ids, int B, int K, int E, int e_begin, int e_end,
                                int32_t* counts, int32_t* m, int32_t* row_of, int32_t* src_of,
                                int cap_e, void* ws, hipStream_t stream);

// dispatch.hip
constexpr int kMaxSeg = 64;
struct SegTable {
    const void* ptr[kMaxSeg];
    int start[kMaxSeg + 1];   // prefix sums of segment rows
    int n;
};
// kind: 0 = f32 copy, 1 = bf16 copy, 2 = bf16 -> fp8 quantise
hipError_t launch_dispatch(const SegTable& seg, int B, int H, int kind, const int32_t* row_of,
                           int K, void* xd, float* xd_scales, int cap, hipStream_t stream);

// combine.hip
// kind: 0 = f32 -> f32, 1 = bf16 -> bf16, 2 = bf16 -> f32
hipError_t launch_combine(const void* y, int kind, const int32_t* row_of, const float* w,
                          int B, int K, int H, void* out, int cap, hipStream_t stream);

// ffn kernels: shared argument block
struct FfnArgs {
    const void* a;            // activations (cap, Kdim)
    const float* a_scales;    // fp8 only: (cap, ceil(Kdim/128))
    const int32_t* offsets;   // contiguous layout: (E_loc + 1); nullptr for the masked layout
    const int32_t* m_counts;  // masked layout: (E_loc) valid rows of expert j, in [j*cap_e, ...)
    int cap_e;                // masked layout: rows per expert block (cap = E_loc * cap_e)
    int E_loc, cap, Kdim, N;  // N = output columns (I for gate/up, H for down)
    int ldw;                  // weight row pitch in elements (Kdim, or the packed pitch)
    const void* w0;           // gate or down (E_loc, N, ldw): rows of Kdim at pitch ldw
    const void* w1;           // up (gate/up only)
    const float* w0_scales;   // fp8 only: (E_loc, N, ceil(Kdim/128))
    const float* w1_scales;
    void* out;                // (cap, N)
    float* out_scales;        // fp8 h only: (cap, ceil(N/128))
    int rows_hint;            // cap / E_loc, picks the tile shape
    bool w_scales_pow2;       // fp8: every weight scale is a power of two
};

hipError_t launch_ffn_f32(const FfnArgs& a, bool gated, hipStream_t stream);   // ffn_f32.hip
hipError_t launch_ffn_bf16(const FfnArgs& a, bool gated, hipStream_t stream);  // ffn_bf16.hip
hipError_t launch_ffn_fp8(const FfnArgs& a, bool gated, hipStream_t stream);   // ffn_fp8.hip

int device_cu_count();   // api.hip: compute units of the current device (cached)

// pack.hip: rows of row_bytes bytes (a multiple of 4) copied to a pitch of
// ld_bytes (a multiple of 128, >= row_bytes), the padding zeroed
hipError_t launch_pack_rows(const void* src, long long n_rows, int row_bytes, int ld_bytes, void* dst,
                            hipStream_t stream);

}  // namespace moeep
