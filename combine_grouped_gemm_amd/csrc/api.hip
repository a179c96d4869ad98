// C ABI of libmoeep: host-side argument checks, then kernel launches on the
// caller's stream.  Nothing here allocates, synchronises or copies from the
// device; a failed check returns before anything is enqueued.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.hpp"
#include "moeep.h"

static_assert(MOE_LAYOUT_NOALLOC_SCRATCH_BYTES == moeep::kLayoutScratchBytes,
              "the header states the library's layout scratch size");

namespace moeep {

int device_cu_count() {
    static thread_local int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

}  // namespace moeep

namespace {

thread_local char g_last_error[512] = "";

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

moe_status_t launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    g_last_error[0] = '\0';
    return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                                        \
    do {                                                          \
        if (!(cond)) return fail(MOE_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

moe_status_t check_route_shape(int B, int E, int K) {
    REQUIRE(B >= 0, "B must be >= 0 (got %d)", B);
    REQUIRE(E >= 1 && E <= 1024, "E must be in [1, 1024] (got %d)", E);
    REQUIRE(K >= 1 && K <= E, "K must be in [1, E] (got K=%d, E=%d)", K, E);
    REQUIRE((long long)B * K <= 0x7fffffffLL && (long long)B * E <= 0x7fffffffLL,
            "B*K and B*E must fit in int32");
    return MOE_OK;
}

// Where the rows of each local expert are: the contiguous layout's offsets
// (E_local + 1), or the masked layout's valid-row counts m (E_local) with
// fixed blocks of cap_e rows.
struct Rows {
    const int32_t* offsets;
    const int32_t* m;
    int cap_e;
};

moe_status_t check_ffn_common(const void* a, Rows rows, int E_local, int cap_rows,
                              int H, int I, moe_dtype_t act_dt, moe_dtype_t w_dt) {
    REQUIRE(a && (rows.offsets || rows.m), "null activation or row-count pointer");
    REQUIRE(E_local >= 1 && E_local <= 1024, "E_local must be in [1, 1024] (got %d)", E_local);
    REQUIRE(cap_rows >= 0, "cap_rows must be >= 0");
    // rows move in 16-byte pieces: 8 elements (bf16, fp32), 16 for fp8
    const int q = act_dt == MOE_FP8_E4M3 ? 16 : 8;
    REQUIRE(H >= q && H % q == 0 && I >= q && I % q == 0,
            "H and I must be positive multiples of %d for this dtype (got H=%d, I=%d)", q, H, I);
    REQUIRE((long long)cap_rows * (H > I ? H : I) <= 0x7fffffffLL * 4LL, "cap_rows * H too large");
    REQUIRE(aligned16(a), "activation pointer must be 16-byte aligned");
    const bool ok = (act_dt == MOE_F32 && w_dt == MOE_F32) || (act_dt == MOE_BF16 && w_dt == MOE_BF16) ||
                    (act_dt == MOE_FP8_E4M3 && (w_dt == MOE_FP8_E4M3 || w_dt == MOE_FP8_E4M3_PO2));
    if (!ok) return fail(MOE_ERR_UNSUPPORTED, "unsupported (act_dt, w_dt) = (%d, %d)", act_dt, w_dt);
    return MOE_OK;
}

moe_status_t check_y_dtype(moe_dtype_t act_dt, moe_dtype_t y_dt) {
    const bool ok = (act_dt == MOE_F32 && y_dt == MOE_F32) || (act_dt == MOE_BF16 && y_dt == MOE_BF16) ||
                    (act_dt == MOE_FP8_E4M3 && y_dt == MOE_BF16);
    if (!ok) return fail(MOE_ERR_UNSUPPORTED, "unsupported (act_dt, y_dt) = (%d, %d)", act_dt, y_dt);
    return MOE_OK;
}

moeep::FfnArgs ffn_args(const void* a, const float* a_scales, Rows rows, int E_local,
                        int cap_rows, int Kdim, int N, const void* w0, const void* w1,
                        const float* w0s, const float* w1s, void* out, float* out_scales,
                        int expected_rows, moe_dtype_t w_dt, int ldw) {
    moeep::FfnArgs f;
    f.w_scales_pow2 = w_dt == MOE_FP8_E4M3_PO2;
    f.ldw = ldw;
    f.a = a;
    f.a_scales = a_scales;
    f.offsets = rows.offsets;
    f.m_counts = rows.m;
    f.cap_e = rows.cap_e;
    f.E_loc = E_local;
    f.cap = cap_rows;
    f.Kdim = Kdim;
    f.N = N;
    f.w0 = w0;
    f.w1 = w1;
    f.w0_scales = w0s;
    f.w1_scales = w1s;
    f.out = out;
    f.out_scales = out_scales;
    f.rows_hint = expected_rows > 0 ? expected_rows : cap_rows / E_local;
    return f;
}

hipError_t run_ffn(const moeep::FfnArgs& f, moe_dtype_t act_dt, bool gated, hipStream_t stream) {
    if (f.cap == 0) return hipSuccess;
    switch (act_dt) {
        case MOE_F32: return moeep::launch_ffn_f32(f, gated, stream);
        case MOE_BF16: return moeep::launch_ffn_bf16(f, gated, stream);
        default: return moeep::launch_ffn_fp8(f, gated, stream);
    }
}

size_t elem_size(moe_dtype_t d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

// Row pitch (elements) of packed weights: whole 128-byte lines, plus one line
// when the row length is a multiple of 4 KiB (rows exactly 4 KiB apart
// stream markedly slower than rows one line further apart).
int packed_ld(int cols, size_t esz) {
    size_t bytes = ((size_t)cols * esz + 127) / 128 * 128;
    if (bytes % 4096 == 0) bytes += 128;
    return (int)(bytes / esz);
}

// a weight dtype argument: the element type, and whether the rows sit at the packed pitch
struct WType {
    moe_dtype_t dt;
    bool packed;
};
WType split_w(moe_dtype_t w_dt) { return WType{w_dt & ~MOE_W_PACKED, (w_dt & MOE_W_PACKED) != 0}; }
int weight_ld(WType wt, int cols) { return wt.packed ? packed_ld(cols, elem_size(wt.dt)) : cols; }

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

size_t ffn_workspace_bytes(int cap_rows, int I, moe_dtype_t act_dt) {
    if (cap_rows < 0 || I < 1) return 0;
    size_t bytes = round256((size_t)cap_rows * I * elem_size(act_dt));
    if (act_dt == MOE_FP8_E4M3) bytes += round256((size_t)cap_rows * (((size_t)I + 127) / 128) * sizeof(float));
    return bytes;
}

moe_status_t ffn_gate_up(const void* xd, const float* xd_scales, Rows rows,
                             int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                             const void* w_gate, const void* w_up, const float* w_gate_scales,
                             const float* w_up_scales, moe_dtype_t w_dt, void* h, float* h_scales,
                             int expected_rows, hipStream_t stream) {
    const WType wt = split_w(w_dt);
    moe_status_t s = check_ffn_common(xd, rows, E_local, cap_rows, H, I, act_dt, wt.dt);
    if (s != MOE_OK) return s;
    REQUIRE(w_gate && w_up && h, "null weight or h pointer");
    REQUIRE(aligned16(w_gate) && aligned16(w_up) && aligned16(h), "weights and h must be 16-byte aligned");
    if (act_dt == MOE_FP8_E4M3)
        REQUIRE(xd_scales && w_gate_scales && w_up_scales && h_scales, "fp8 needs all scale pointers");
    auto f = ffn_args(xd, xd_scales, rows, E_local, cap_rows, H, I, w_gate, w_up, w_gate_scales,
                      w_up_scales, h, h_scales, expected_rows, wt.dt, weight_ld(wt, H));
    return launched(run_ffn(f, act_dt, true, stream), "ffn gate/up");
}

moe_status_t ffn_down(const void* h, const float* h_scales, Rows rows, int E_local,
                          int cap_rows, int H, int I, moe_dtype_t act_dt, const void* w_down,
                          const float* w_down_scales, moe_dtype_t w_dt, void* y, moe_dtype_t y_dt,
                          int expected_rows, hipStream_t stream) {
    const WType wt = split_w(w_dt);
    moe_status_t s = check_ffn_common(h, rows, E_local, cap_rows, H, I, act_dt, wt.dt);
    if (s != MOE_OK) return s;
    s = check_y_dtype(act_dt, y_dt);
    if (s != MOE_OK) return s;
    REQUIRE(w_down && y, "null weight or y pointer");
    REQUIRE(aligned16(w_down) && aligned16(y), "weights and y must be 16-byte aligned");
    if (act_dt == MOE_FP8_E4M3) REQUIRE(h_scales && w_down_scales, "fp8 needs all scale pointers");
    auto f = ffn_args(h, h_scales, rows, E_local, cap_rows, I, H, w_down, nullptr, w_down_scales,
                      nullptr, y, nullptr, expected_rows, wt.dt, weight_ld(wt, I));
    return launched(run_ffn(f, act_dt, false, stream), "ffn down");
}

moe_status_t grouped_ffn(const void* xd, const float* xd_scales, Rows rows,
                             int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const float* w_gate_scales, const float* w_up_scales,
                             const float* w_down_scales, moe_dtype_t w_dt, void* y, moe_dtype_t y_dt,
                             void* ws, size_t ws_bytes, int expected_rows, hipStream_t stream) {
    moe_status_t s = check_ffn_common(xd, rows, E_local, cap_rows, H, I, act_dt, split_w(w_dt).dt);
    if (s != MOE_OK) return s;
    s = check_y_dtype(act_dt, y_dt);
    if (s != MOE_OK) return s;
    REQUIRE(ws, "null workspace");
    REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, "workspace must be 256-byte aligned");
    const size_t need = ffn_workspace_bytes(cap_rows, I, act_dt);
    REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    void* h = ws;
    float* h_scales = nullptr;
    if (act_dt == MOE_FP8_E4M3)
        h_scales = reinterpret_cast<float*>(static_cast<char*>(ws) + round256((size_t)cap_rows * I));
    s = ffn_gate_up(xd, xd_scales, rows, E_local, cap_rows, H, I, act_dt, w_gate, w_up,
                        w_gate_scales, w_up_scales, w_dt, h, h_scales, expected_rows, stream);
    if (s != MOE_OK) return s;
    return ffn_down(h, h_scales, rows, E_local, cap_rows, H, I, act_dt, w_down, w_down_scales,
                        w_dt, y, y_dt, expected_rows, stream);
}


}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_last_error; }

const char* moe_version(void) { return "libmoeep 0.1 (gfx950)"; }

moe_status_t moe_route(const float* logits, int B, int E, int K, int32_t* topk_ids, float* topk_w,
                       hipStream_t stream) {
    moe_status_t s = check_route_shape(B, E, K);
    if (s != MOE_OK) return s;
    if (B > 0) REQUIRE(logits && topk_ids && topk_w, "null pointer argument");
    return launched(moeep::launch_route(logits, B, E, K, topk_ids, topk_w, nullptr, 0, stream), "moe_route");
}

moe_status_t moe_route_mapped(const float* logits, int B, int E, int K, const int32_t* phys_of_logical,
                              int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    moe_status_t s = check_route_shape(B, E, K);
    if (s != MOE_OK) return s;
    REQUIRE(phys_of_logical, "null phys_of_logical");
    if (B > 0) REQUIRE(logits && topk_ids && topk_w, "null pointer argument");
    return launched(moeep::launch_route(logits, B, E, K, topk_ids, topk_w, phys_of_logical, 0, stream),
                    "moe_route_mapped");
}

moe_status_t moe_route_shared(const float* logits, int B, int E, int K, int n_shared, int32_t* ids,
                              float* w, hipStream_t stream) {
    moe_status_t s = check_route_shape(B, E, K);
    if (s != MOE_OK) return s;
    REQUIRE(n_shared >= 0 && E + n_shared <= 1024, "need 0 <= n_shared and E + n_shared <= 1024");
    REQUIRE((long long)B * (K + n_shared) <= 0x7fffffffLL, "B*(K+n_shared) must fit in int32");
    if (B > 0) REQUIRE(logits && ids && w, "null pointer argument");
    return launched(moeep::launch_route(logits, B, E, K, ids, w, nullptr, n_shared, stream),
                    "moe_route_shared");
}

moe_status_t moe_eplb_place(const int64_t* load, int E, int n_groups, int32_t* phys_of_logical) {
    REQUIRE(E >= 1 && E <= 1024, "E must be in [1, 1024] (got %d)", E);
    REQUIRE(n_groups >= 1 && E % n_groups == 0, "n_groups must divide E (got E=%d, n_groups=%d)", E,
            n_groups);
    REQUIRE(load && phys_of_logical, "null load or phys_of_logical");
    int64_t total = 0;     // group totals and their differences stay within it
    for (int e = 0; e < E; ++e) {
        REQUIRE(load[e] >= 0, "load[%d] < 0", e);
        REQUIRE(load[e] <= INT64_MAX - total, "the loads' total must fit in int64");
        total += load[e];
    }
    moeep::place_experts(load, E, n_groups, phys_of_logical);
    g_last_error[0] = '\0';
    return MOE_OK;
}

size_t moe_layout_workspace_bytes(int B, int K, int E) {
    // 0 for sizes moe_layout rejects (B * K past int32 included)
    if (B < 0 || K < 1 || E < 1 || (long long)B * K > 0x7fffffffLL) return 0;
    return moeep::layout_workspace_bytes(B, K, E);
}

moe_status_t moe_layout(const int32_t* topk_ids, int B, int K, int E, int e_begin, int e_end,
                        int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                        int cap_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
    moe_status_t s = check_route_shape(B, E, K);
    if (s != MOE_OK) return s;
    REQUIRE(e_begin >= 0 && e_begin < e_end && e_end <= E,
            "need 0 <= e_begin < e_end <= E (got %d, %d, E=%d)", e_begin, e_end, E);
    REQUIRE(cap_rows >= 0, "cap_rows must be >= 0");
    REQUIRE(counts && offsets && ws, "null counts, offsets or workspace");
    if (B > 0) REQUIRE(topk_ids && row_of, "null topk_ids or row_of");
    if (cap_rows > 0) REQUIRE(src_of, "null src_of");
    REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, "workspace must be 256-byte aligned");
    REQUIRE(ws_bytes >= moeep::layout_workspace_bytes(B, K, E),
            "workspace too small: %zu < %zu bytes", ws_bytes, moeep::layout_workspace_bytes(B, K, E));
    return launched(moeep::launch_layout(topk_ids, B, K, E, e_begin, e_end, counts, offsets, row_of,
                                         src_of, cap_rows, ws, stream),
                    "moe_layout");
}

moe_status_t moe_layout_noalloc(const int32_t* topk_ids, int B, int K, int E, int e_begin, int e_end,
                                int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                int cap_rows, hipStream_t stream) {
    moe_status_t s = check_route_shape(B, E, K);
    if (s != MOE_OK) return s;
    REQUIRE(e_begin >= 0 && e_begin < e_end && e_end <= E,
            "need 0 <= e_begin < e_end <= E (got %d, %d, E=%d)", e_begin, e_end, E);
    REQUIRE(cap_rows >= 0, "cap_rows must be >= 0");
    REQUIRE(counts && offsets, "null counts or offsets");
    if (B > 0) REQUIRE(topk_ids && row_of, "null topk_ids or row_of");
    if (cap_rows > 0) REQUIRE(src_of, "null src_of");
    const size_t need = moeep::layout_workspace_bytes(B, K, E);
    REQUIRE(need <= moeep::kLayoutScratchBytes,
            "moe_layout_noalloc: B=%d, K=%d, E=%d needs %zu bytes of layout workspace, more than the "
            "library's %zu (use moe_layout with a caller workspace)",
            B, K, E, need, moeep::kLayoutScratchBytes);
    void* ws = nullptr;
    const hipError_t e = moeep::layout_scratch_ptr(&ws);
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "moe_layout_noalloc: no device address for the layout scratch: %s",
                    hipGetErrorString(e));
    return launched(moeep::launch_layout(topk_ids, B, K, E, e_begin, e_end, counts, offsets, row_of,
                                         src_of, cap_rows, ws, stream),
                    "moe_layout_noalloc");
}

moe_status_t moe_layout_masked(const int32_t* topk_ids, int B, int K, int E, int e_begin, int e_end,
                               int32_t* counts, int32_t* m, int32_t* row_of, int32_t* src_of,
                               int cap_per_expert, void* ws, size_t ws_bytes, hipStream_t stream) {
    moe_status_t s = check_route_shape(B, E, K);
    if (s != MOE_OK) return s;
    REQUIRE(e_begin >= 0 && e_begin < e_end && e_end <= E,
            "need 0 <= e_begin < e_end <= E (got %d, %d, E=%d)", e_begin, e_end, E);
    REQUIRE(cap_per_expert >= 1, "cap_per_expert must be >= 1 (got %d)", cap_per_expert);
    REQUIRE((long long)(e_end - e_begin) * cap_per_expert <= 0x7fffffffLL,
            "E_local * cap_per_expert must fit in int32");
    REQUIRE(counts && m && src_of && ws, "null counts, m, src_of or workspace");
    if (B > 0) REQUIRE(topk_ids && row_of, "null topk_ids or row_of");
    REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, "workspace must be 256-byte aligned");
    REQUIRE(ws_bytes >= moeep::layout_workspace_bytes(B, K, E),
            "workspace too small: %zu < %zu bytes", ws_bytes, moeep::layout_workspace_bytes(B, K, E));
    return launched(moeep::launch_layout_masked(topk_ids, B, K, E, e_begin, e_end, counts, m, row_of,
                                                src_of, cap_per_expert, ws, stream),
                    "moe_layout_masked");
}

moe_status_t moe_dispatch(const void* const* seg_x, const int32_t* seg_rows, int n_seg,
                          moe_dtype_t x_dt, int H, const int32_t* row_of, int K, void* xd,
                          moe_dtype_t xd_dt, float* xd_scales, int cap_rows, hipStream_t stream) {
    REQUIRE(n_seg >= 1 && n_seg <= MOE_MAX_SEGMENTS, "n_seg must be in [1, %d]", MOE_MAX_SEGMENTS);
    REQUIRE(seg_x && seg_rows, "null segment tables");
    REQUIRE(K >= 1 && K <= 1024, "K must be in [1, 1024]");
    // 16-byte pieces: 8 elements; fp8 rows feed the fp8 GEMMs, which need 16
    const int q = xd_dt == MOE_FP8_E4M3 ? 16 : 8;
    REQUIRE(H >= q && H % q == 0, "H must be a positive multiple of %d for this dtype (got %d)", q, H);
    REQUIRE(cap_rows >= 0, "cap_rows must be >= 0");
    int kind;
    if (x_dt == MOE_F32 && xd_dt == MOE_F32) kind = 0;
    else if (x_dt == MOE_BF16 && xd_dt == MOE_BF16) kind = 1;
    else if (x_dt == MOE_BF16 && xd_dt == MOE_FP8_E4M3) kind = 2;
    else return fail(MOE_ERR_UNSUPPORTED, "unsupported dispatch (x_dt, xd_dt) = (%d, %d)", x_dt, xd_dt);
    moeep::SegTable seg;
    seg.n = n_seg;
    seg.start[0] = 0;
    long long B = 0;
    for (int i = 0; i < n_seg; ++i) {
        REQUIRE(seg_rows[i] >= 0, "seg_rows[%d] < 0", i);
        if (seg_rows[i] > 0) {
            REQUIRE(seg_x[i] != nullptr, "seg_x[%d] is null", i);
            REQUIRE(aligned16(seg_x[i]), "seg_x[%d] must be 16-byte aligned", i);
        }
        seg.ptr[i] = seg_x[i];
        B += seg_rows[i];
        REQUIRE(B * K <= 0x7fffffffLL, "total tokens * K must fit in int32");
        seg.start[i + 1] = (int)B;
    }
    if (B > 0) {
        REQUIRE(row_of && xd, "null row_of or xd");
        REQUIRE(aligned16(xd), "xd must be 16-byte aligned");
        if (kind == 2) REQUIRE(xd_scales, "fp8 dispatch needs xd_scales");
    }
    return launched(moeep::launch_dispatch(seg, (int)B, H, kind, row_of, K, xd, xd_scales, cap_rows, stream),
                    "moe_dispatch");
}

size_t moe_ffn_workspace_bytes(int cap_rows, int I, moe_dtype_t act_dt) {
    return ffn_workspace_bytes(cap_rows, I, act_dt);
}

static bool packable_dtype(moe_dtype_t w_dt) {
    return w_dt == MOE_F32 || w_dt == MOE_BF16 || w_dt == MOE_FP8_E4M3 || w_dt == MOE_FP8_E4M3_PO2;
}

int moe_weight_ld(int cols, moe_dtype_t w_dt) {
    if (cols < 1 || cols > (1 << 24) || !packable_dtype(w_dt & ~MOE_W_PACKED)) return -1;
    return packed_ld(cols, elem_size(w_dt & ~MOE_W_PACKED));
}

size_t moe_packed_weight_bytes(int E_local, int rows, int cols, moe_dtype_t w_dt) {
    const int ld = moe_weight_ld(cols, w_dt);
    if (ld < 0 || E_local < 0 || rows < 0) return 0;
    return (size_t)E_local * (size_t)rows * (size_t)ld * elem_size(w_dt & ~MOE_W_PACKED);
}

moe_status_t moe_pack_weights(const void* w, int E_local, int rows, int cols, moe_dtype_t w_dt,
                              void* w_packed, hipStream_t stream) {
    const moe_dtype_t dt = w_dt & ~MOE_W_PACKED;
    if (!packable_dtype(dt)) return fail(MOE_ERR_UNSUPPORTED, "unsupported weight dtype %d", w_dt);
    REQUIRE(E_local >= 0 && rows >= 0, "E_local and rows must be >= 0");
    REQUIRE(cols >= 8 && cols % 8 == 0 && cols <= (1 << 24), "cols must be a positive multiple of 8 (got %d)", cols);
    if ((long long)E_local * rows == 0) {
        g_last_error[0] = '\0';
        return MOE_OK;
    }
    REQUIRE(w && w_packed, "null weight pointer");
    REQUIRE(aligned16(w) && aligned16(w_packed), "weights must be 16-byte aligned");
    const size_t esz = elem_size(dt);
    const size_t row_bytes = (size_t)cols * esz, ld_bytes = (size_t)packed_ld(cols, esz) * esz;
    const long long n_rows = (long long)E_local * rows;
    const char* s0 = static_cast<const char*>(w);
    const char* d0 = static_cast<const char*>(w_packed);
    REQUIRE(d0 + (size_t)n_rows * ld_bytes <= s0 || s0 + (size_t)n_rows * row_bytes <= d0,
            "w and w_packed must not overlap");
    return launched(moeep::launch_pack_rows(w, n_rows, (int)row_bytes, (int)ld_bytes, w_packed, stream),
                    "moe_pack_weights");
}

moe_status_t moe_ffn_gate_up(const void* xd, const float* xd_scales, const int32_t* offsets,
                             int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                             const void* w_gate, const void* w_up, const float* w_gate_scales,
                             const float* w_up_scales, moe_dtype_t w_dt, void* h, float* h_scales,
                             int expected_rows, hipStream_t stream) {
    return ffn_gate_up(xd, xd_scales, Rows{offsets, nullptr, 0}, E_local, cap_rows, H, I, act_dt,
                       w_gate, w_up, w_gate_scales, w_up_scales, w_dt, h, h_scales, expected_rows,
                       stream);
}

moe_status_t moe_ffn_down(const void* h, const float* h_scales, const int32_t* offsets, int E_local,
                          int cap_rows, int H, int I, moe_dtype_t act_dt, const void* w_down,
                          const float* w_down_scales, moe_dtype_t w_dt, void* y, moe_dtype_t y_dt,
                          int expected_rows, hipStream_t stream) {
    return ffn_down(h, h_scales, Rows{offsets, nullptr, 0}, E_local, cap_rows, H, I, act_dt, w_down,
                    w_down_scales, w_dt, y, y_dt, expected_rows, stream);
}

moe_status_t moe_grouped_ffn(const void* xd, const float* xd_scales, const int32_t* offsets,
                             int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const float* w_gate_scales, const float* w_up_scales,
                             const float* w_down_scales, moe_dtype_t w_dt, void* y, moe_dtype_t y_dt,
                             void* ws, size_t ws_bytes, int expected_rows, hipStream_t stream) {
    return grouped_ffn(xd, xd_scales, Rows{offsets, nullptr, 0}, E_local, cap_rows, H, I, act_dt,
                       w_gate, w_up, w_down, w_gate_scales, w_up_scales, w_down_scales, w_dt, y, y_dt,
                       ws, ws_bytes, expected_rows, stream);
}

// masked layout: rows of local expert j are [j*cap_e, j*cap_e + m[j]) of E_local*cap_e
#define MASKED_ROWS()                                                                          \
    REQUIRE(cap_per_expert >= 1, "cap_per_expert must be >= 1 (got %d)", cap_per_expert);     \
    REQUIRE(E_local >= 1 && E_local <= 1024, "E_local must be in [1, 1024] (got %d)", E_local); \
    REQUIRE((long long)E_local * cap_per_expert <= 0x7fffffffLL, "E_local * cap_per_expert must fit in int32")

moe_status_t moe_ffn_gate_up_masked(const void* xd, const float* xd_scales, const int32_t* m,
                                    int E_local, int cap_per_expert, int H, int I, moe_dtype_t act_dt,
                                    const void* w_gate, const void* w_up, const float* w_gate_scales,
                                    const float* w_up_scales, moe_dtype_t w_dt, void* h,
                                    float* h_scales, int expected_rows, hipStream_t stream) {
    MASKED_ROWS();
    REQUIRE(m, "null m");
    return ffn_gate_up(xd, xd_scales, Rows{nullptr, m, cap_per_expert}, E_local, E_local * cap_per_expert,
                       H, I, act_dt, w_gate, w_up, w_gate_scales, w_up_scales, w_dt, h, h_scales,
                       expected_rows, stream);
}

moe_status_t moe_ffn_down_masked(const void* h, const float* h_scales, const int32_t* m, int E_local,
                                 int cap_per_expert, int H, int I, moe_dtype_t act_dt,
                                 const void* w_down, const float* w_down_scales, moe_dtype_t w_dt,
                                 void* y, moe_dtype_t y_dt, int expected_rows, hipStream_t stream) {
    MASKED_ROWS();
    REQUIRE(m, "null m");
    return ffn_down(h, h_scales, Rows{nullptr, m, cap_per_expert}, E_local, E_local * cap_per_expert,
                    H, I, act_dt, w_down, w_down_scales, w_dt, y, y_dt, expected_rows, stream);
}

moe_status_t moe_grouped_ffn_masked(const void* xd, const float* xd_scales, const int32_t* m,
                                    int E_local, int cap_per_expert, int H, int I, moe_dtype_t act_dt,
                                    const void* w_gate, const void* w_up, const void* w_down,
                                    const float* w_gate_scales, const float* w_up_scales,
                                    const float* w_down_scales, moe_dtype_t w_dt, void* y,
                                    moe_dtype_t y_dt, void* ws, size_t ws_bytes, int expected_rows,
                                    hipStream_t stream) {
    MASKED_ROWS();
    REQUIRE(m, "null m");
    return grouped_ffn(xd, xd_scales, Rows{nullptr, m, cap_per_expert}, E_local,
                       E_local * cap_per_expert, H, I, act_dt, w_gate, w_up, w_down, w_gate_scales,
                       w_up_scales, w_down_scales, w_dt, y, y_dt, ws, ws_bytes, expected_rows, stream);
}

moe_status_t moe_combine(const void* y, moe_dtype_t y_dt, int cap_rows, const int32_t* row_of,
                         const float* topk_w, int B, int K, int H, void* out, moe_dtype_t out_dt,
                         hipStream_t stream) {
    REQUIRE(B >= 0 && K >= 1 && K <= 1024, "need B >= 0 and 1 <= K <= 1024");
    REQUIRE((long long)B * K <= 0x7fffffffLL, "B*K must fit in int32");
    REQUIRE(H >= 8 && H % 8 == 0, "H must be a positive multiple of 8 (got %d)", H);
    REQUIRE(cap_rows >= 0, "cap_rows must be >= 0");
    int kind;
    if (y_dt == MOE_F32 && out_dt == MOE_F32) kind = 0;
    else if (y_dt == MOE_BF16 && out_dt == MOE_BF16) kind = 1;
    else if (y_dt == MOE_BF16 && out_dt == MOE_F32) kind = 2;
    else return fail(MOE_ERR_UNSUPPORTED, "unsupported combine (y_dt, out_dt) = (%d, %d)", y_dt, out_dt);
    if (B > 0) {
        REQUIRE(y && row_of && topk_w && out, "null pointer argument");
        REQUIRE(aligned16(y) && aligned16(out), "y and out must be 16-byte aligned");
    }
    return launched(moeep::launch_combine(y, kind, row_of, topk_w, B, K, H, out, cap_rows, stream),
                    "moe_combine");
}

}  // extern "C"
