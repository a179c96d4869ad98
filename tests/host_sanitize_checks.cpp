// Host-side checks of libmoeep, built with AddressSanitizer and UBSan
// (host code only): every argument-validation path of the C ABI, the
// workspace queries, the status strings and the host expert-placement
// routine.  Nothing here reaches the GPU: each rejected call fails its host
// check before any HIP call, empty batches return before any launch, and
// the device pointers are stand-in addresses that are never dereferenced.
// Prints "host checks ok" and exits 0 when every expectation holds.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "moeep.h"

namespace {

int failures = 0;

void expect(bool cond, const char* what, int line) {
    if (!cond) {
        std::printf("FAIL line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

void expect_status(moe_status_t got, moe_status_t want, const char* what, int line) {
    if (got != want) {
        std::printf("FAIL line %d: %s returned %d, expected %d (%s)\n", line, what, (int)got, (int)want,
                    moe_last_error());
        ++failures;
    } else if (want != MOE_OK && std::strlen(moe_last_error()) == 0) {
        std::printf("FAIL line %d: %s gave no error text\n", line, what);
        ++failures;
    }
}
#define STATUS(call, want) expect_status((call), (want), #call, __LINE__)

// stand-in device addresses: 256-byte aligned, misaligned, never dereferenced
void* const D = reinterpret_cast<void*>(uintptr_t{1} << 20);
void* const D_MIS = reinterpret_cast<void*>((uintptr_t{1} << 20) + 4);
const float* const DF = static_cast<const float*>(D);
float* const DFm = static_cast<float*>(D);
int32_t* const DI = static_cast<int32_t*>(D);

void status_strings() {
    for (int s = 0; s < 4; ++s) EXPECT(moe_status_string((moe_status_t)s) != nullptr);
    EXPECT(moe_status_string((moe_status_t)99) != nullptr);
    EXPECT(std::strstr(moe_version(), "gfx950") != nullptr);
}

void route() {
    STATUS(moe_route(DF, 4, 0, 1, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route(DF, 4, 2000, 2, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route(DF, 4, 8, 9, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route(DF, -1, 8, 2, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route(DF, INT_MAX, 1024, 8, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);   // B*K, B*E
    STATUS(moe_route(nullptr, 4, 8, 2, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route(nullptr, 0, 8, 2, nullptr, nullptr, nullptr), MOE_OK);             // empty batch
    STATUS(moe_route_mapped(DF, 4, 8, 2, nullptr, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route_shared(DF, 4, 8, 2, -1, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route_shared(DF, 4, 1000, 2, 30, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_route_shared(DF, INT_MAX / 4, 8, 2, 8, DI, DFm, nullptr), MOE_ERR_INVALID_ARG);
}

void placement() {
    std::vector<int64_t> load(256);
    std::vector<int32_t> phys(256);
    STATUS(moe_eplb_place(load.data(), 0, 1, phys.data()), MOE_ERR_INVALID_ARG);
    STATUS(moe_eplb_place(load.data(), 8, 3, phys.data()), MOE_ERR_INVALID_ARG);
    STATUS(moe_eplb_place(nullptr, 8, 2, phys.data()), MOE_ERR_INVALID_ARG);
    load[3] = -1;
    STATUS(moe_eplb_place(load.data(), 8, 2, phys.data()), MOE_ERR_INVALID_ARG);
    // valid loads of several shapes: a permutation with E / G experts per group
    std::mt19937_64 rng(7);
    const int shapes[][2] = {{256, 8}, {256, 1}, {256, 256}, {1024, 8}, {7, 7}, {12, 4}};
    for (const auto& sh : shapes) {
        const int E = sh[0], G = sh[1];
        load.assign(E, 0);
        phys.assign(E, -1);
        for (auto& l : load) l = (int64_t)(rng() % 100000);
        STATUS(moe_eplb_place(load.data(), E, G, phys.data()), MOE_OK);
        std::vector<int> seen(E, 0);
        for (int e = 0; e < E; ++e) {
            EXPECT(phys[e] >= 0 && phys[e] < E);
            if (phys[e] >= 0 && phys[e] < E) ++seen[phys[e]];
        }
        for (int e = 0; e < E; ++e) EXPECT(seen[e] == 1);
    }
    // loads whose group totals do not fit in 64 bits are rejected, not summed
    load.assign(8, INT64_MAX / 3);
    phys.assign(8, -1);
    STATUS(moe_eplb_place(load.data(), 8, 2, phys.data()), MOE_ERR_INVALID_ARG);
    // the largest accepted totals
    load.assign(8, INT64_MAX / 8);
    STATUS(moe_eplb_place(load.data(), 8, 1, phys.data()), MOE_OK);
}

void layout() {
    const size_t ws = moe_layout_workspace_bytes(4, 2, 8);
    EXPECT(ws % 256 == 0);
    EXPECT(moe_layout_workspace_bytes(-1, 2, 8) == 0);
    EXPECT(moe_layout_workspace_bytes(INT_MAX / 1024, 1024, 1024) % 256 == 0);
    EXPECT(moe_layout_workspace_bytes(INT_MAX, 8, 8) == 0);                             // B*K past int32
    STATUS(moe_layout(DI, 4, 2, 8, 3, 3, DI, DI, DI, DI, 8, D, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout(DI, 4, 2, 8, 0, 9, DI, DI, DI, DI, 8, D, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout(DI, 4, 2, 8, 0, 8, DI, DI, DI, DI, 8, D_MIS, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout(DI, 4, 2, 8, 0, 8, DI, DI, DI, DI, 8, D, 4, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout(DI, 4, 2, 8, 0, 8, nullptr, DI, DI, DI, 8, D, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout(DI, 4, 2, 8, 0, 8, DI, DI, DI, DI, -1, D, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout(DI, INT_MAX / 2, 8, 8, 0, 8, DI, DI, DI, DI, 8, D, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout_masked(DI, 4, 2, 8, 0, 8, DI, DI, DI, DI, 0, D, ws, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_layout_masked(DI, 4, 2, 1024, 0, 1024, DI, DI, DI, DI, INT_MAX / 2, D, ws, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_layout_masked(DI, 4, 2, 8, 0, 8, DI, nullptr, DI, DI, 4, D, ws, nullptr), MOE_ERR_INVALID_ARG);
}

void dispatch() {
    const void* segs[MOE_MAX_SEGMENTS + 1];
    int32_t rows[MOE_MAX_SEGMENTS + 1];
    for (int i = 0; i <= MOE_MAX_SEGMENTS; ++i) {
        segs[i] = D;
        rows[i] = 4;
    }
    STATUS(moe_dispatch(segs, rows, 0, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 8, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_dispatch(segs, rows, MOE_MAX_SEGMENTS + 1, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 8,
                        nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_dispatch(nullptr, rows, 1, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 8, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_dispatch(segs, rows, 1, MOE_BF16, 100, DI, 2, D, MOE_BF16, nullptr, 8, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_dispatch(segs, rows, 1, MOE_BF16, 128, DI, 0, D, MOE_BF16, nullptr, 8, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_dispatch(segs, rows, 1, MOE_F32, 128, DI, 2, D, MOE_FP8_E4M3, nullptr, 8, nullptr),
           MOE_ERR_UNSUPPORTED);
    STATUS(moe_dispatch(segs, rows, 1, 42, 128, DI, 2, D, MOE_BF16, nullptr, 8, nullptr), MOE_ERR_UNSUPPORTED);
    STATUS(moe_dispatch(segs, rows, 1, MOE_BF16, 128, DI, 2, D, MOE_FP8_E4M3, nullptr, 8, nullptr),
           MOE_ERR_INVALID_ARG);                                                       // no scales
    STATUS(moe_dispatch(segs, rows, 1, MOE_BF16, 128, DI, 2, D_MIS, MOE_BF16, nullptr, 8, nullptr),
           MOE_ERR_INVALID_ARG);                                                       // misaligned xd
    segs[1] = D_MIS;
    STATUS(moe_dispatch(segs, rows, 2, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 16, nullptr),
           MOE_ERR_INVALID_ARG);                                                       // misaligned segment
    segs[1] = nullptr;
    STATUS(moe_dispatch(segs, rows, 2, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 16, nullptr),
           MOE_ERR_INVALID_ARG);                                                       // null segment
    segs[1] = D;
    rows[1] = -3;
    STATUS(moe_dispatch(segs, rows, 2, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 16, nullptr),
           MOE_ERR_INVALID_ARG);
    rows[0] = INT_MAX;
    rows[1] = INT_MAX;
    STATUS(moe_dispatch(segs, rows, 2, MOE_BF16, 128, DI, 2, D, MOE_BF16, nullptr, 16, nullptr),
           MOE_ERR_INVALID_ARG);                                                       // tokens overflow
    rows[0] = rows[1] = 0;                                                             // empty batch
    STATUS(moe_dispatch(segs, rows, 2, MOE_BF16, 128, nullptr, 2, nullptr, MOE_BF16, nullptr, 0, nullptr),
           MOE_OK);
}

void ffn() {
    const moe_dtype_t BF = MOE_BF16, F8 = MOE_FP8_E4M3, F32 = MOE_F32;
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 8, 64, 128, 128, BF, D, D, nullptr, nullptr, F8, D, nullptr, 0,
                           nullptr), MOE_ERR_UNSUPPORTED);
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 0, 64, 128, 128, BF, D, D, nullptr, nullptr, BF, D, nullptr, 0,
                           nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 8, 64, 100, 128, BF, D, D, nullptr, nullptr, BF, D, nullptr, 0,
                           nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 8, INT_MAX, 1 << 20, 128, BF, D, D, nullptr, nullptr, BF, D,
                           nullptr, 0, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up(D_MIS, nullptr, DI, 8, 64, 128, 128, BF, D, D, nullptr, nullptr, BF, D, nullptr, 0,
                           nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 8, 64, 128, 128, BF, nullptr, D, nullptr, nullptr, BF, D, nullptr,
                           0, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 8, 64, 128, 128, F8, D, D, nullptr, nullptr, F8, D, nullptr, 0,
                           nullptr), MOE_ERR_INVALID_ARG);                             // fp8 scales
    STATUS(moe_ffn_gate_up(D, nullptr, nullptr, 8, 64, 128, 128, BF, D, D, nullptr, nullptr, BF, D, nullptr,
                           0, nullptr), MOE_ERR_INVALID_ARG);
    // no rows: nothing to launch
    STATUS(moe_ffn_gate_up(D, nullptr, DI, 8, 0, 128, 128, BF, D, D, nullptr, nullptr, BF, D, nullptr, 0,
                           nullptr), MOE_OK);
    STATUS(moe_ffn_down(D, nullptr, DI, 8, 64, 128, 128, BF, D, nullptr, BF, D, F32, 0, nullptr),
           MOE_ERR_UNSUPPORTED);
    STATUS(moe_ffn_down(D, nullptr, DI, 8, 64, 128, 128, 9, D, nullptr, 9, D, BF, 0, nullptr),
           MOE_ERR_UNSUPPORTED);
    STATUS(moe_ffn_down(D, nullptr, DI, 8, 64, 128, 128, BF, nullptr, nullptr, BF, D, BF, 0, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_down(D, nullptr, DI, 8, 64, 128, 128, F8, D, nullptr, F8, D, BF, 0, nullptr),
           MOE_ERR_INVALID_ARG);
    const size_t ws = moe_ffn_workspace_bytes(64, 128, BF);
    EXPECT(ws >= 64u * 128u * 2u && ws % 256 == 0);
    EXPECT(moe_ffn_workspace_bytes(-1, 128, BF) == 0);
    EXPECT(moe_ffn_workspace_bytes(INT_MAX, INT_MAX, F8) > 0);
    STATUS(moe_grouped_ffn(D, nullptr, DI, 8, 64, 128, 128, BF, D, D, D, nullptr, nullptr, nullptr, BF, D, BF,
                           D, 16, 0, nullptr), MOE_ERR_INVALID_ARG);                   // small workspace
    STATUS(moe_grouped_ffn(D, nullptr, DI, 8, 64, 128, 128, BF, D, D, D, nullptr, nullptr, nullptr, BF, D, BF,
                           D_MIS, ws, 0, nullptr), MOE_ERR_INVALID_ARG);               // misaligned
    STATUS(moe_grouped_ffn(D, nullptr, DI, 8, 64, 128, 128, BF, D, D, D, nullptr, nullptr, nullptr, BF, D, BF,
                           nullptr, ws, 0, nullptr), MOE_ERR_INVALID_ARG);
    // masked variants
    STATUS(moe_ffn_gate_up_masked(D, nullptr, DI, 8, 0, 128, 128, BF, D, D, nullptr, nullptr, BF, D, nullptr, 0,
                                  nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up_masked(D, nullptr, nullptr, 8, 8, 128, 128, BF, D, D, nullptr, nullptr, BF, D,
                                  nullptr, 0, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_gate_up_masked(D, nullptr, DI, 1024, INT_MAX / 2, 128, 128, BF, D, D, nullptr, nullptr, BF,
                                  D, nullptr, 0, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_ffn_down_masked(D, nullptr, nullptr, 8, 8, 128, 128, BF, D, nullptr, BF, D, BF, 0, nullptr),
           MOE_ERR_INVALID_ARG);
    STATUS(moe_grouped_ffn_masked(D, nullptr, nullptr, 8, 8, 128, 128, BF, D, D, D, nullptr, nullptr, nullptr,
                                  BF, D, BF, D, ws, 0, nullptr), MOE_ERR_INVALID_ARG);
}

void combine() {
    STATUS(moe_combine(D, MOE_BF16, 8, DI, DF, 4, 0, 128, D, MOE_BF16, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_combine(D, MOE_BF16, 8, DI, DF, 4, 2, 100, D, MOE_BF16, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_combine(D, MOE_BF16, 8, DI, DF, INT_MAX, 8, 128, D, MOE_BF16, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_combine(D, MOE_BF16, -1, DI, DF, 4, 2, 128, D, MOE_BF16, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_combine(D, MOE_FP8_E4M3, 8, DI, DF, 4, 2, 128, D, MOE_BF16, nullptr), MOE_ERR_UNSUPPORTED);
    STATUS(moe_combine(nullptr, MOE_BF16, 8, DI, DF, 4, 2, 128, D, MOE_BF16, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_combine(D, MOE_BF16, 8, DI, DF, 4, 2, 128, D_MIS, MOE_BF16, nullptr), MOE_ERR_INVALID_ARG);
    STATUS(moe_combine(nullptr, MOE_BF16, 0, nullptr, nullptr, 0, 2, 128, nullptr, MOE_BF16, nullptr), MOE_OK);
    // dtype codes that name no type
    STATUS(moe_combine(D, 7, 8, DI, DF, 4, 2, 128, D, MOE_BF16, nullptr), MOE_ERR_UNSUPPORTED);
    STATUS(moe_combine(D, MOE_BF16, 8, DI, DF, 4, 2, 128, D, -1, nullptr), MOE_ERR_UNSUPPORTED);
}

}  // namespace

int main() {
    status_strings();
    route();
    placement();
    layout();
    dispatch();
    ffn();
    combine();
    if (failures) {
        std::printf("%d host check(s) failed\n", failures);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
