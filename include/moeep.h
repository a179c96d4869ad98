/*
 * moeep.h -- C ABI of libmoeep, the single-GPU data-parallel path of an
 * expert-parallel Mixture-of-Experts layer on AMD Instinct MI355X (gfx950):
 *
 *     route -> layout -> dispatch -> grouped SwiGLU FFN -> combine
 *
 * Sources, cited by page title and section:
 *   [Anatomy]  "Anatomy of a high-performance EP kernel" (euno.news, Korean;
 *              Chinese translation on 66bd.net), section "What we have to
 *              do" and its router figure, section "Dispatch".
 *   [Moreh]    Moreh, "21K output tokens/s DeepSeek inference on AMD
 *              Instinct MI300X GPUs with Expert Parallelism", sections
 *              "Parallelisation method", "Load balancing across GPUs",
 *              "Using HIP Graphs".
 *   [SGLang]   SGLang documentation, "Expert Parallelism", section
 *              "Framework Overview" (the dispatch -> pre-permute -> grouped
 *              GEMM -> post-permute -> combine flow) and the MoE-runner
 *              backend table (contiguous layout, fp8 block quantisation).
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers to caller-owned memory unless
 *     marked "host".  Tensors are row-major and dense.  The library never
 *     allocates, frees, synchronises or copies device->host; every call only
 *     enqueues kernels on `stream` (0 = the null stream) and returns.
 *   - Arguments are checked on the host before anything is enqueued.  A
 *     non-OK status means nothing was enqueued and no output was touched;
 *     moe_last_error() then holds a message (thread-local).
 *   - MOE_ERR_HIP reports a failed kernel launch.  Faults inside a kernel
 *     surface, as always with HIP, at the caller's next synchronisation.
 *   - Sizes: 1 <= K <= E <= 1024; 0 <= e_begin < e_end <= E; B >= 0;
 *     H and I multiples of 8 (of 16 when activations are fp8); row base
 *     pointers 16-byte aligned.
 *   - Calls on one stream run in order; calls that share output or
 *     workspace buffers on different streams race.
 *   - Expert ids outside [0, E) in topk_ids are treated as unrouted slots.
 *   - Non-finite logits or activations are outside the method; results
 *     are then unspecified (but all memory accesses stay in bounds).
 */
#ifndef MOEEP_H
#define MOEEP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status and dtype codes are plain 32-bit integers with named values, so
   every value a caller passes (an unknown dtype code, an out-of-range
   status for moe_status_string) is well defined and gets a status or a
   string back. */
typedef int32_t moe_status_t;
enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* a pointer, size or alignment check failed */
    MOE_ERR_UNSUPPORTED = 2,   /* a valid but unimplemented dtype/shape combination */
    MOE_ERR_HIP = 3            /* a kernel launch failed */
};

typedef int32_t moe_dtype_t;
enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_FP8_E4M3 = 2,          /* OCP e4m3fn (finite max 448), with fp32 1x128 block scales */
    MOE_FP8_E4M3_PO2 = 3       /* weights only: e4m3fn whose fp32 block scales are all powers
                                  of two 2^e, e in [-127, 127] (the E8M0 scale convention of
                                  the microscaling formats); the matrix cores apply such
                                  scales, and only a scale's exponent field is read */
};

/* Largest number of simulated source segments moe_dispatch accepts. */
#define MOE_MAX_SEGMENTS 64
/* fp8 scale block length along the contraction (row) dimension. */
#define MOE_FP8_BLOCK 128

const char* moe_status_string(moe_status_t status);
const char* moe_last_error(void);
const char* moe_version(void);

/*
 * moe_route -- top-K expert selection and gate weights.
 * [Anatomy] "What we have to do": each token's (E) logit row is reduced to
 * the indices of its K largest logits, a (B, K) assignment tensor.  Gate
 * weights are the softmax over the K selected logits (the full softmax
 * renormalised over the picks).
 *
 *   logits   (B, E) fp32, finite.
 *   topk_ids (B, K) int32 out: slot k holds the k-th largest logit; equal
 *            logits are taken in ascending expert id (-0.0 equals +0.0).
 *   topk_w   (B, K) fp32 out: exp(l_k - l_0) / sum_j exp(l_j - l_0).
 * B = 0 is a no-op.
 */
moe_status_t moe_route(const float* logits, int B, int E, int K,
                       int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * moe_layout -- per-expert histogram, exclusive prefix sum and permutation
 * of the routed slots into expert-contiguous rows.  [Anatomy] "Dispatch":
 * each expert receives its own number of rows and the grouped GEMM runs
 * over one row set per expert; [SGLang] "Framework Overview": pre-permute.
 *
 *   topk_ids (B, K) int32.
 *   counts   (E) int32 out: slots routed to each of the E experts.
 *   offsets  (e_end - e_begin + 1) int32 out: exclusive scan of counts over
 *            the local experts [e_begin, e_end), total last.  Local expert j
 *            (global id e_begin + j) owns rows [offsets[j], offsets[j+1]).
 *   row_of   (B, K) int32 out: destination row of slot (t, k), -1 if its
 *            expert is not local.
 *   src_of   (cap_rows) int32 out: slot t*K + k held by each row; -1 for the
 *            rows [offsets[E_loc], cap_rows).
 *   Rows of one expert are ordered by (t, k) ascending, so the result is
 *   deterministic and bit-identical run to run.
 *   cap_rows >= B * K * (fraction routed locally); B * K always suffices.
 *   If more local slots than cap_rows arrive, the rows past cap_rows are
 *   dropped: their row_of is -1 and offsets still count them.
 *   ws / ws_bytes: device workspace of at least
 *   moe_layout_workspace_bytes(B, K, E) bytes, 256-byte aligned.
 */
/*
 * moe_route_mapped -- moe_route with a placement map.  [Moreh] load
 * balancing between GPUs: experts are renumbered so each rank's set is a
 * contiguous id range, and the gating network emits the renumbered ids.
 * Selection, slot order, ties and gates are exactly those of moe_route on
 * the logical ids; each chosen id e is written as phys_of_logical[e].
 *   phys_of_logical (E) int32 device table, a permutation of [0, E) (e.g.
 *   from moe_eplb_place); entries are used as given.
 * Errors as for moe_route, plus a null phys_of_logical.
 */
moe_status_t moe_route_mapped(const float* logits, int B, int E, int K, const int32_t* phys_of_logical,
                              int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * moe_route_shared -- moe_route plus n_shared always-on (shared) experts.
 * [Moreh] "Overview": besides the routed experts a shared expert runs for
 * every token regardless of routing; "Library optimizations": its GEMMs are
 * merged with others (horizontal fusion).  Here the shared experts become
 * ordinary groups of the same grouped FFN: every output row holds the K
 * routed picks of moe_route (same ids, order and renormalised gates) followed
 * by n_shared slots with ids E, E+1, ..., E+n_shared-1 and gate 1.0.
 *   ids, w  (B, K + n_shared) int32 / fp32 out.
 * Run the rest of the layer with E' = E + n_shared experts and K' = K +
 * n_shared slots (the shared experts' weights after the routed ones): every
 * token then lands in each shared expert's group, and combine adds the
 * shared outputs with weight 1.
 * Errors as for moe_route, plus n_shared < 0 or E + n_shared > 1024.
 */
moe_status_t moe_route_shared(const float* logits, int B, int E, int K, int n_shared, int32_t* ids,
                              float* w, hipStream_t stream);

/*
 * moe_eplb_place -- expert placement for load balancing (host function; no
 * GPU work).  [Moreh] load balancing between GPUs: group E experts into
 * n_groups sets of E/n_groups with activation totals as equal as possible
 * and renumber them so set g is the id range [g*S, (g+1)*S), S = E/n_groups.
 * [SGLang] workload balancer: balancedness is mean/max of the per-rank load.
 * Algorithm (the report gives none): experts in decreasing load (ties: lower
 * id) each join the least-loaded set with room (ties: lower set); then, while
 * the most and the least loaded sets differ, the swap between them whose load
 * difference d (0 < d < gap) is closest to gap/2 is made (ties: lower ids);
 * ids inside a set ascend with the logical id.
 *   load  (E) int64 host, >= 0, total <= INT64_MAX: activation counts (e.g.
 *         summed moe_layout counts).
 *   phys_of_logical (E) int32 host out.
 * Returns MOE_ERR_INVALID_ARG for E outside [1, 1024], n_groups not dividing
 * E, a negative load, loads whose total does not fit in int64, or null
 * pointers.
 */
moe_status_t moe_eplb_place(const int64_t* load, int E, int n_groups, int32_t* phys_of_logical);

size_t moe_layout_workspace_bytes(int B, int K, int E);
moe_status_t moe_layout(const int32_t* topk_ids, int B, int K, int E, int e_begin, int e_end,
                        int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                        int cap_rows, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_layout_noalloc -- moe_layout for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results minus the workspace,
 * which the library holds itself as one static device array of
 * MOE_LAYOUT_NOALLOC_SCRATCH_BYTES per GPU (kept until the process ends).
 * Calls no hipMalloc or hipFree.  A batch whose workspace
 * (moe_layout_workspace_bytes(B, K, E)) exceeds that size is rejected with
 * MOE_ERR_INVALID_ARG before anything is enqueued: 4 MiB holds E * ceil(B*K
 * / 256) int32 chunk histograms, e.g. E = 256 up to B*K = 1,048,320 slots
 * (the T = 8192, K = 8 prefill needs 256 KiB); batches of at most 4096 slots
 * use no workspace at all.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * serialised by the caller.  Nothing in the array has to start at zero: each
 * call writes every histogram entry it reads.  The first call on a GPU looks
 * up the array's device address for that GPU (hipGetSymbolAddress) with the
 * caller's device current; a failure there returns MOE_ERR_HIP.
 */
#define MOE_LAYOUT_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status_t moe_layout_noalloc(const int32_t* topk_ids, int B, int K, int E, int e_begin, int e_end,
                                int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                int cap_rows, hipStream_t stream);

/*
 * moe_layout_masked -- the fixed-capacity ("masked") layout.  [SGLang]
 * MoE-runner table: the grouped GEMM takes a contiguous layout for prefill
 * and a masked layout for decode; the dispatch paragraph pairs the
 * low-latency decode mode with graph capture.  Local expert j owns the fixed
 * row block [j*cap_per_expert, (j+1)*cap_per_expert) of an
 * (E_local*cap_per_expert)-row buffer, so no prefix sum is needed and every
 * size is static.
 *   counts   (E) int32 out: slots routed to each expert (all E experts).
 *   m        (E_local) int32 out: valid rows of local expert j,
 *            min(counts[e_begin + j], cap_per_expert) -- the mask.
 *   row_of   (B, K) int32 out: j*cap_per_expert + rank of (t, k) among its
 *            expert's slots in (t, k) order; -1 for non-local slots and for
 *            slots with rank >= cap_per_expert (dropped, still counted).
 *   src_of   (E_local*cap_per_expert) int32 out: slot t*K+k of each row, -1
 *            for rows past m[j] in each block.
 *   ws       as for moe_layout (moe_layout_workspace_bytes(B, K, E)).
 * Arguments are checked as for moe_layout, plus cap_per_expert >= 1 and
 * E_local*cap_per_expert < 2^31.  moe_dispatch and moe_combine take this
 * row_of unchanged with cap_rows = E_local*cap_per_expert; the FFN takes m
 * through the *_masked entry points below.
 */
moe_status_t moe_layout_masked(const int32_t* topk_ids, int B, int K, int E, int e_begin, int e_end,
                               int32_t* counts, int32_t* m, int32_t* row_of, int32_t* src_of,
                               int cap_per_expert, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_dispatch -- scatter token rows into the dense expert-contiguous
 * buffer that feeds the grouped GEMM.  [Anatomy] "Dispatch": the tokens for
 * the local experts are gathered into one dense buffer so the grouped GEMM
 * takes them in one call.  On one GPU the transport is an HBM copy; the
 * tokens arrive from n_seg simulated source ranks ([Anatomy] "What we have
 * to do": every data-parallel rank holds its own (B_i, H) activations).
 *
 *   seg_x    host array of n_seg device pointers, segment i is (seg_rows[i], H)
 *            of x_dt.  Global token t is the segment-major concatenation.
 *   seg_rows host array of n_seg row counts (B = their sum).
 *   row_of   (B, K) int32 from moe_layout.
 *   xd       (cap_rows, H) of xd_dt out: xd[row_of[t,k]] = x[t] for every
 *            local slot.  Rows not named by row_of are not written.
 *   xd_scales (cap_rows, ceil(H/128)) fp32 out, fp8 only (else may be NULL).
 * Supported (x_dt -> xd_dt): F32 -> F32 and BF16 -> BF16 (bit-exact
 * copies); BF16 -> FP8_E4M3 (each token quantised once: per 128-element
 * block s = the smallest power of two 2^e with amax <= 448 * 2^e, e >= -127
 * (1 if amax = 0; the E8M0 scale convention), code = RNE(v/s) saturated to
 * +-448, with fp32 arithmetic; all K copies carry identical codes and
 * scales).
 */
moe_status_t moe_dispatch(const void* const* seg_x, const int32_t* seg_rows, int n_seg,
                          moe_dtype_t x_dt, int H, const int32_t* row_of, int K,
                          void* xd, moe_dtype_t xd_dt, float* xd_scales,
                          int cap_rows, hipStream_t stream);

/*
 * Grouped SwiGLU expert FFN.  [Moreh] "Overview": experts are small FFN
 * layers; [Anatomy] "Dispatch": one grouped GEMM over a separate row set
 * per expert; [SGLang] MoE-runner table: contiguous (prefill) layout and
 * fp8 block-wise quantisation.  For each local expert j and its rows
 * [offsets[j], offsets[j+1]) of xd:
 *     g = Xd W_gate[j]^T,  u = Xd W_up[j]^T   (fp32 accumulation)
 *     h = silu(g) * u                          stored as act_dt
 *     y = h W_down[j]^T                        (fp32 accumulation) stored as y_dt
 * Weights use the (out, in) layout: w_gate, w_up (E_local, I, H);
 * w_down (E_local, H, I), local expert j first.  fp8 weights carry fp32
 * scales per (output row, 128-wide block of the input dim):
 * w_gate_scales, w_up_scales (E_local, I, ceil(H/128)),
 * w_down_scales (E_local, H, ceil(I/128)).  fp8 activations carry
 * xd_scales (cap_rows, ceil(H/128)) and h_scales (cap_rows, ceil(I/128)).
 * h is quantised like the dispatched activations.  Rows past
 * offsets[E_local] of h and y are not written.
 *
 * Supported (act_dt, w_dt, y_dt): (F32, F32, F32), (BF16, BF16, BF16),
 * (FP8_E4M3, FP8_E4M3, BF16), (FP8_E4M3, FP8_E4M3_PO2, BF16).  The
 * activation block scales of the fp8 path (xd_scales from moe_dispatch,
 * h_scales) are always powers of two; FP8_E4M3_PO2 declares that the
 * weight scales are too, which lets the row-rich kernels apply every scale
 * in the matrix cores (same results up to fp32 rounding order).  Any w_dt
 * may carry MOE_W_PACKED: weights packed by moe_pack_weights (below).
 *
 * moe_ffn_gate_up computes h; moe_ffn_down computes y from h;
 * moe_grouped_ffn runs both with h (and h_scales) carved from `ws`, which
 * must hold moe_ffn_workspace_bytes(cap_rows, I, act_dt) bytes.
 * The row counts per expert are read on the device: no host
 * synchronisation, launch sizes depend only on the arguments.
 * expected_rows is a hint, the rows a local expert is expected to receive
 * (e.g. B * K / E for balanced routing); it only selects the tile shape and
 * never changes results.  expected_rows <= 0 means cap_rows / E_local.
 */
size_t moe_ffn_workspace_bytes(int cap_rows, int I, moe_dtype_t act_dt);

/*
 * Packed expert weights: a one-time layout transform of this library, not a
 * step of the method (the pages leave the weights' memory layout open).  The
 * FFN kernels stream every weight row along its input dimension in 128-byte
 * steps; a row whose length is not a whole number of 128-byte lines makes
 * every step straddle two lines, and rows exactly a multiple of 4 KiB apart
 * stream markedly slower than rows one line further apart.
 *
 * moe_weight_ld(cols, w_dt): the packed row pitch in elements for rows of
 *   `cols` elements of w_dt -- the row length rounded up to whole 128-byte
 *   lines, plus one line when that is a multiple of 4 KiB.  -1 if cols is
 *   outside [1, 2^24] or w_dt is not a weight dtype.
 * moe_packed_weight_bytes: E_local * rows * ld elements, in bytes (0 on
 *   invalid arguments).
 * moe_pack_weights: w (E_local, rows, cols) of w_dt, row-major and
 *   contiguous, is written to w_packed (E_local, rows, ld): each row
 *   unchanged, elements [cols, ld) zero.  cols must be a positive multiple
 *   of 8; both pointers 16-byte aligned, caller-owned, not overlapping.
 *   Asynchronous on `stream`; E_local * rows == 0 is a no-op.
 *
 * An FFN call whose w_dt carries the flag MOE_W_PACKED (e.g. MOE_BF16 |
 * MOE_W_PACKED) reads every weight matrix it takes at the packed pitch:
 * w_gate, w_up (E_local, I, moe_weight_ld(H)), w_down (E_local, H,
 * moe_weight_ld(I)).  Results are identical to the call on the unpacked
 * weights; fp8 weight scales are never packed.
 */
#define MOE_W_PACKED 0x100
int moe_weight_ld(int cols, moe_dtype_t w_dt);
size_t moe_packed_weight_bytes(int E_local, int rows, int cols, moe_dtype_t w_dt);
moe_status_t moe_pack_weights(const void* w, int E_local, int rows, int cols, moe_dtype_t w_dt,
                              void* w_packed, hipStream_t stream);

moe_status_t moe_ffn_gate_up(const void* xd, const float* xd_scales, const int32_t* offsets,
                             int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                             const void* w_gate, const void* w_up,
                             const float* w_gate_scales, const float* w_up_scales, moe_dtype_t w_dt,
                             void* h, float* h_scales, int expected_rows, hipStream_t stream);
moe_status_t moe_ffn_down(const void* h, const float* h_scales, const int32_t* offsets,
                          int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                          const void* w_down, const float* w_down_scales, moe_dtype_t w_dt,
                          void* y, moe_dtype_t y_dt, int expected_rows, hipStream_t stream);
moe_status_t moe_grouped_ffn(const void* xd, const float* xd_scales, const int32_t* offsets,
                             int E_local, int cap_rows, int H, int I, moe_dtype_t act_dt,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const float* w_gate_scales, const float* w_up_scales,
                             const float* w_down_scales, moe_dtype_t w_dt,
                             void* y, moe_dtype_t y_dt, void* ws, size_t ws_bytes,
                             int expected_rows, hipStream_t stream);

/*
 * The same three calls over the masked layout of moe_layout_masked: local
 * expert j's rows are [j*cap_per_expert, j*cap_per_expert + m[j]) of
 * buffers with E_local*cap_per_expert rows (xd, h, y and their scales);
 * m (E_local, device) is read on the device and clamped to
 * [0, cap_per_expert].  Everything else -- weights, dtypes, numerics,
 * workspace (moe_ffn_workspace_bytes(E_local*cap_per_expert, I, act_dt)),
 * expected_rows -- is as above.  Rows past m[j] in a block are not written.
 */
moe_status_t moe_ffn_gate_up_masked(const void* xd, const float* xd_scales, const int32_t* m,
                                    int E_local, int cap_per_expert, int H, int I, moe_dtype_t act_dt,
                                    const void* w_gate, const void* w_up,
                                    const float* w_gate_scales, const float* w_up_scales,
                                    moe_dtype_t w_dt, void* h, float* h_scales, int expected_rows,
                                    hipStream_t stream);
moe_status_t moe_ffn_down_masked(const void* h, const float* h_scales, const int32_t* m,
                                 int E_local, int cap_per_expert, int H, int I, moe_dtype_t act_dt,
                                 const void* w_down, const float* w_down_scales, moe_dtype_t w_dt,
                                 void* y, moe_dtype_t y_dt, int expected_rows, hipStream_t stream);
moe_status_t moe_grouped_ffn_masked(const void* xd, const float* xd_scales, const int32_t* m,
                                    int E_local, int cap_per_expert, int H, int I, moe_dtype_t act_dt,
                                    const void* w_gate, const void* w_up, const void* w_down,
                                    const float* w_gate_scales, const float* w_up_scales,
                                    const float* w_down_scales, moe_dtype_t w_dt,
                                    void* y, moe_dtype_t y_dt, void* ws, size_t ws_bytes,
                                    int expected_rows, hipStream_t stream);

/*
 * moe_combine -- gate-weighted gather-reduce back to token order.
 * [Anatomy] the paragraph after the router figure: results go back to
 * where their tokens live; [SGLang] "Framework Overview": post-permute and
 * combine.  out[t] = sum over k with row_of[t,k] >= 0, in ascending k, of
 * topk_w[t,k] * y[row_of[t,k]], accumulated in fp32 and rounded once to
 * out_dt (RNE).  Tokens with no local slot get 0.  With only part of the
 * experts local this is the rank's partial sum.
 *   y (cap_rows, H) y_dt; row_of, topk_w (B, K); out (B, H) out_dt.
 *   Rows named by row_of outside [0, cap_rows) are skipped like -1.
 * Supported (y_dt, out_dt): (F32, F32), (BF16, BF16), (BF16, F32).
 */
moe_status_t moe_combine(const void* y, moe_dtype_t y_dt, int cap_rows, const int32_t* row_of,
                         const float* topk_w, int B, int K, int H,
                         void* out, moe_dtype_t out_dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEEP_H */
