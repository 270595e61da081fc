/*
 * hmm.h -- C ABI of the MI355X (gfx950) fused MoE-FFN expert library, libhmm.so.
 *
 * The operation is the one of the HyperMegaMoE RFC ("HyperParallel Multicore
 * HyperMegaMoE fused forward/backward operator"):
 *
 *   forward  (section 2.1, 3.1, 4.1): for every token t and every k < K, with
 *            e = topk_ids[t,k]:  [g|u] = x[t] . up_proj_weight[e];
 *            a = silu(g) * u;  o = a . down_proj_weight[e];
 *            y[t] = sum_k topk_weights[t,k] * o.
 *   backward (section 2.2): dx, d_up_proj_weight, d_down_proj_weight and
 *            d_topk_weights of that function; topk_ids gets no gradient.
 *
 * Like the RFC's two-phase interface (section 2.3 and 10: a workspace-size
 * query, then the execution call, for the forward and for the grad op), each
 * call has a *_sizes query.  Everything except the five user tensors (offsets,
 * group lists, tile tables, intermediate buffers) lives in caller-provided
 * workspace and saved buffers (section 3.3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as tensors are DEVICE pointers (HBM of the current HIP
 *   device); all are caller-owned and caller-allocated.  The library never
 *   allocates device memory.  Its only state is, per host thread and device,
 *   one pinned host word and event for the id check (and for the fused
 *   forward), the backward's second stream (default priority) with its three
 *   events, the optional stage-timing events, and the device array of
 *   hmm_forward_noalloc (64 MiB per device, fixed at load).  That state is made
 *   on the first call that needs it.
 * - All tensors are dense, row-major (last index fastest), with no padding.
 *   bf16 tensors are arrays of 16-bit bfloat16 values; every device pointer must
 *   be 16-byte aligned.
 * - ``stream`` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *   is enqueued asynchronously on it, in order; outputs are valid once the
 *   stream reaches that point.  Only HMM_FLAG_VALIDATE_IDS (a wait for the
 *   routing's id check) and HMM_FLAG_FUSED_FORWARD (a wait for its launch) add
 *   a host wait.
 * - Every check that needs only host data (null pointers, shapes, dtypes,
 *   alignment, workspace size) runs before any HIP call: on failure nothing is
 *   enqueued (RFC section 4.2: invalid input is rejected at the host boundary
 *   and never reaches a device kernel).
 * - Errors are returned as hmm_status; nothing is thrown across the ABI.
 *   hmm_last_error_message() gives a per-thread text for the last failure.
 *   A failed call leaves no state behind: the next call behaves like a fresh
 *   one (RFC section 5.3 and 7.3).
 * - Calls that share a workspace or saved buffer must be ordered by the caller
 *   (same stream, or events); concurrent calls from several host threads on the
 *   same buffers are not supported.
 * - HIP graph capture: calls without HMM_FLAG_VALIDATE_IDS and
 *   HMM_FLAG_FUSED_FORWARD allocate nothing, issue no memset and never wait on
 *   the host, so they may be captured (the backward's second stream joins the
 *   capture through its events).  Make one call of the same kind on the device
 *   before capturing, so the per-device state above exists.
 */
#ifndef HMM_H
#define HMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hmm_status {
  HMM_OK = 0,
  HMM_ERR_NULL_POINTER = 1,          /* a required pointer is NULL */
  HMM_ERR_BAD_SHAPE = 2,             /* T,H,I,E,K inconsistent or out of the supported range */
  HMM_ERR_BAD_DTYPE = 3,             /* unknown or unsupported dtype selection */
  HMM_ERR_MISALIGNED = 4,            /* a device pointer is not 16-byte aligned */
  HMM_ERR_UNSUPPORTED = 5,           /* valid problem the library does not implement */
  HMM_ERR_WORKSPACE_TOO_SMALL = 6,   /* workspace_bytes below the *_sizes figure */
  HMM_ERR_EXPERT_ID_OUT_OF_RANGE = 7,/* some topk_ids value is outside [0, E) */
  HMM_ERR_HIP = 8,                   /* a HIP runtime call failed */
  HMM_ERR_TIMEOUT = 9                /* a bounded device wait gave up; the outputs are incomplete */
} hmm_status;

typedef enum hmm_dtype {
  HMM_BF16 = 0,
  HMM_F32 = 1,
  HMM_FP8_E4M3 = 2,    /* E4M3 with one float32 scale per token row / weight column */
  HMM_MXFP8_E4M3 = 3,  /* E4M3 with one E8M0 exponent per 32 elements along H (MX) */
  HMM_FP8_E4M3_GROUP = 4  /* E4M3 with one float32 scale per 128 elements along H */
} hmm_dtype;

/* Check topk_ids: the routing (its own launch, or on small bf16 problems the
 * up-projection's launch) raises a flag for an id outside [0, E) and also
 * stores it into a pinned host word; the host reads that word and
 * returns HMM_ERR_EXPERT_ID_OUT_OF_RANGE.  The host waits for that copy only
 * after the call's kernels are enqueued, so the check adds no idle time on the
 * GPU; the products of a failing call run with the invalid slots dropped, and
 * its outputs are unspecified.  Without the flag, slots with an invalid id are
 * dropped (they contribute zero) and the flag is recorded in ``saved``
 * (hmm_saved_layout.id_error). */
#define HMM_FLAG_VALIDATE_IDS 1u

/* Tiling of the grouped products.  By default the library picks: 256-row tiles
 * (plus 64-row tiles for expert remainders) when the problem fills the chip,
 * 64x64 tiles when it is small.  These flags force one choice (for tuning and
 * tests); at most one may be set.  A backward must be given the same flags as
 * the forward that filled its ``saved`` buffer. */
#define HMM_FLAG_TILES_LARGE 2u
#define HMM_FLAG_TILES_NARROW 4u

/* Run the forward of a small problem (narrow tiling, S <= 8192, E <= 256, bf16
 * outputs, bf16 up-projection, no shared expert) as ONE persistent launch: routing, both
 * products and the combine, with tile-ready counters between them (RFC 6.1).
 * The results are identical to the kernel sequence.  On MI355X it is slower
 * today (every array one tile writes for another has to go through the
 * device-wide coherence point, because the eight XCDs have separate L2s), so it
 * is opt-in; ignored where it does not apply.
 * Every wait between its tiles is bounded (RFC 5.3 and 7.3: a failure must be
 * diagnosable, not a hang).  A wait that gives up (possible only when not all
 * of the launch's workgroups are resident at once, e.g. beside other work on
 * the device) stops its workgroup and stores a flag into a pinned host word;
 * hmm_forward then waits for the launch to finish and returns HMM_ERR_TIMEOUT,
 * with y and the saved intermediates incomplete.  With this flag hmm_forward
 * therefore returns only after its launch has completed. */
#define HMM_FLAG_FUSED_FORWARD 8u

/* The backward of a large-tiled problem (not the narrow tiling, bf16 outputs)
 * whose act_grad has fewer than 4 waves of 256-row tiles on the chip runs its
 * weight gradients on a second stream of the library's (one per host thread and
 * device, default priority), beside the dX chain on the caller's stream: W2Grad
 * starts with act_grad, W1Grad starts once act_grad has written dH and runs
 * beside input_grad and Combine(dX) (RFC 2.2).  The caller's stream waits for
 * both through events, so the call's ordering on ``stream`` is unchanged.  (With
 * longer products, two of them sharing the L2 caches are slower than one after
 * the other.)  This flag keeps every launch on the caller's stream, in series;
 * results are identical either way. */
#define HMM_FLAG_SERIAL_BACKWARD 16u

/* FP8 backward: act_grad and input_grad, the two products of the dX chain, run on
 * E4M3 with per-row dynamic scales (the MoeDistributeDispatchV2 page's case-3 rule,
 * scale = 448 / max|row|, descale 1 / scale kept, applied to every operand): dy per
 * token and each row of down_proj_weight[e] over H for act_grad; the intermediate
 * dH per row and each row of up_proj_weight[e] over 2I for input_grad.  The weight
 * gradients, the combine and a shared expert's products stay bf16.  Bf16 outputs
 * only (else HMM_ERR_UNSUPPORTED); H a multiple of 128.  Needs the larger
 * workspace that hmm_backward_sizes reports with the flag set; the forward
 * ignores it. */
#define HMM_FLAG_FP8_BACKWARD 32u

/* Problem description.
 *   T  tokens (>= 0; T = 0 is a no-op that still writes zero weight gradients)
 *   H  hidden size, multiple of 64, 64 <= H <= 65536
 *   I  intermediate size, multiple of 64, 64 <= I <= 65536
 *   E  experts held by this device, 1 <= E <= 1024
 *   K  experts per token, 1 <= K <= 16  (the dispatch op's top-k bound)
 *   T*K must stay below 2^31.
 *   out_dtype   HMM_BF16: y, dy, dx, d_up_proj_weight and d_down_proj_weight
 *               are bf16.  HMM_F32 (accuracy mode, RFC 7.1's 1e-3 agreement with
 *               an unrounded computation): those five are float32, and every
 *               intermediate is kept in float32 or as a bf16 pair hi + lo
 *               (hi = bf16(v), lo = bf16(v - hi)); about twice the MFMA work.
 *               Needs gmm1_dtype HMM_BF16.
 *   gmm1_dtype  HMM_BF16, or HMM_FP8_E4M3 for the FP8 up-projection: tokens
 *               are quantised per row, the up-projection weight per
 *               (expert, column), both as scale = 448 / max|.| (the per-token
 *               dynamic quantisation of MoeDistributeDispatchV2, case 3);
 *               H must then be a multiple of 128.  Only the up-projection
 *               changes: the rest of the forward and the backward stay bf16.
 *               HMM_MXFP8_E4M3: the MX quantisation of MoeDistributeDispatchV2
 *               (case 5) instead: blocks of 32 along H, one power-of-two scale
 *               per block (tokens per row, the weight per (expert, column)), see
 *               hmm_quant_rows_mx; the block exponents feed the scaled FP8
 *               matrix instruction directly.  H a multiple of 128.
 *               HMM_FP8_E4M3_GROUP: the per-group quantisation of
 *               MoeDistributeDispatchV2 case 4 (see hmm_quant_rows_group): each
 *               128-deep group's E4M3 sums are scaled by its token and weight
 *               descales and added in group order.  The up-projection runs on
 *               64-row tiles only; with 256-row tiles for the other products a
 *               second routing pass writes its tile table into the forward
 *               workspace.  H a multiple of 128.
 *   flags       HMM_FLAG_* bits; a backward takes the same value as its forward.
 *   shared_I    0, or the intermediate size Is of a shared expert (a multiple of
 *               64 in [64, 65536]): then the calls are hmm_forward_shared and
 *               hmm_backward_shared, which take its weights. */
typedef struct hmm_problem {
  int64_t T, H, I, E, K;
  int32_t out_dtype;
  int32_t gmm1_dtype;
  uint32_t flags;
  uint32_t shared_I;
} hmm_problem;

/* Byte offsets of the arrays a forward call records in ``saved`` (for tests
 * and tools; the backward reads them).  S = T*K.
 *   counts[E] int32      tokens per expert (the per-expert histogram)
 *   offsets[E+1] int32   exclusive prefix sum of counts; offsets[E] = S
 *   sorted_slot[S] int32 slot (t*K+k) placed at permuted row p; slots of one
 *                        expert are contiguous and in ascending slot order
 *   row_of_slot[S] int32 inverse of sorted_slot (-1 for a dropped slot)
 *   tok_of_row[S] int32  token of permuted row p (sorted_slot[p] / K)
 *   tiles                int32 tile tables of the grouped products
 *   h[S,2I] bf16         up-projection output per permuted row ([gate | up])
 *   a[S,I] bf16          SwiGLU output per permuted row
 *   aw[S,I] bf16         topk weight * a, the W2-gradient operand
 *                        (out_dtype HMM_F32: h is float32 [S,2I]; a and aw are
 *                        bf16 [S,2I] holding hi in columns [0,I), lo in [I,2I))
 *   id_error int32       1 if an id was out of range on the recording call
 * With a shared expert (shared_I = Is > 0; all of these are empty without one):
 *   shared_offsets[2] int32  {0, T}: one group holding every token
 *   shared_idx[T] int32      0 .. T-1 (the group's rows are the tokens in order)
 *   shared_ones[T] float32   1.0, the shared expert's combine weight
 *   shared_tiles             int32 tile table of that group
 *   shared_h[T,2Is] bf16     the shared up-projection output ([gate | up])
 *   shared_a[T,Is] bf16      the shared SwiGLU output
 *                            (HMM_F32: shared_h float32 [T,2Is], shared_a bf16
 *                            [T,2Is] as hi | lo) */
typedef struct hmm_saved_layout {
  size_t counts, offsets, sorted_slot, row_of_slot, tok_of_row, tiles, h, a, aw, id_error;
  size_t shared_offsets, shared_idx, shared_ones, shared_tiles, shared_h, shared_a;
  size_t total;
} hmm_saved_layout;

/* Sizes of the forward's workspace and saved buffers for ``p`` (bytes). */
hmm_status hmm_forward_sizes(const hmm_problem* p, size_t* workspace_bytes, size_t* saved_bytes);

/* Byte offsets of the arrays inside ``saved``. */
hmm_status hmm_saved_layout_of(const hmm_problem* p, hmm_saved_layout* out);

/* Forward (RFC section 2.1: Dispatch -> GMM1 -> SwiGLU -> GMM2 -> Combine).
 *   x             bf16 [T,H]       tokens of this device
 *   topk_ids      int32 [T,K]      global expert ids (here: 0 <= id < E)
 *   topk_weights  float32 [T,K]    routing weights
 *   up_w          bf16 [E,H,2I]    up_proj_weight; columns [0,I) gate, [I,2I) up
 *   down_w        bf16 [E,I,H]     down_proj_weight
 *   y             bf16 [T,H]       output (overwritten; float32 with HMM_F32)
 *   saved         forward_sizes' saved_bytes; filled for the backward, must
 *                 stay untouched until the matching backward has run
 *   workspace     forward_sizes' workspace_bytes of scratch (free after the
 *                 call has executed on the stream)
 * On HMM_ERR_EXPERT_ID_OUT_OF_RANGE (with HMM_FLAG_VALIDATE_IDS) the contents
 * of y and saved are unspecified.  Needs p->shared_I == 0 (else
 * HMM_ERR_BAD_SHAPE: use hmm_forward_shared). */
hmm_status hmm_forward(const hmm_problem* p, const void* x, const int32_t* topk_ids,
                       const float* topk_weights, const void* up_w, const void* down_w, void* y,
                       void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                       void* stream);

/* hmm_forward without a workspace argument, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same problem, inputs, outputs and
 * saved buffer as hmm_forward (same kernels, identical results); the forward
 * workspace comes from a device array inside the library instead.
 * - That array holds 64 MiB (67108864 bytes).  It is allocated when the library
 *   is loaded on a device (one copy per device, kept until the process ends)
 *   and is never freed.  A problem whose hmm_forward_sizes workspace exceeds it
 *   returns HMM_ERR_WORKSPACE_TOO_SMALL before any HIP call.  Routed problems
 *   need about S*H*2 bytes, plus small routing tables.  For example, T=256 and K=8
 *   at H=7168 fit, and T=4000, H=2048, K=8 does not (131 MB).
 * - The call allocates no device or pinned host memory and creates no HIP
 *   object (no hipMalloc, hipFree, hipHostMalloc or event creation); stage
 *   timing is paused during it.  So it takes
 *   neither HMM_FLAG_VALIDATE_IDS nor HMM_FLAG_FUSED_FORWARD (HMM_ERR_UNSUPPORTED):
 *   invalid ids are dropped and flagged in ``saved`` instead.  No shared expert.
 * - Nothing in the array has to start at any value: every call writes what it
 *   later reads.  The array keeps the last call's contents.
 * - All calls on one device share the one array: calls that overlap in time
 *   on a device (several streams, or host threads) race on it and must be
 *   ordered by the caller. */
hmm_status hmm_forward_noalloc(const hmm_problem* p, const void* x, const int32_t* topk_ids,
                               const float* topk_weights, const void* up_proj_weight,
                               const void* down_proj_weight, void* y, void* saved, size_t saved_bytes,
                               void* stream);

/* Forward with a shared expert (RFC section 6.1: a shared expert fused into the
 * same pipeline, its output merged at the Combine).  Every token also goes
 * through one dense SwiGLU FFN of intermediate size Is = p->shared_I:
 *   [gs|us] = x[t] . shared_up_w;  as = silu(gs) * us;  os = as . shared_down_w;
 *   y[t] = sum_k topk_weights[t,k] * o_k  +  os,
 * the shared term added last, in the same float32 sum, before the one rounding
 * of y.  Its products run on the same kernels as the routed experts' (as one
 * more group of all T tokens; bf16 also when gmm1_dtype is FP8).
 *   shared_up_w    bf16 [H,2Is]   columns [0,Is) gate, [Is,2Is) up
 *   shared_down_w  bf16 [Is,H]
 * The other arguments are those of hmm_forward; the sizes come from
 * hmm_forward_sizes of the same problem.  With p->shared_I == 0 this is
 * hmm_forward (the shared pointers are ignored). */
hmm_status hmm_forward_shared(const hmm_problem* p, const void* x, const int32_t* topk_ids,
                              const float* topk_weights, const void* up_w, const void* down_w,
                              const void* shared_up_w, const void* shared_down_w, void* y, void* saved,
                              size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the backward's workspace (bytes). */
hmm_status hmm_backward_sizes(const hmm_problem* p, size_t* workspace_bytes);

/* Backward (RFC section 2.2: Dispatch(dY) -> act_grad (dY . W2^T) -> SwiGLUGrad
 * -> input_grad GMM -> Combine(dX); W2Grad and W1Grad GMMs; d_topk_weights).
 *   dy              bf16 [T,H]       gradient of y (float32 with HMM_F32)
 *   x, topk_ids, topk_weights, up_w, down_w   the forward's inputs (topk_ids
 *                   is only shape-checked: the routing recorded in ``saved``
 *                   is used)
 *   saved           the buffer filled by the matching forward
 *   dx              bf16 [T,H]       overwritten
 *   d_up_w          bf16 [E,H,2I]    overwritten (experts without tokens: zeros)
 *   d_down_w        bf16 [E,I,H]     overwritten (experts without tokens: zeros)
 *                   (dx, d_up_w and d_down_w are float32 with HMM_F32)
 *   d_topk_weights  float32 [T,K]    overwritten (0 for dropped slots)
 * Needs p->shared_I == 0 (else HMM_ERR_BAD_SHAPE: use hmm_backward_shared). */
hmm_status hmm_backward(const hmm_problem* p, const void* dy, const void* x, const int32_t* topk_ids,
                        const float* topk_weights, const void* up_w, const void* down_w,
                        const void* saved, size_t saved_bytes, void* dx, void* d_up_w, void* d_down_w,
                        float* d_topk_weights, void* workspace, size_t workspace_bytes, void* stream);

/* Backward with a shared expert: hmm_backward's outputs, plus
 *   d_shared_up_w    bf16 [H,2Is]   overwritten (zeros for T = 0)
 *   d_shared_down_w  bf16 [Is,H]    overwritten
 *                    (float32 with HMM_F32)
 * and dx then also holds the shared expert's term (added after the K routed
 * terms, in the same float32 sum).  ``saved`` is the buffer filled by the
 * matching hmm_forward_shared.  With p->shared_I == 0 this is hmm_backward. */
hmm_status hmm_backward_shared(const hmm_problem* p, const void* dy, const void* x, const int32_t* topk_ids,
                               const float* topk_weights, const void* up_w, const void* down_w,
                               const void* shared_up_w, const void* shared_down_w, const void* saved,
                               size_t saved_bytes, void* dx, void* d_up_w, void* d_down_w, void* d_shared_up_w,
                               void* d_shared_down_w, float* d_topk_weights, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Routing alone (RFC section 4.1 top-k expand; 3.1 offset construction; 6.2
 * sort by expert): writes counts[E], offsets[E+1], sorted_slot[S] and
 * row_of_slot[S] (int32 device arrays) as described for hmm_saved_layout.
 * ``workspace`` needs hmm_route_workspace_size bytes.  With
 * HMM_FLAG_VALIDATE_IDS an out-of-range id returns
 * HMM_ERR_EXPERT_ID_OUT_OF_RANGE after the routing has been written. */
hmm_status hmm_route_workspace_size(const hmm_problem* p, size_t* workspace_bytes);
hmm_status hmm_route(const hmm_problem* p, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                     int32_t* sorted_slot, int32_t* row_of_slot, void* workspace, size_t workspace_bytes,
                     void* stream);

/* FP8 E4M3 quantisation stages of the FP8 up-projection, exported for tests
 * and tools (hmm_forward runs the same kernels internally).  Per-token dynamic
 * quantisation as in MoeDistributeDispatchV2 (function description, case 3):
 * in float32, scale = 448 / max|row| (1 for an all-zero row), the code is the
 * round-to-nearest-even E4M3 (OCP e4m3fn) cast of value * scale, and the
 * stored factor is descale = 1 / scale.
 *   hmm_quant_rows_fp8: x bf16 [T,H] -> xq [T,H] E4M3 bytes, descale [T] f32.
 *   hmm_quant_cols_fp8: w bf16 [E,H,N] -> wq [E,H,N] E4M3 bytes, descale [E,N]
 *                       f32, one scale per (expert, column), the maximum taken
 *                       over H; needs hmm_quant_cols_workspace_size bytes of
 *                       workspace (column maxima per chunk of 256 rows).
 * T >= 0, E >= 1; H and N multiples of 8, positive, N <= 2^24 (else
 * HMM_ERR_UNSUPPORTED); all arrays below 4 GiB.
 * Pointers are device pointers, 16-byte aligned, caller-owned; errors as for
 * every other call, checked before any launch. */
hmm_status hmm_quant_rows_fp8(const void* x, int64_t T, int64_t H, uint8_t* xq, float* descale, void* stream);
hmm_status hmm_quant_cols_workspace_size(int64_t E, int64_t H, int64_t N, size_t* workspace_bytes);
hmm_status hmm_quant_cols_fp8(const void* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, float* descale,
                              void* workspace, size_t workspace_bytes, void* stream);

/* MX quantisation stages (MoeDistributeDispatchV2 case 5, quantMode 4), exported
 * for tests and tools (hmm_forward runs the same kernels with HMM_MXFP8_E4M3).
 * Per block of 32 consecutive elements along H: e = floor(log2 max|v|) - 8 (8 is
 * the exponent of E4M3's largest value, 448), clamped to [-127, 127] (-127 for an
 * all-zero block); code = round-to-nearest-even E4M3 of v * 2^-e saturated at
 * +-448; the block's E8M0 byte is e + 127, and v ~ code * 2^e.
 *   hmm_quant_rows_mx: x bf16 [T,H] -> xq [T,H] E4M3 bytes, xs [T,H/32] E8M0 bytes.
 *   hmm_quant_cols_mx: w bf16 [E,H,N] -> wq [E,H,N] E4M3 bytes, ws [E,N,H/32] E8M0
 *                      bytes (blocks of 32 rows of one column; column-major
 *                      exponents so a column's blocks are contiguous).
 * H a multiple of 32, N of 8 and at most 2^24; arrays below 4 GiB; device pointers,
 * 16-byte aligned. */
hmm_status hmm_quant_rows_mx(const void* x, int64_t T, int64_t H, uint8_t* xq, uint8_t* xs, void* stream);
hmm_status hmm_quant_cols_mx(const void* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, uint8_t* ws, void* stream);

/* Per-group dynamic quantisation, MoeDistributeDispatchV2, function description,
 * case 4 (quantMode 3): case 3's rule over groups of 128 consecutive hidden
 * elements (the page gives no group size): scale = 448 / max|group| in float32
 * (1 for an all-zero group), code = round-to-nearest-even E4M3 of v * scale,
 * and the float32 descale 1 / scale is kept.  The weight gets the rule per
 * (expert, column, block of 128 rows), so each group of the contraction has one
 * token descale and one weight descale per column.
 *   hmm_quant_rows_group: x bf16 [T,H] -> xq [T,H] E4M3 bytes, dsx [T,H/128] float32.
 *   hmm_quant_cols_group: w bf16 [E,H,N] -> wq [E,H,N] E4M3 bytes, dsw [E,H/128,N] float32.
 * H a multiple of 128, N of 8 and at most 2^24; arrays below 4 GiB; device pointers,
 * 16-byte aligned; T = 0 is a no-op.  hmm_forward runs the same kernels with
 * gmm1_dtype HMM_FP8_E4M3_GROUP. */
hmm_status hmm_quant_rows_group(const void* x, int64_t T, int64_t H, uint8_t* xq, float* dsx, void* stream);
hmm_status hmm_quant_cols_group(const void* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, float* dsw,
                                void* stream);

/* Names of statuses, and the calling thread's last error text. */
const char* hmm_status_string(hmm_status s);
const char* hmm_last_error_message(void);

/* Build identification: the offload target the kernels were compiled for. */
const char* hmm_build_info(void);

/* Test and diagnosis hook: the number of polls after which a wait of the fused
 * forward (HMM_FLAG_FUSED_FORWARD) gives up, for the launches that follow on
 * any thread; 0 restores the default (about a second).  A small value makes the
 * waits give up on purpose, so the error path can be exercised with every
 * workgroup still ending normally.  Not for concurrent use with forwards in
 * flight. */
hmm_status hmm_set_fused_spin_limit(uint32_t polls);

/* Stage timing, for benchmarks and tools.  While enabled on the calling
 * thread, every kernel launch (and the id read-back) of hmm_forward,
 * hmm_backward and hmm_route is bracketed by two HIP events recorded on the
 * call's stream, so the timings cover exactly that stage as it ran in the
 * stream.  hmm_profile_read waits for the recorded events and returns, per
 * stage name, the number of launches and their summed device time; it then
 * clears the record.  Events are created on first use (at most 16384 per
 * thread; beyond that further launches are not timed and ``dropped`` counts
 * them).  Enabling costs two event records per launch; disabled, nothing. */
typedef struct hmm_stage_time {
  char name[32];
  int32_t launches;
  double ms;
} hmm_stage_time;
hmm_status hmm_profile_enable(int32_t on);
hmm_status hmm_profile_read(hmm_stage_time* out, int32_t max_stages, int32_t* n_stages, int32_t* dropped);

#ifdef __cplusplus
}
#endif

#endif /* HMM_H */
