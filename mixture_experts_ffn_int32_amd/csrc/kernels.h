// Launchers of the libhmm kernels (host-callable), and the constants the host
// planner shares with them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hmm {

constexpr int MAX_EXPERTS = 1024;     // E limit (the dispatch op's moeExpertNum bound)
constexpr int RT_THREADS = 256;       // routing block size
constexpr int RT_SLOTS = 1024;        // slots per routing block
constexpr int RT_SCAN_THREADS = 1024; // the single scan block (>= MAX_EXPERTS)
constexpr int RT_ONE_THREADS = 1024;  // one-workgroup routing of small problems
constexpr int RT_ONE_MAX_SLOTS = 8192;
constexpr int RT_ONE_MAX_EXPERTS = 256;

constexpr int TILE_BIG = 256;         // rows of a big row-grouped product tile
constexpr int TILE_SMALL = 64;        // rows of a small tile (expert remainders, small experts)
// A tile table entry is two int32 words: (expert | rows << 16, first row).  The
// tile's row count rides with its expert id (E <= 1024, rows <= 256), so a
// product reads one entry and not also the expert's end in the offsets array: a
// dependent load fewer before its first data load.
__host__ __device__ inline int32_t tile_word(int e, int rows) { return (int32_t)(e | (rows << 16)); }
__host__ __device__ inline int tile_expert(int32_t w) { return w & 0xffff; }
__host__ __device__ inline int tile_rows(int32_t w) { return (int)((uint32_t)w >> 16); }

// Upper bounds of the tile-table lengths for S routed rows over E experts.
// An expert with c rows gets floor(c/256) big tiles, one more if the remainder
// r = c mod 256 exceeds 128 rows, else ceil(r/64) <= 2 small tiles.  So
// #big <= sum_e (c_e + 127) / 256 <= (S + 127 E) / 256, and, since ceil(r/64)
// <= 1 + (r - 1)/64 for r > 0 and at most min(E, S) experts have rows,
// #small <= min(2 E, min(E, S) + S / 64).
// Small problems (few big tiles for the whole chip) use only TILE_SMALL-row tiles
// and narrow 64x64 product tiles; then #small = sum_e ceil(c_e / 64) <=
// (S + 63 min(E, S)) / 64.
inline bool small_mode(int64_t S, int64_t H, int64_t I) {
  const int64_t n = (H > 2 * I ? H : 2 * I);
  return ((S + TILE_BIG - 1) / TILE_BIG) * ((n + 255) / 256) < 256;
}
inline int64_t max_big_tiles(int64_t S, int64_t E, bool small) {
  return small ? 0 : (S + (TILE_BIG / 2 - 1) * E) / TILE_BIG;
}
inline int64_t max_small_tiles(int64_t S, int64_t E, bool small) {
  const int64_t ne = E < S ? E : S;
  if (small) return (S + (TILE_SMALL - 1) * ne) / TILE_SMALL;
  const int64_t a = 2 * E, b = ne + S / TILE_SMALL;
  return a < b ? a : b;
}
inline int64_t tile_table_ints(int64_t S, int64_t E, bool small) {
  return 4 + 2 * (max_big_tiles(S, E, small) + max_small_tiles(S, E, small));
}

// The shared expert's routing tables: one expert holding all T tokens in token
// order: offsets[2] = {0, T}, idx[T] = 0..T-1 (its sorted_slot and tok_of_row),
// ones[T] = 1.0 (its weights) and tiles (tile_table_ints(T, 1, !big_on)).  The
// routing launch writes them too when idx is not NULL.
struct SharedTables {
  int64_t T;
  int max_big, big_on;
  int32_t* offsets;
  int32_t* idx;
  float* ones;
  int32_t* tiles;
};

// routing (route.hip)
hipError_t launch_route(const int32_t* ids, int64_t S, int E, int K, int max_big, int big_on, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slot, int32_t* row_of_slot, int32_t* tok_of_row,
                        int32_t* tiles, int32_t* err, int32_t* blockhist, int32_t* blockbase, int32_t* blockerr,
                        int32_t* host_err, const SharedTables& shared, hipStream_t stream);

// grouped products (gemm.hip).  All matrices bf16 (uint16_t storage).
struct RowGroups {
  const int32_t* tiles;        // tile table written by route_scan (layout in route.hip)
  const int32_t* offsets;      // [E+1]
  const int32_t* sorted_slot;  // [S] slot of permuted row p
  const int32_t* tok_of_row;   // [S] token of permuted row p (= sorted_slot[p] / K)
  int64_t max_big, max_small;  // table capacities
  int64_t T, S;                // tokens, routed rows (extents of the buffer resources)
  bool narrow;                 // small-problem mode: 64x64 tiles over the small table only
  bool coh = false;            // the arrays above were written in the same launch (fused
                               // kernel): read them at the device-wide coherence point
};

// Every bf16 product launcher takes n = 1 or 2 jobs: the routed experts and,
// second, the shared expert (its own groups, width and weights); the jobs share
// each launch (co-scheduled), and take the tiling mode of the first job.
//
// h = x[tok] . W1[e] (gate|up), a = silu(g) u, aw = w a       (forward up-projection + SwiGLU)
struct Gmm1Job {
  RowGroups g;
  const uint16_t* x;
  const uint16_t* w1;
  const float* tw;
  int64_t H, I;
  uint16_t *h, *a, *aw;  // aw may be NULL (not stored)
};
hipError_t launch_gmm1_swiglu(const Gmm1Job* jobs, int n, hipStream_t stream);
// The routing and the up-projection in one launch, for small problems (S <=
// ROUTED_MAX_SLOTS, E <= RT_ONE_MAX_EXPERTS) on the narrow tiling, bf16, without
// a shared expert: every up-projection workgroup routes the ids itself as far as
// its own tile needs, and the launch stores every routing array launch_route
// stores (the later launches read them).
constexpr int ROUTED_MAX_SLOTS = 4096;
// ... and at most this many tiles in the launch (the table's capacity times the
// column tiles), one workgroup per CU: every workgroup pays a few microseconds
// for its routing, which the saved routing launch (about 7 us with its kernel
// boundary) covers only while the launch runs in one round.  Measured forwards:
// 140 and 188 tiles 2.7-3 us faster than with the routing launch, 508 the same,
// 760 and 1016 tiles 7-10 us slower.
constexpr int ROUTED_MAX_TILES = 256;
struct RoutedGmm1Job {
  Gmm1Job up;  // up.g: the narrow tables' capacities (its arrays are not read)
  const int32_t* ids;
  int E, K, max_big;
  int32_t *counts, *offsets, *sorted_slot, *row_of_slot, *tok_of_row, *tiles, *err, *host_err;
};
hipError_t launch_route_gmm1_swiglu(const RoutedGmm1Job& j, hipStream_t stream);
// o = a . W2[e]                                                (forward down-projection)
struct Gmm2Job {
  RowGroups g;
  const uint16_t* a;
  const uint16_t* w2;
  int64_t H, I;
  uint16_t* o;
};
hipError_t launch_gmm2(const Gmm2Job* jobs, int n, hipStream_t stream);
// G = dY[tok] . W2[e]^T; dH = SwiGLUGrad(w G); dwpart = partial sums of G a
struct ActGradJob {
  RowGroups g;
  const uint16_t* dy;
  const uint16_t* w2;
  const float* tw;
  const uint16_t* h;  // [S][2I]: g | u (a = bf16(silu(g) u) is recomputed from them)
  int64_t H, I;
  uint16_t* dh;
  float* dwpart;  // may be NULL (not stored)
  int dw_cols;
};
hipError_t launch_act_grad(const ActGradJob* jobs, int n, hipStream_t stream);
// dXp = dH . W1[e]^T
struct InputGradJob {
  RowGroups g;
  const uint16_t* dh;
  const uint16_t* w1;
  int64_t H, I;
  uint16_t* dxp;
};
hipError_t launch_input_grad(const InputGradJob* jobs, int n, hipStream_t stream);
// Weight gradients C[e] = sum over the expert's rows p of A[p]^T B[p]:
//   dW1[e] = sum_p x[tok(p)]^T dH[p]   (dw1_job; A gathered through tok_of_row)
//   dW2[e] = sum_p aw[p]^T dY[tok(p)]  (dw2_job; B gathered)
struct DwJob {
  const int32_t* offsets;     // [E+1]
  const int32_t* tok_of_row;  // [S]
  int64_t E;
  const uint16_t* A;
  const uint16_t* B;
  int64_t a_rows, b_rows, M, N;
  uint16_t* out;              // [E][M][N]
  const int32_t* order = nullptr;  // [E]: the experts in launch order (NULL: 0, 1, ...)
};
inline DwJob dw1_job(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                     const uint16_t* x, const uint16_t* dh, int64_t H, int64_t I, uint16_t* dw1) {
  return DwJob{offsets, tok_of_row, E, x, dh, T, S, H, 2 * I, dw1};
}
inline DwJob dw2_job(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                     const uint16_t* aw, const uint16_t* dy, int64_t H, int64_t I, uint16_t* dw2) {
  return DwJob{offsets, tok_of_row, E, aw, dy, S, T, I, H, dw2};
}
hipError_t launch_dw1(const DwJob* jobs, int n, bool narrow, hipStream_t stream);
// order[r] = the expert of rank r by descending row count (ties: lower id first),
// for the weight gradients to start the longest reductions first (route.hip)
hipError_t launch_expert_order(const int32_t* counts, int E, int32_t* order, hipStream_t stream);
hipError_t launch_dw2(const DwJob* jobs, int n, bool narrow, hipStream_t stream);
// Small problems (narrow tiles): the independent products share a launch,
// act_grad with W2Grad, then input_grad with W1Grad (the same products as above;
// with a shared expert, its two products join each launch).
hipError_t launch_act_grad_dw2_narrow(const ActGradJob* ag, const DwJob* dw2, int n, hipStream_t stream);
hipError_t launch_input_grad_dw1_narrow(const InputGradJob* ig, const DwJob* dw1, int n, hipStream_t stream);
// number of d_topk_weights partial columns written by launch_act_grad for a given I
int act_grad_dw_cols(int64_t I, bool narrow);

// FP8 E4M3 quantisation (quant.hip): per-token rows of x, per-(expert, column)
// columns of a weight [E][H][N]; descales are 1 / scale in float32.
hipError_t launch_quant_rows_fp8(const uint16_t* x, int64_t T, int64_t H, uint8_t* xq, float* dsx,
                                 hipStream_t stream);
int64_t quant_cols_chunks(int64_t H);  // pmax holds quant_cols_chunks(H) * E * N floats
hipError_t launch_quant_cols_fp8(const uint16_t* w, int64_t E, int64_t H, int64_t N, float* pmax, uint8_t* wq,
                                 float* dsw, hipStream_t stream);
// MX quantisation (quant.hip; MoeDistributeDispatchV2 case 5): blocks of 32
// along H, one E8M0 exponent byte per block; H a multiple of 32.
//   x [T][H] -> xq [T][H] E4M3, xs [T][H/32];  w [E][H][N] -> wq, ws [E][N][H/32]
hipError_t launch_quant_rows_mx(const uint16_t* x, int64_t T, int64_t H, uint8_t* xq, uint8_t* xs,
                                hipStream_t stream);
hipError_t launch_quant_cols_mx(const uint16_t* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, uint8_t* ws,
                                hipStream_t stream);
// Per-group quantisation (quant.hip; MoeDistributeDispatchV2 case 4): groups of
// 128 along H with a float32 scale each; H a multiple of 128.
//   x [T][H] -> xq [T][H] E4M3, dsx [T][H/128];  w [E][H][N] -> wq, dsw [E][H/128][N]
hipError_t launch_quant_rows_group(const uint16_t* x, int64_t T, int64_t H, uint8_t* xq, float* dsx,
                                   hipStream_t stream);
hipError_t launch_quant_cols_group(const uint16_t* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, float* dsw,
                                   hipStream_t stream);
// Per-group FP8 up-projection + SwiGLU (gemm_fp8.hip): each 128-deep K step's sums
// times dsx[tok][g] dsw[e][g][n], added in group order; 64x64 tiles only (narrow).
hipError_t launch_gmm1_group(const RowGroups& g, const uint8_t* xq, const float* dsx, const uint8_t* wq,
                             const float* dsw, const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                             uint16_t* aw, hipStream_t stream);
// MX up-projection + SwiGLU (gemm_fp8.hip): h = bf16(sum_k xq 2^xs . wq 2^ws) by the
// scaled instruction, then as launch_gmm1_swiglu.  H must be a multiple of 128.
hipError_t launch_gmm1_mx(const RowGroups& g, const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                          uint16_t* aw, hipStream_t stream);
// FP8 up-projection + SwiGLU (gemm_fp8.hip): h = bf16((xq[tok] . wq[e]) dsx[tok] dsw[e]), then as
// launch_gmm1_swiglu.  H must be a multiple of 128.
hipError_t launch_gmm1_fp8(const RowGroups& g, const uint8_t* xq, const float* dsx, const uint8_t* wq,
                           const float* dsw, const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                           uint16_t* aw, hipStream_t stream);

// FP8 backward (gemm_fp8.hip): the dX chain's products on E4M3 with per-row
// descales of both operands (codes from launch_quant_rows_fp8 on row views).
//   act_grad:   G = (dyq[tok] . w2q[e]^T) dsy[tok] dsw2[e][i], then the SwiGLUGrad
//               epilogue of launch_act_grad (dH, d_topk_weights partials);
//               dyq [T][H], w2q [E][I][H] (rows i), dsw2 [E][I]; H a multiple of 128
//   input_grad: dXp = bf16((dhq[p] . w1q[e]^T) dsh[p] dsw1[e][h]);
//               dhq [S][2I], w1q [E][H][2I] (rows h), dsw1 [E][H]
// Both on the tiling of ``g`` (256 + 64-row tiles, or 64x64 when narrow).
hipError_t launch_act_grad_fp8(const RowGroups& g, const uint8_t* dyq, const float* dsy, const uint8_t* w2q,
                               const float* dsw2, const float* topk_w, const uint16_t* h, int64_t H, int64_t I,
                               uint16_t* dh, float* dwpart, int dw_cols, hipStream_t stream);
hipError_t launch_input_grad_fp8(const RowGroups& g, const uint8_t* dhq, const float* dsh, const uint8_t* w1q,
                                 const float* dsw1, int64_t H, int64_t I, uint16_t* dxp, hipStream_t stream);

// pointwise (pointwise.hip).  ``extra`` [T][H] (may be NULL): the shared expert's rows,
// added with weight 1 after the K routed terms.
hipError_t launch_combine(const uint16_t* rows, const int32_t* row_of_slot, const float* topk_w, int64_t T,
                          int K, int64_t H, const uint16_t* extra, uint16_t* out, hipStream_t stream);
// combine(dX) (unweighted) with d_topk_weights[s] = sum_c dwpart[row_of_slot[s]][c] folded in
hipError_t launch_combine_dx(const uint16_t* rows, const int32_t* row_of_slot, int64_t T, int K, int64_t H,
                             const uint16_t* extra, uint16_t* dx, const float* dwpart, int dw_cols, float* dw,
                             hipStream_t stream);

// Fused small-problem forward (fused.hip): routing, up-projection + SwiGLU,
// down-projection and combine in one launch of at most max_groups workgroups
// (all resident), synchronised through fused_forward_sync_words(S, E) counters
// in ``sync`` that the call resets itself (epoch: a nonzero per-call value).
// Needs S <= RT_ONE_MAX_SLOTS, E <= RT_ONE_MAX_EXPERTS and the narrow tiling.
// A wait that gives up stores 1 into *host_status (pinned host memory the caller
// cleared) and that workgroup stops; set_fused_spin_cap sets the polls before a
// wait gives up for later launches (0: the default, about a second).
int64_t fused_forward_sync_words(int64_t S, int64_t E);
void set_fused_spin_cap(uint32_t polls);
hipError_t launch_fused_forward(const int32_t* ids, int64_t T, int64_t H, int64_t I, int E, int K, const uint16_t* x,
                                const uint16_t* w1, const uint16_t* w2, const float* topk_w, uint16_t* y,
                                int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* row_of_slot,
                                int32_t* tok_of_row, int32_t* tiles, int32_t* err, int32_t* host_err, uint16_t* h,
                                uint16_t* a, uint16_t* aw, uint16_t* o, uint32_t* sync, uint32_t epoch,
                                uint32_t* host_status, int max_groups, hipStream_t stream);

// float32-output (accuracy) mode (gemm_f32.hip, pointwise.hip).  Operands that are
// not exact bf16 inputs are bf16 [hi | lo] pairs of twice the width; see gemm_f32.hip.
hipError_t launch_gmm1_f32(const RowGroups& g, const uint16_t* x, const uint16_t* w1, const float* topk_w, int64_t H,
                           int64_t I, float* h, uint16_t* a2, uint16_t* aw2, hipStream_t stream);
hipError_t launch_gmm2_f32(const RowGroups& g, const uint16_t* a2, const uint16_t* w2, int64_t H, int64_t I, float* o,
                           hipStream_t stream);
hipError_t launch_act_grad_f32(const RowGroups& g, const uint16_t* dy2, const uint16_t* w2, const float* topk_w,
                               const float* h, const uint16_t* a2, int64_t H, int64_t I, uint16_t* dh2, float* dwpart,
                               int dw_cols, hipStream_t stream);
hipError_t launch_input_grad_f32(const RowGroups& g, const uint16_t* dh2, const uint16_t* w1, int64_t H, int64_t I,
                                 float* dxp, hipStream_t stream);
hipError_t launch_dw1_f32(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                          const uint16_t* x, const uint16_t* dh2, int64_t H, int64_t I, float* dw1, bool narrow,
                          hipStream_t stream);
hipError_t launch_dw2_f32(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                          const uint16_t* aw2, const uint16_t* dy2, int64_t H, int64_t I, float* dw2, bool narrow,
                          hipStream_t stream);
int act_grad_f32_dw_cols(int64_t I, bool narrow);  // d_topk_weights partial columns of launch_act_grad_f32
hipError_t launch_combine_f32(const float* rows, const int32_t* row_of_slot, const float* topk_w, int64_t T, int K,
                              int64_t H, const float* extra, float* out, hipStream_t stream);
hipError_t launch_combine_dx_f32(const float* rows, const int32_t* row_of_slot, int64_t T, int K, int64_t H,
                                 const float* extra, float* dx, const float* dwpart, int dw_cols, float* dw,
                                 hipStream_t stream);
// x float32 [n][H] -> bf16 [n][2H] = [hi | lo]
hipError_t launch_split_rows(const float* x, int64_t n, int64_t H, uint16_t* out, hipStream_t stream);

}  // namespace hmm
