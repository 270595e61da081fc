// Policies of the bf16 products (what A and B are, how their tiles are
// addressed, what the epilogue does), for gemm_core.h's main loop: the
// row-grouped up-projection + SwiGLU, down-projection, act_grad + SwiGLUGrad and
// input_grad, and the two weight gradients.  Included by the launchers
// (gemm.hip) and by the fused small-problem kernels (fused.hip).
#pragma once

#include "gemm_core.h"

namespace hmm {
namespace {

// ------------------------------------------------------------- gmm1 + SwiGLU
template <class Cc, bool SMALL>
struct Gmm1 : RowTile<Cc, SMALL> {
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::nt;
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  struct Args {
    RowGroups g;
    const uint16_t* x;
    const uint16_t* w1;
    const float* tw;
    int64_t T, H, I;
    uint16_t *h, *a, *aw;  // aw may be NULL (not stored)
    int n_ntiles;
    bool coh = false;  // ``a`` goes to the coherence point (read by another XCD in the same launch)
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  int i0;
  // the B tile holds BN/2 gate columns then the BN/2 matching up columns; the
  // epilogue pairs them through LDS
  __device__ static __forceinline__ int ncol0(int wn, int nb) { return wn * C::TN + nb * 32; }
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    i0 = nt * (C::BN / 2);
    ra_ = make_rsrc(A.x, A.T * A.H * 2);
    this->template a_rows<true>(A.g, A.H, aoff);
    init_b(A);
    return true;
  }
  // the weight side of tile (e, nt): its resource, the offsets of the tile's gate
  // and up columns, and the K steps
  __device__ __forceinline__ void init_b(const Args& A) {
    rb_ = make_rsrc(A.w1 + (int64_t)e * A.H * 2 * A.I, A.H * 2 * A.I * 2);
    const int tid = threadIdx.x;
    constexpr int CPR = C::BN / 8, HALF = C::BN / 16;
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, c8 = c % CPR;
      const int64_t gi = min((int64_t)(i0 + (c8 % HALF) * 8), A.I - 8);   // gate column (clamped)
      const int64_t col = (c8 < HALF) ? gi : A.I + gi;
      boff[i] = (uint32_t)((kr * 2 * A.I + col) * 2);
    }
    nk = (int)(A.H / C::BK);
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(kt * C::BK * 2 * ar->I * 2);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }
  // g and u (rounded to bf16) are staged in LDS as the [BM][BN] tile (gate
  // columns first); then each thread takes 8 consecutive columns of one row and
  // writes h (both halves), a = bf16(silu(g) u) and aw = bf16(w a) as 16-byte chunks.
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    constexpr int LD = C::BN + 8;
    static_assert(C::BM * LD * 2 + C::BM * 4 <= 2 * C::STAGE * 2, "staging must fit in the LDS buffers");
    float* wrow = reinterpret_cast<float*>(smem + C::BM * LD);
    const int tid = threadIdx.x;
    for (int t = tid; t < C::BM; t += C::NTHR)
      wrow[t] = this->row_weight(ar->tw, ar->g, t);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          smem[acc_row<C>(wm, mb, r, lane) * LD + ncol0(wn, nb) + (lane & 31)] = f2bf(acc[mb][nb][r]);
    __syncthreads();
    const int64_t I = ar->I;
    constexpr int CPR = C::BN / 16;  // 8-column chunks of the gate half
    for (int c = tid; c < C::BM * CPR; c += C::NTHR) {
      const int row = c / CPR, c8 = c % CPR;
      const int64_t i = i0 + c8 * 8;
      if (row >= rows || i >= I) continue;
      const int64_t p = row0 + row;
      const u32x4 gv = *reinterpret_cast<const u32x4*>(smem + row * LD + c8 * 8);
      const u32x4 uv = *reinterpret_cast<const u32x4*>(smem + row * LD + C::BN / 2 + c8 * 8);
      float g[8], u[8], av[8], aw[8];
      unpack8(gv, g);
      unpack8(uv, u);
      const float w = wrow[row];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[j] = round_bf(g[j] * sigmoidf_(g[j]) * u[j]);
        aw[j] = w * av[j];
      }
      store16_stream(ar->h + p * 2 * I + i, gv);
      store16_stream(ar->h + p * 2 * I + I + i, uv);
      put16(ar->a, ar->g.S * I * 2, p * I + i, pack8(av), ar->coh);
      if (ar->aw) store16_stream(ar->aw + p * I + i, pack8(aw));
    }
  }
};

// ------------------------------------------------------------- gmm2
// COH_A: ``a`` was written in the same launch (the fused forward): read it at
// the coherence point.  A template parameter, so the main loop has no branch.
template <class Cc, bool SMALL, bool COH_A = false>
struct Gmm2 : RowTile<Cc, SMALL>, PlainCols<Cc> {
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::n0;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  struct Args {
    RowGroups g;
    const uint16_t* a;
    const uint16_t* w2;
    int64_t S, H, I;
    uint16_t* o;
    int n_ntiles;
    bool coh = false;  // ``o`` goes to the coherence point (read by another XCD in the same launch)
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.a, A.S * A.I * 2);
    this->template a_rows<false>(A.g, A.I, aoff);
    rb_ = make_rsrc(A.w2 + (int64_t)e * A.I * A.H, A.I * A.H * 2);
    const int tid = threadIdx.x;
    constexpr int CPR = C::BN / 8;
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, c8 = c % CPR;
      const int64_t col = min((int64_t)(n0 + c8 * 8), A.H - 8);
      boff[i] = (uint32_t)((kr * A.H + col) * 2);
    }
    nk = (int)(A.I / C::BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
    if constexpr (COH_A) {
#pragma unroll
      for (int i = 0; i < C::CA; ++i) r[i] = bload_coh(ra_, aoff[i], kt * C::BK * 2);
    } else {
#pragma unroll
      for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
    }
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(kt * C::BK * ar->H * 2);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    store_tile<C, Gmm2>(acc, wm, wn, lane, smem, ar->o, ar->H, row0, rows, n0, ar->H, ar->coh, ar->S);
  }
};

// ------------------------------------------------------------- act_grad + SwiGLUGrad
template <class Cc, bool SMALL>
struct ActGrad : RowTile<Cc, SMALL>, PlainCols<Cc> {
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::n0; using B_::nt;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  struct Args {
    RowGroups g;
    const uint16_t* dy;
    const uint16_t* w2;
    const float* tw;
    const uint16_t* h;
    int64_t T, H, I;
    uint16_t* dh;
    float* dwpart;  // may be NULL (the sums are not stored)
    int dw_cols;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.dy, A.T * A.H * 2);
    this->template a_rows<true>(A.g, A.H, aoff);
    rb_ = make_rsrc(A.w2 + (int64_t)e * A.I * A.H, A.I * A.H * 2);
    this->b_rows(A.H, A.I, boff);
    nk = (int)(A.H / C::BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    static_assert((sgrad_lds_floats<C>() + C::BM) * 4 <= 2 * C::STAGE * 2, "staging must fit in the LDS buffers");
    float* gst = reinterpret_cast<float*>(smem);
    float* wrow = gst + sgrad_lds_floats<C>();
    for (int t = threadIdx.x; t < C::BM; t += C::NTHR)
      wrow[t] = this->row_weight(ar->tw, ar->g, t);
    swiglu_grad_epilogue<C>(acc, wm, wn, lane, gst, wrow, rows, row0, n0, ar->I, ar->h, ar->dh, ar->dwpart,
                            ar->dw_cols);
  }
};

// ------------------------------------------------------------- input_grad
template <class Cc, bool SMALL>
struct InputGrad : RowTile<Cc, SMALL>, PlainCols<Cc> {
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::n0;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  struct Args {
    RowGroups g;
    const uint16_t* dh;
    const uint16_t* w1;
    int64_t S, H, I;
    uint16_t* dxp;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.dh, A.S * 2 * A.I * 2);
    this->template a_rows<false>(A.g, 2 * A.I, aoff);
    rb_ = make_rsrc(A.w1 + (int64_t)e * A.H * 2 * A.I, A.H * 2 * A.I * 2);
    this->b_rows(2 * A.I, A.H, boff);
    nk = (int)(2 * A.I / C::BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    store_tile<C, InputGrad>(acc, wm, wn, lane, smem, ar->dxp, ar->H, row0, rows, n0, ar->H);
  }
};

// ------------------------------------------------------------- weight gradients
// C[e][m][n] = sum over the expert's rows p of A[p][m] * B[p][n]; both operands
// are read along their row (m or n contiguous) and transposed by the LDS read.
template <class Cc, bool GATHER_A, bool GATHER_B>
struct Dw : PlainCols<Cc> {
  typedef Cc C;
  static constexpr bool SCHED_HINT = false;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = false, B_KMAJ = false;
  struct Args {
    const int32_t* offsets;
    const int32_t* tok_of_row;
    int64_t E;
    const uint16_t* A;  // [rows or tokens][M]
    const uint16_t* B;  // [rows or tokens][N]
    int64_t a_rows, b_rows;  // rows held by A and B
    int64_t M, N;
    uint16_t* Cout;     // [E][M][N]
    int mt, nt;
    const int32_t* order;  // [E] launch order of the experts, or NULL (0, 1, ...)
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  int e, m0, n0, nk, p0, p1;
  // byte offsets of the rows of the next step to be loaded (computed by index())
  uint32_t rowoff_a[C::CA], rowoff_b[C::CB];
  // row indices of a step of the gathered operand(s), as fetched
  struct Raw {
    int32_t a[GATHER_A ? C::CA : 1], b[GATHER_B ? C::CB : 1];
  };
  // The cost of a tile grows with its expert's row count, so every XCD gets an
  // equal slice of every expert's tiles (not a contiguous run of experts): XCD x
  // (workgroups b with b % 8 == x) walks the experts in launch order (``order``:
  // longest reductions first, so the largest expert's tiles do not end the
  // launch alone) and takes tiles [x * per, (x + 1) * per) of each, per =
  // ceil(mt * nt / 8); inside a slice the tiles are rasterised in groups of
  // GROUP_M row tiles.
  __device__ __forceinline__ bool init(const Args& A, int b) {
    ar = &A;
    const int per_e = A.mt * A.nt;
    const int per = (per_e + 7) / 8;
    const int j = b >> 3;
    const int rank = j / per;
    if (rank >= A.E) return false;
    e = A.order ? A.order[rank] : rank;
    const int t = (b & 7) * per + (j - rank * per);
    if (t >= per_e) return false;
    int r, c;
    raster(t, A.mt, A.nt, r, c);
    m0 = r * C::BM;
    n0 = c * C::BN;
    p0 = A.offsets[e];
    p1 = A.offsets[e + 1];
    nk = (p1 - p0 + C::BK - 1) / C::BK;
    ra_ = make_rsrc(A.A, A.a_rows * A.M * 2);
    rb_ = make_rsrc(A.B, A.b_rows * A.N * 2);
    return true;
  }
  // Loads of the token index of every row this thread will read in step kt
  // (rows past the expert's end load its last row's index, unused).
  template <int R, int CN>
  __device__ __forceinline__ void fetch_rows(int kt, int32_t (&raw)[CN]) {
    const int tid = threadIdx.x;
    constexpr int CPR = R / 8;
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const int p = min(p0 + kt * C::BK + (tid + i * C::NTHR) / CPR, p1 - 1);
      raw[i] = ar->tok_of_row[p];
    }
  }
  __device__ __forceinline__ void fetch(int kt, Raw& r) {
    if constexpr (GATHER_A) fetch_rows<C::BM>(kt, r.a);
    if constexpr (GATHER_B) fetch_rows<C::BN>(kt, r.b);
  }
  // row part of the offsets of step kt: rows p past the expert's end and columns
  // past the matrix get the resource's end (reads zeros)
  template <bool GATHER, int R, int CN, int CR>
  __device__ __forceinline__ void rows_of(int64_t nrows, int64_t ld, int64_t c0, int kt, const int32_t (&raw)[CR],
                                          uint32_t (&ro)[CN]) {
    const int tid = threadIdx.x;
    constexpr int CPR = R / 8;
    const uint32_t end = (uint32_t)(nrows * ld * 2);
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, c8 = c % CPR;
      const int p = p0 + kt * C::BK + kr;
      const uint32_t col = (uint32_t)c0 + c8 * 8;  // every offset fits 32 bits (resources < 4 GiB)
      uint32_t row = (uint32_t)p;
      if constexpr (GATHER) row = (uint32_t)raw[i];
      ro[i] = (p < p1 && col < (uint32_t)ld) ? (row * (uint32_t)ld + col) * 2u : end;
    }
  }
  __device__ __forceinline__ void index(int kt, const Raw& r) {
    rows_of<GATHER_A, C::BM, C::CA>(ar->a_rows, ar->M, m0, kt, r.a, rowoff_a);
    rows_of<GATHER_B, C::BN, C::CB>(ar->b_rows, ar->N, n0, kt, r.b, rowoff_b);
  }
  __device__ __forceinline__ void load_a(int, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, rowoff_a[i], 0);
  }
  __device__ __forceinline__ void load_b(int, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, rowoff_b[i], 0);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    store_tile<C, Dw>(acc, wm, wn, lane, smem, ar->Cout + (int64_t)e * ar->M * ar->N, ar->N, m0,
                      (int)min((int64_t)C::BM, ar->M - m0), n0, ar->N);
  }
};

}  // namespace
}  // namespace hmm
