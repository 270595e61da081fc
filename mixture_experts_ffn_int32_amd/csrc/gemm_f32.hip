// Products of the float32-output (accuracy) mode.
//
// The bf16 path rounds h, a, o, dH, dXp and the outputs to bf16 (about 3 decimal
// digits); the RFC's 1e-3 agreement with an unrounded computation (section 7.1)
// needs more.  Here every value that is not an exact bf16 input is carried in
// float32, and where such a value is a matrix operand it is split into two bf16
// parts, v = hi + lo with hi = bf16(v) and lo = bf16(v - hi) (about 16 bits of
// mantissa in all).  The split operand is stored as a bf16 matrix twice as wide
// ([hi | lo]), and the product runs over the doubled K while the other operand
// (an exact bf16 input) is read twice:
//   o     = [a_hi | a_lo] . [W2 ; W2]                  (K = 2I)
//   G     = [dY_hi | dY_lo] . [W2^T ; W2^T]            (K = 2H)
//   dXp   = [dH_hi | dH_lo] . [W1^T ; W1^T]            (K = 4I)
//   dW1   = x^T . dH_hi + x^T . dH_lo                  (two passes over the rows)
//   dW2   = aw_hi^T dY_hi + aw_hi^T dY_lo + aw_lo^T dY_hi   (three passes)
// The lo x lo term of dW2 is below float32 resolution of the result and is left
// out.  Accumulation is float32 in the MFMAs; results are stored as float32
// straight from the accumulators.  Same main loop, tile tables and tilings as
// the bf16 products, except that small problems use 64x64 tiles on two waves
// (each wave holding two 32-column blocks, which the up-projection's epilogue
// needs to see a gate column and its up column in one lane).
#include "gemm_core.h"

namespace hmm {
namespace {

typedef Cfg<64, 64, 2, 1> NarrowF;

__device__ __forceinline__ void split_bf(float v, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

// float32 results straight from the accumulators: for every accumulator register
// the 32 lanes of a half-wave write 32 consecutive floats of one row.
template <class C, class P>
__device__ __forceinline__ void store_acc_f32(const f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, float* out,
                                              int64_t ld, int64_t row_base, int valid_rows, int64_t col_base,
                                              int64_t ncols) {
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row<C>(wm, mb, r, lane);
        const int64_t col = col_base + P::ncol0(wn, nb) + (lane & 31);
        if (row < valid_rows && col < ncols) out[(row_base + row) * ld + col] = acc[mb][nb][r];
      }
}

// topk weight of each row of the tile, staged in LDS (the buffers are free after the main loop)
template <class C>
__device__ __forceinline__ float* stage_weights(const RowGroups& g, const float* tw, int row0, int rows, uint16_t* smem) {
  float* wrow = reinterpret_cast<float*>(smem);
  for (int t = threadIdx.x; t < C::BM; t += C::NTHR) wrow[t] = (t < rows) ? tw[g.sorted_slot[row0 + t]] : 0.f;
  __syncthreads();
  return wrow;
}

// ------------------------------------------------------------- up-projection + SwiGLU
// h = x[tok] . W1[e] kept in float32; a = silu(g) u and aw = w a stored as [hi | lo].
template <class Cc, bool SMALL>
struct Gmm1F32 : RowTile<Cc, SMALL> {
  static constexpr bool SCHED_HINT = false;
  static_assert(Cc::TN % 64 == 0, "every wave needs gate/up block pairs");
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
    float* h;       // [S][2I]
    uint16_t* a2;   // [S][2I]: a_hi | a_lo
    uint16_t* aw2;  // [S][2I]: aw_hi | aw_lo (may be NULL: not stored)
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  int i0;
  __device__ static __forceinline__ int ncol0(int wn, int nb) { return wn * C::TN + nb * 32; }
  // B tile: 32-column blocks alternate between gate and up columns of the same
  // intermediate columns: block b holds i0 + (b/2)*32 + [0, 32), gate if b is even
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    i0 = nt * (C::BN / 2);
    ra_ = make_rsrc(A.x, A.T * A.H * 2);
    this->template a_rows<true>(A.g, A.H, aoff);
    rb_ = make_rsrc(A.w1 + (int64_t)e * A.H * 2 * A.I, A.H * 2 * A.I * 2);
    const int tid = threadIdx.x;
    constexpr int CPR = C::BN / 8;
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, col_t = (c % CPR) * 8;
      const int b = col_t / 32;
      const int64_t gi = min((int64_t)(i0 + (b >> 1) * 32 + col_t % 32), A.I - 8);
      const int64_t col = (b & 1) ? A.I + gi : gi;
      boff[i] = (uint32_t)((kr * 2 * A.I + col) * 2);
    }
    nk = (int)(A.H / C::BK);
    return true;
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
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    const float* wrow = stage_weights<C>(ar->g, ar->tw, row0, rows, smem);
    const int64_t I = ar->I;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int j = 0; j < C::NB / 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row<C>(wm, mb, r, lane);
          const int64_t i = i0 + wn * (C::TN / 2) + j * 32 + (lane & 31);
          if (row >= rows || i >= I) continue;
          const int64_t p = row0 + row;
          const float g = acc[mb][2 * j][r], u = acc[mb][2 * j + 1][r];
          const float a = g * sigmoidf_(g) * u;
          const float aw = wrow[row] * a;
          ar->h[p * 2 * I + i] = g;
          ar->h[p * 2 * I + I + i] = u;
          uint16_t hi, lo;
          split_bf(a, hi, lo);
          ar->a2[p * 2 * I + i] = hi;
          ar->a2[p * 2 * I + I + i] = lo;
          if (ar->aw2) {
            split_bf(aw, hi, lo);
            ar->aw2[p * 2 * I + i] = hi;
            ar->aw2[p * 2 * I + I + i] = lo;
          }
        }
  }
};

// ------------------------------------------------------------- down-projection
template <class Cc, bool SMALL>
struct Gmm2F32 : RowTile<Cc, SMALL>, PlainCols<Cc> {
  static constexpr bool SCHED_HINT = false;
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::n0;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  struct Args {
    RowGroups g;
    const uint16_t* a2;
    const uint16_t* w2;
    int64_t S, H, I;
    float* o;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.a2, A.S * 2 * A.I * 2);
    this->template a_rows<false>(A.g, 2 * A.I, aoff);
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
    nk = (int)(2 * A.I / C::BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(((int64_t)kt * C::BK % ar->I) * ar->H * 2);  // W2 read once per half of K
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t*) {
    store_acc_f32<C, Gmm2F32>(acc, wm, wn, lane, ar->o, ar->H, row0, rows, n0, ar->H);
  }
};

// ------------------------------------------------------------- act_grad + SwiGLUGrad
// G = dY[tok] . W2[e]^T over K = 2H ([dY_hi | dY_lo]).  Epilogue as in the bf16
// product: one wave column of G at a time is staged in LDS (float32), then each
// thread takes 8 consecutive columns of one row, reads g, u (float32) and
// a = a_hi + a_lo as 16-byte vectors, writes dH = [dg_hi | du_hi | dg_lo | du_lo]
// as 16-byte vectors and adds its share of sum_i G a; the row sums are reduced in a
// fixed order (8-lane butterfly, then wave columns in order): one partial per
// (row, N tile).
template <class Cc, bool SMALL>
struct ActGradF32 : RowTile<Cc, SMALL>, PlainCols<Cc> {
  static constexpr bool SCHED_HINT = false;
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::n0;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  struct Args {
    RowGroups g;
    const uint16_t* dy2;  // [T][2H]
    const uint16_t* w2;
    const float* tw;
    const float* h;       // [S][2I]
    const uint16_t* a2;   // [S][2I]
    int64_t T, H, I;
    uint16_t* dh2;        // [S][4I]
    float* dwpart;        // [S][dw_cols] (may be NULL: not stored)
    int dw_cols;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.dy2, A.T * 2 * A.H * 2);
    this->template a_rows<true>(A.g, 2 * A.H, aoff);
    rb_ = make_rsrc(A.w2 + (int64_t)e * A.I * A.H, A.I * A.H * 2);
    this->b_rows(A.H, A.I, boff);
    nk = (int)(2 * A.H / C::BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(((int64_t)kt * C::BK % ar->H) * 2);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    constexpr int LDF = C::TN + 4;
    constexpr int CPR = C::TN / 8;
    constexpr int PER = C::BM * CPR / C::NTHR;
    static_assert(C::BM * CPR % C::NTHR == 0 && C::NTHR % CPR == 0, "chunk mapping");
    static_assert((C::BM * LDF + C::BM) * 4 <= 2 * C::STAGE * 2, "staging must fit in the LDS buffers");
    float* gst = reinterpret_cast<float*>(smem);
    float* wrow = gst + C::BM * LDF;
    const int tid = threadIdx.x;
    for (int t = tid; t < C::BM; t += C::NTHR) wrow[t] = (t < rows) ? ar->tw[ar->g.sorted_slot[row0 + t]] : 0.f;
    const int64_t I = ar->I;
    float part[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) part[k] = 0.f;
    for (int q = 0; q < C::WN; ++q) {
      if (wn == q) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              gst[acc_row<C>(wm, mb, r, lane) * LDF + nb * 32 + (lane & 31)] = acc[mb][nb][r];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int c = tid + k * C::NTHR;
        const int row = c / CPR, c8 = c % CPR;
        const int64_t i = n0 + q * C::TN + c8 * 8;
        float s = 0.f;
        if (row < rows && i < I) {
          const int64_t p = row0 + row;
          float g[8], u[8], ah[8], al[8], dg[8], du[8];
          const f32x4* hp = reinterpret_cast<const f32x4*>(ar->h + p * 2 * I + i);
          const f32x4* up = reinterpret_cast<const f32x4*>(ar->h + p * 2 * I + I + i);
          const f32x4 g0 = hp[0], g1 = hp[1], u0 = up[0], u1 = up[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            g[j] = g0[j]; g[4 + j] = g1[j];
            u[j] = u0[j]; u[4 + j] = u1[j];
          }
          unpack8(*reinterpret_cast<const u32x4*>(ar->a2 + p * 2 * I + i), ah);
          unpack8(*reinterpret_cast<const u32x4*>(ar->a2 + p * 2 * I + I + i), al);
          const float w = wrow[row];
          const float* G = gst + row * LDF + c8 * 8;
          float dgh[8], dgl[8], duh[8], dul[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            s += G[j] * (ah[j] + al[j]);
            const float dA = w * G[j];
            const float sg = sigmoidf_(g[j]);
            dg[j] = dA * u[j] * sg * (1.f + g[j] * (1.f - sg));
            du[j] = dA * g[j] * sg;
            dgh[j] = round_bf(dg[j]);
            dgl[j] = dg[j] - dgh[j];
            duh[j] = round_bf(du[j]);
            dul[j] = du[j] - duh[j];
          }
          uint16_t* d = ar->dh2 + p * 4 * I + i;
          *reinterpret_cast<u32x4*>(d) = pack8(dgh);
          *reinterpret_cast<u32x4*>(d + I) = pack8(duh);
          *reinterpret_cast<u32x4*>(d + 2 * I) = pack8(dgl);
          *reinterpret_cast<u32x4*>(d + 3 * I) = pack8(dul);
        }
#pragma unroll
        for (int d = CPR / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d);
        part[k] += s;
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = tid + k * C::NTHR;
      const int row = c / CPR;
      if (ar->dwpart && c % CPR == 0 && row < rows)
        ar->dwpart[(int64_t)(row0 + row) * ar->dw_cols + n0 / C::BN] = part[k];
    }
  }
};

// ------------------------------------------------------------- input_grad
template <class Cc, bool SMALL>
struct InputGradF32 : RowTile<Cc, SMALL>, PlainCols<Cc> {
  static constexpr bool SCHED_HINT = false;
  typedef RowTile<Cc, SMALL> B_;
  typedef Cc C;
  using B_::e; using B_::row0; using B_::rows; using B_::nk; using B_::n0;
  using PlainCols<Cc>::ncol0;
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  struct Args {
    RowGroups g;
    const uint16_t* dh2;
    const uint16_t* w1;
    int64_t S, H, I;
    float* dxp;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!this->init_rows(A.g, idx, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.dh2, A.S * 4 * A.I * 2);
    this->template a_rows<false>(A.g, 4 * A.I, aoff);
    rb_ = make_rsrc(A.w1 + (int64_t)e * A.H * 2 * A.I, A.H * 2 * A.I * 2);
    this->b_rows(2 * A.I, A.H, boff);
    nk = (int)(4 * A.I / C::BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * C::BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(((int64_t)kt * C::BK % (2 * ar->I)) * 2);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t*) {
    store_acc_f32<C, InputGradF32>(acc, wm, wn, lane, ar->dxp, ar->H, row0, rows, n0, ar->H);
  }
};

// ------------------------------------------------------------- weight gradients
// C[e][m][n] = sum over passes q and the expert's rows p of A_q[p][m] B_q[p][n]:
//   MODE 1 (dW1): A = x[tok] (gathered), B = dH2 columns [q 2I, q 2I + 2I), q = 0, 1
//   MODE 2 (dW2): A = aw2 columns [qa I, qa I + I), B = dY2[tok] columns [qb H, qb H + H),
//                 (qa, qb) = (0, 0), (0, 1), (1, 0)
template <class Cc, int MODE>
struct DwF32 : PlainCols<Cc> {
  typedef Cc C;
  using PlainCols<Cc>::ncol0;
  static constexpr bool SCHED_HINT = false;
  static constexpr bool A_KMAJ = false, B_KMAJ = false;
  static constexpr int PASSES = MODE == 1 ? 2 : 3;
  static constexpr bool GATHER_A = MODE == 1, GATHER_B = MODE == 2;
  struct Args {
    const int32_t* offsets;
    const int32_t* tok_of_row;
    int64_t E;
    const uint16_t* A;
    const uint16_t* B;
    int64_t a_rows, b_rows;    // rows held by A and B
    int64_t lda, ldb;          // their row pitches (elements)
    int64_t M, N;              // logical widths of one pass
    int64_t a_shift, b_shift;  // column offset of a lo pass
    float* Cout;               // [E][M][N]
    int mt, nt;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  int e, m0, n0, nk, nk1, p0, p1;
  uint32_t rowoff_a[C::CA], rowoff_b[C::CB];
  __device__ static __forceinline__ int qa(int q) { return (MODE == 2 && q == 2) ? 1 : 0; }
  __device__ static __forceinline__ int qb(int q) { return q == 1 ? 1 : 0; }
  // XCD-balanced slices of every expert's tiles, as for the bf16 weight gradients
  __device__ __forceinline__ bool init(const Args& A, int b) {
    ar = &A;
    const int per_e = A.mt * A.nt;
    const int per = (per_e + 7) / 8;
    const int j = b >> 3;
    e = j / per;
    if (e >= A.E) return false;
    const int t = (b & 7) * per + (j - e * per);
    if (t >= per_e) return false;
    int r, c;
    raster(t, A.mt, A.nt, r, c);
    m0 = r * C::BM;
    n0 = c * C::BN;
    p0 = A.offsets[e];
    p1 = A.offsets[e + 1];
    nk1 = (p1 - p0 + C::BK - 1) / C::BK;
    nk = PASSES * nk1;
    ra_ = make_rsrc(A.A, A.a_rows * A.lda * 2);
    rb_ = make_rsrc(A.B, A.b_rows * A.ldb * 2);
    return true;
  }
  // row indices of a step of the gathered operand, as fetched (see gemm_tile)
  struct Raw {
    int32_t a[GATHER_A ? C::CA : 1], b[GATHER_B ? C::CB : 1];
  };
  template <int R, int CN>
  __device__ __forceinline__ void fetch_rows(int kk, int32_t (&raw)[CN]) {
    const int tid = threadIdx.x;
    constexpr int CPR = R / 8;
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const int p = min(p0 + kk * C::BK + (tid + i * C::NTHR) / CPR, p1 - 1);
      raw[i] = ar->tok_of_row[p];
    }
  }
  __device__ __forceinline__ void fetch(int kt, Raw& r) {
    const int kk = kt % nk1;
    if constexpr (GATHER_A) fetch_rows<C::BM>(kk, r.a);
    if constexpr (GATHER_B) fetch_rows<C::BN>(kk, r.b);
  }
  template <bool GATHER, int R, int CN, int CR>
  __device__ __forceinline__ void rows_of(int64_t nrows, int64_t ld, int64_t width, int64_t shift, int64_t c0, int kk,
                                          const int32_t (&raw)[CR], uint32_t (&ro)[CN]) {
    const int tid = threadIdx.x;
    constexpr int CPR = R / 8;
    const uint32_t end = (uint32_t)(nrows * ld * 2);
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, c8 = c % CPR;
      const int p = p0 + kk * C::BK + kr;
      const uint32_t col = (uint32_t)c0 + c8 * 8;  // every offset fits 32 bits (resources < 4 GiB)
      uint32_t row = (uint32_t)p;
      if constexpr (GATHER) row = (uint32_t)raw[i];
      ro[i] = (p < p1 && col < (uint32_t)width) ? (row * (uint32_t)ld + (uint32_t)shift + col) * 2u : end;
    }
  }
  __device__ __forceinline__ void index(int kt, const Raw& r) {
    const int q = kt / nk1, kk = kt - q * nk1;
    rows_of<GATHER_A, C::BM, C::CA>(ar->a_rows, ar->lda, ar->M, qa(q) * ar->a_shift, m0, kk, r.a, rowoff_a);
    rows_of<GATHER_B, C::BN, C::CB>(ar->b_rows, ar->ldb, ar->N, qb(q) * ar->b_shift, n0, kk, r.b, rowoff_b);
  }
  __device__ __forceinline__ void load_a(int, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, rowoff_a[i], 0);
  }
  __device__ __forceinline__ void load_b(int, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, rowoff_b[i], 0);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t*) {
    store_acc_f32<C, DwF32>(acc, wm, wn, lane, ar->Cout + (int64_t)e * ar->M * ar->N, ar->N, m0,
                            (int)min((int64_t)C::BM, ar->M - m0), n0, ar->N);
  }
};

template <class C, int MODE>
hipError_t launch_dw_f32(const int32_t* offsets, const int32_t* tok_of_row, int64_t E, const uint16_t* A_,
                         const uint16_t* B_, int64_t a_rows, int64_t b_rows, int64_t lda, int64_t ldb, int64_t M,
                         int64_t N, int64_t a_shift, int64_t b_shift, float* out, hipStream_t stream) {
  typedef DwF32<C, MODE> P;
  typename P::Args A{offsets, tok_of_row, E, A_, B_, a_rows, b_rows, lda, ldb, M, N, a_shift, b_shift, out,
                     (int)((M + C::BM - 1) / C::BM), (int)((N + C::BN - 1) / C::BN)};
  return launch<P>(A, E * 8 * ((A.mt * A.nt + 7) / 8), stream);
}

}  // namespace

int act_grad_f32_dw_cols(int64_t I, bool narrow) {
  const int64_t bn = narrow ? NarrowF::BN : Big::BN;  // Big and Small share BN
  return (int)((I + bn - 1) / bn);
}

hipError_t launch_gmm1_f32(const RowGroups& g, const uint16_t* x, const uint16_t* w1, const float* topk_w, int64_t H,
                           int64_t I, float* h, uint16_t* a2, uint16_t* aw2, hipStream_t stream) {
  return launch_rows_c<Gmm1F32, NarrowF>(g, [&](int bn) { return (int)((I + bn / 2 - 1) / (bn / 2)); },
                                         [&](auto& A, int nnt) {
    A.g = g; A.x = x; A.w1 = w1; A.tw = topk_w; A.T = g.T; A.H = H; A.I = I; A.h = h; A.a2 = a2; A.aw2 = aw2;
    A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_gmm2_f32(const RowGroups& g, const uint16_t* a2, const uint16_t* w2, int64_t H, int64_t I, float* o,
                           hipStream_t stream) {
  return launch_rows_c<Gmm2F32, NarrowF>(g, [&](int bn) { return (int)((H + bn - 1) / bn); }, [&](auto& A, int nnt) {
    A.g = g; A.a2 = a2; A.w2 = w2; A.S = g.S; A.H = H; A.I = I; A.o = o; A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_act_grad_f32(const RowGroups& g, const uint16_t* dy2, const uint16_t* w2, const float* topk_w,
                               const float* h, const uint16_t* a2, int64_t H, int64_t I, uint16_t* dh2, float* dwpart,
                               int dw_cols, hipStream_t stream) {
  return launch_rows_c<ActGradF32, NarrowF>(g, [&](int bn) { return (int)((I + bn - 1) / bn); },
                                            [&](auto& A, int nnt) {
    A.g = g; A.dy2 = dy2; A.w2 = w2; A.tw = topk_w; A.h = h; A.a2 = a2; A.T = g.T; A.H = H; A.I = I; A.dh2 = dh2;
    A.dwpart = dwpart; A.dw_cols = dw_cols; A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_input_grad_f32(const RowGroups& g, const uint16_t* dh2, const uint16_t* w1, int64_t H, int64_t I,
                                 float* dxp, hipStream_t stream) {
  return launch_rows_c<InputGradF32, NarrowF>(g, [&](int bn) { return (int)((H + bn - 1) / bn); },
                                              [&](auto& A, int nnt) {
    A.g = g; A.dh2 = dh2; A.w1 = w1; A.S = g.S; A.H = H; A.I = I; A.dxp = dxp; A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_dw1_f32(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                          const uint16_t* x, const uint16_t* dh2, int64_t H, int64_t I, float* dw1, bool narrow,
                          hipStream_t stream) {
  if (narrow)
    return launch_dw_f32<NarrowF, 1>(offsets, tok_of_row, E, x, dh2, T, S, H, 4 * I, H, 2 * I, 0, 2 * I, dw1, stream);
  return launch_dw_f32<Big, 1>(offsets, tok_of_row, E, x, dh2, T, S, H, 4 * I, H, 2 * I, 0, 2 * I, dw1, stream);
}

hipError_t launch_dw2_f32(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                          const uint16_t* aw2, const uint16_t* dy2, int64_t H, int64_t I, float* dw2, bool narrow,
                          hipStream_t stream) {
  if (narrow)
    return launch_dw_f32<NarrowF, 2>(offsets, tok_of_row, E, aw2, dy2, S, T, 2 * I, 2 * H, I, H, I, H, dw2, stream);
  return launch_dw_f32<Big, 2>(offsets, tok_of_row, E, aw2, dy2, S, T, 2 * I, 2 * H, I, H, I, H, dw2, stream);
}

}  // namespace hmm
