// Grouped bf16 products of the MoE-FFN on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One main loop serves the six grouped products of the path (HyperMegaMoE RFC
// section 2.1: GMM1/up_proj, SwiGLU, GMM2/down_proj; section 2.2: act_grad,
// SwiGLUGrad, input_grad, W1Grad, W2Grad).  A policy class per product says
// where the A and B tiles come from and what the epilogue does:
//
//   product     grouping  A (layout)                 B (layout)               epilogue
//   gmm1        rows      x[tok(p)]  (K-major, gather) W1[e] [H,2I] (N-major)  SwiGLU -> h, a, aw
//   gmm2        rows      a[p]       (K-major)         W2[e] [I,H]  (N-major)  store o
//   act_grad    rows      dY[tok(p)] (K-major, gather) W2[e] as [I][H] (K-maj) SwiGLUGrad -> dH, dw partials
//   input_grad  rows      dH[p]      (K-major)         W1[e] as [H][2I] (K-maj) store dXp
//   dw1         reduction x[tok(p)]^T (M-major, gather) dH[p] (N-major)        store dW1[e]
//   dw2         reduction aw[p]^T    (M-major)          dY[tok(p)] (N-major)   store dW2[e]
//
// Tile shapes (each wave owns MB x NB accumulator blocks of 32 x 32):
//   Big   256 x 256 x 64, 8 waves as 2 x 4, 128 x 64 per wave (one workgroup per CU,
//         two waves per SIMD)
//   Small  64 x 256 x 64, 4 waves as 1 x 4,  64 x 64 per wave (expert remainders, small experts)
//   Narrow 64 x  64 x 64, 4 waves as 2 x 2,  32 x 32 per wave (whole problem small: many
//         workgroups instead of a few big tiles)
// "rows" products run over the routing's tile tables: each expert's rows are
// covered by big tiles, and a remainder of at most 128 rows by small tiles, so
// a small or long-tail expert does not pay for a 256-row tile (RFC 6.3, expert
// x block granularity).  "reduction" products run one big tile per (expert,
// M-tile, N-tile) and reduce over that expert's rows; an expert without rows
// writes zeros.
//
// Both operand tiles go through LDS, double buffered.  Global loads are buffer
// loads (32-bit per-thread offsets against a resource of the operand, the K step
// in the scalar offset; an offset past the resource's end reads zeros) and run
// three K steps ahead of the MFMAs: while LDS holds step k, two register sets
// hold steps k+1 and k+2.  Row indices of gathered reduction operands are
// fetched one step before their data.
// K-major tiles sit in LDS as [row][k] (pitch 72 elements) and are read with
// ds_read_b128; M/N-major tiles sit as [k][m] and are read with the gfx950
// transposing ds_read_b64_tr_b16, so no operand is transposed in memory.  LDS
// has 64 banks of 4 bytes and serves 32 lanes of a 64-bit read per pass: the
// four k rows such a pass touches (64 bytes each) fall in distinct banks when
// the row pitch is 64 bytes past a multiple of 256, hence pitch BM+32.  Work is rasterised in groups of 8 row tiles walked column by column,
// and workgroup ids are remapped so that the consecutive logical tiles of such
// a group run on one XCD and share its L2.
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
    uint16_t *h, *a, *aw;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  int i0;
  // the B tile holds BN/2 gate columns then the BN/2 matching up columns; the
  // epilogue pairs them through LDS
  __device__ static __forceinline__ int ncol0(int wn, int nb) { return wn * C::TN + nb * 32; }
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!this->init_rows(A.g, logical, A.n_ntiles)) return false;
    i0 = nt * (C::BN / 2);
    ra_ = make_rsrc(A.x, A.T * A.H * 2);
    this->template a_rows<true>(A.g, A.H, aoff);
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
    nk = (int)(A.H / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(kt * BK * 2 * ar->I * 2);
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
    for (int t = tid; t < C::BM; t += C::NTHR) wrow[t] = (t < rows) ? ar->tw[ar->g.sorted_slot[row0 + t]] : 0.f;
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
      *reinterpret_cast<u32x4*>(ar->h + p * 2 * I + i) = gv;
      *reinterpret_cast<u32x4*>(ar->h + p * 2 * I + I + i) = uv;
      *reinterpret_cast<u32x4*>(ar->a + p * I + i) = pack8(av);
      *reinterpret_cast<u32x4*>(ar->aw + p * I + i) = pack8(aw);
    }
  }
};

// ------------------------------------------------------------- gmm2
template <class Cc, bool SMALL>
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
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!this->init_rows(A.g, logical, A.n_ntiles)) return false;
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
    nk = (int)(A.I / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(kt * BK * ar->H * 2);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    store_tile<C, Gmm2>(acc, wm, wn, lane, smem, ar->o, ar->H, row0, rows, n0, ar->H);
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
    const uint16_t* a;
    int64_t T, H, I;
    uint16_t* dh;
    float* dwpart;
    int dw_cols;
    int n_ntiles;
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!this->init_rows(A.g, logical, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.dy, A.T * A.H * 2);
    this->template a_rows<true>(A.g, A.H, aoff);
    rb_ = make_rsrc(A.w2 + (int64_t)e * A.I * A.H, A.I * A.H * 2);
    this->b_rows(A.H, A.I, boff);
    nk = (int)(A.H / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], kt * BK * 2);
  }
  // G stays in float32: one wave column (TN columns) at a time it is staged in
  // LDS, then each thread takes 8 consecutive columns of one row, reads g, u and
  // a as 16-byte chunks, writes dH = [dg | du] as 16-byte chunks and adds its
  // share of sum_i G a.  The row sums are reduced in a fixed order (8-lane
  // butterfly, then wave columns in order): one partial per (row, N tile).
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem) {
    constexpr int LDF = C::TN + 4;                      // float pitch of the staged G
    constexpr int CPR = C::TN / 8;                      // 8-column chunks per row of a wave column
    constexpr int PER = C::BM * CPR / C::NTHR;          // chunks per thread per wave column
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
          float g[8], u[8], av[8], dg[8], du[8];
          unpack8(*reinterpret_cast<const u32x4*>(ar->h + p * 2 * I + i), g);
          unpack8(*reinterpret_cast<const u32x4*>(ar->h + p * 2 * I + I + i), u);
          unpack8(*reinterpret_cast<const u32x4*>(ar->a + p * I + i), av);
          const float w = wrow[row];
          const float* G = gst + row * LDF + c8 * 8;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            s += G[j] * av[j];
            const float dA = w * G[j];
            const float sg = sigmoidf_(g[j]);
            dg[j] = dA * u[j] * sg * (1.f + g[j] * (1.f - sg));
            du[j] = dA * g[j] * sg;
          }
          *reinterpret_cast<u32x4*>(ar->dh + p * 2 * I + i) = pack8(dg);
          *reinterpret_cast<u32x4*>(ar->dh + p * 2 * I + I + i) = pack8(du);
        }
        // the CPR threads of a row are consecutive lanes: fixed-order butterfly
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
      if (c % CPR == 0 && row < rows) ar->dwpart[(int64_t)(row0 + row) * ar->dw_cols + n0 / C::BN] = part[k];
    }
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
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!this->init_rows(A.g, logical, A.n_ntiles)) return false;
    ra_ = make_rsrc(A.dh, A.S * 2 * A.I * 2);
    this->template a_rows<false>(A.g, 2 * A.I, aoff);
    rb_ = make_rsrc(A.w1 + (int64_t)e * A.H * 2 * A.I, A.H * 2 * A.I * 2);
    this->b_rows(2 * A.I, A.H, boff);
    nk = (int)(2 * A.I / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * BK * 2);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], kt * BK * 2);
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
  static constexpr bool RAW_INDEX = true;  // init maps the workgroup index to XCDs itself
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
  };
  const Args* ar;
  rsrc_t ra_, rb_;
  int e, m0, n0, nk, p0, p1;
  // byte offsets of the rows of the next step to be loaded (computed by index())
  uint32_t rowoff_a[C::CA], rowoff_b[C::CB];
  // The cost of a tile grows with its expert's row count, so every XCD gets an
  // equal slice of every expert's tiles (not a contiguous run of experts): XCD x
  // (workgroups b with b % 8 == x) walks the experts in order and takes tiles
  // [x * per, (x + 1) * per) of each, per = ceil(mt * nt / 8); inside a slice the
  // tiles are rasterised in groups of GROUP_M row tiles.
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
    nk = (p1 - p0 + BK - 1) / BK;
    ra_ = make_rsrc(A.A, A.a_rows * A.M * 2);
    rb_ = make_rsrc(A.B, A.b_rows * A.N * 2);
    return true;
  }
  // row part of the offsets of step kt: rows p past the expert's end and columns
  // past the matrix get the resource's end (reads zeros)
  template <bool GATHER, int R, int CN>
  __device__ __forceinline__ void rows_of(int64_t nrows, int64_t ld, int64_t c0, int kt, uint32_t (&ro)[CN]) {
    const int tid = threadIdx.x;
    constexpr int CPR = R / 8;
    const uint32_t end = (uint32_t)(nrows * ld * 2);
#pragma unroll
    for (int i = 0; i < CN; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, c8 = c % CPR;
      const int p = p0 + kt * BK + kr;
      const int64_t col = c0 + c8 * 8;
      uint32_t off = end;
      if (p < p1 && col < ld) {
        const int64_t row = GATHER ? (int64_t)ar->tok_of_row[p] : (int64_t)p;
        off = (uint32_t)((row * ld + col) * 2);
      }
      ro[i] = off;
    }
  }
  __device__ __forceinline__ void index(int kt) {
    rows_of<GATHER_A, C::BM, C::CA>(ar->a_rows, ar->M, m0, kt, rowoff_a);
    rows_of<GATHER_B, C::BN, C::CB>(ar->b_rows, ar->N, n0, kt, rowoff_b);
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

int act_grad_dw_cols(int64_t I, bool narrow) {
  const int64_t bn = narrow ? Narrow::BN : Big::BN;  // Big and Small share BN
  return (int)((I + bn - 1) / bn);
}

hipError_t launch_gmm1_swiglu(const RowGroups& g, const uint16_t* x, const uint16_t* w1, const float* topk_w,
                              int64_t H, int64_t I, uint16_t* h, uint16_t* a, uint16_t* aw, hipStream_t stream) {
  // BN/2 gate columns (and their up columns) per N tile
  return launch_rows<Gmm1>(g, [&](int bn) { return (int)((I + bn / 2 - 1) / (bn / 2)); }, [&](auto& A, int nnt) {
    A.g = g; A.x = x; A.w1 = w1; A.tw = topk_w; A.T = g.T; A.H = H; A.I = I; A.h = h; A.a = a; A.aw = aw;
    A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_gmm2(const RowGroups& g, const uint16_t* a, const uint16_t* w2, int64_t H, int64_t I,
                       uint16_t* o, hipStream_t stream) {
  return launch_rows<Gmm2>(g, [&](int bn) { return (int)((H + bn - 1) / bn); }, [&](auto& A, int nnt) {
    A.g = g; A.a = a; A.w2 = w2; A.S = g.S; A.H = H; A.I = I; A.o = o; A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_act_grad(const RowGroups& g, const uint16_t* dy, const uint16_t* w2, const float* topk_w,
                           const uint16_t* h, const uint16_t* a, int64_t H, int64_t I, uint16_t* dh,
                           float* dwpart, int dw_cols, hipStream_t stream) {
  return launch_rows<ActGrad>(g, [&](int bn) { return (int)((I + bn - 1) / bn); }, [&](auto& A, int nnt) {
    A.g = g; A.dy = dy; A.w2 = w2; A.tw = topk_w; A.h = h; A.a = a; A.T = g.T; A.H = H; A.I = I; A.dh = dh;
    A.dwpart = dwpart; A.dw_cols = dw_cols; A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_input_grad(const RowGroups& g, const uint16_t* dh, const uint16_t* w1, int64_t H, int64_t I,
                             uint16_t* dxp, hipStream_t stream) {
  return launch_rows<InputGrad>(g, [&](int bn) { return (int)((H + bn - 1) / bn); }, [&](auto& A, int nnt) {
    A.g = g; A.dh = dh; A.w1 = w1; A.S = g.S; A.H = H; A.I = I; A.dxp = dxp; A.n_ntiles = nnt;
  }, stream);
}

template <class C, bool GA, bool GB>
hipError_t launch_dw(const int32_t* offsets, const int32_t* tok_of_row, int64_t E, const uint16_t* A_,
                     const uint16_t* B_, int64_t a_rows, int64_t b_rows, int64_t M, int64_t N, uint16_t* out,
                     hipStream_t stream) {
  typedef Dw<C, GA, GB> P;
  typename P::Args A{offsets, tok_of_row, E, A_, B_, a_rows, b_rows, M, N, out,
                     (int)((M + C::BM - 1) / C::BM), (int)((N + C::BN - 1) / C::BN)};
  return launch<P>(A, E * 8 * ((A.mt * A.nt + 7) / 8), stream);
}

hipError_t launch_dw1(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                      const uint16_t* x, const uint16_t* dh, int64_t H, int64_t I, uint16_t* dw1, bool narrow,
                      hipStream_t stream) {
  if (narrow) return launch_dw<Narrow, true, false>(offsets, tok_of_row, E, x, dh, T, S, H, 2 * I, dw1, stream);
  return launch_dw<Big, true, false>(offsets, tok_of_row, E, x, dh, T, S, H, 2 * I, dw1, stream);
}

hipError_t launch_dw2(const int32_t* offsets, const int32_t* tok_of_row, int64_t T, int64_t S, int64_t E,
                      const uint16_t* aw, const uint16_t* dy, int64_t H, int64_t I, uint16_t* dw2, bool narrow,
                      hipStream_t stream) {
  if (narrow) return launch_dw<Narrow, false, true>(offsets, tok_of_row, E, aw, dy, S, T, I, H, dw2, stream);
  return launch_dw<Big, false, true>(offsets, tok_of_row, E, aw, dy, S, T, I, H, dw2, stream);
}

namespace {
template <class C, bool GA, bool GB>
typename Dw<C, GA, GB>::Args dw_args(const int32_t* offsets, const int32_t* tok_of_row, int64_t E, const uint16_t* A_,
                                     const uint16_t* B_, int64_t a_rows, int64_t b_rows, int64_t M, int64_t N,
                                     uint16_t* out) {
  return typename Dw<C, GA, GB>::Args{offsets, tok_of_row, E, A_, B_, a_rows, b_rows, M, N, out,
                                      (int)((M + C::BM - 1) / C::BM), (int)((N + C::BN - 1) / C::BN)};
}
template <class A>
int64_t dw_blocks(const A& a) { return a.E * 8 * ((a.mt * a.nt + 7) / 8); }
}  // namespace

hipError_t launch_act_grad_dw2_narrow(const RowGroups& g, const uint16_t* dy, const uint16_t* w2, const float* topk_w,
                                      const uint16_t* h, const uint16_t* a, const uint16_t* aw, int64_t E, int64_t H,
                                      int64_t I, uint16_t* dh, float* dwpart, int dw_cols, uint16_t* dw2,
                                      hipStream_t stream) {
  typedef ActGrad<Narrow, true> P1;
  typedef Dw<Narrow, false, true> P2;
  const int nnt = (int)((I + Narrow::BN - 1) / Narrow::BN);
  typename P1::Args a1;
  a1.g = g; a1.dy = dy; a1.w2 = w2; a1.tw = topk_w; a1.h = h; a1.a = a; a1.T = g.T; a1.H = H; a1.I = I; a1.dh = dh;
  a1.dwpart = dwpart; a1.dw_cols = dw_cols; a1.n_ntiles = nnt;
  const typename P2::Args a2 = dw_args<Narrow, false, true>(g.offsets, g.tok_of_row, E, aw, dy, g.S, g.T, I, H, dw2);
  return launch_pair<P1, P2>(a1, g.max_small * nnt, a2, dw_blocks(a2), stream);
}

hipError_t launch_input_grad_dw1_narrow(const RowGroups& g, const uint16_t* dh, const uint16_t* w1, const uint16_t* x,
                                        int64_t E, int64_t H, int64_t I, uint16_t* dxp, uint16_t* dw1,
                                        hipStream_t stream) {
  typedef InputGrad<Narrow, true> P1;
  typedef Dw<Narrow, true, false> P2;
  const int nnt = (int)((H + Narrow::BN - 1) / Narrow::BN);
  typename P1::Args a1;
  a1.g = g; a1.dh = dh; a1.w1 = w1; a1.S = g.S; a1.H = H; a1.I = I; a1.dxp = dxp; a1.n_ntiles = nnt;
  const typename P2::Args a2 =
      dw_args<Narrow, true, false>(g.offsets, g.tok_of_row, E, x, dh, g.T, g.S, H, 2 * I, dw1);
  return launch_pair<P1, P2>(a1, g.max_small * nnt, a2, dw_blocks(a2), stream);
}

}  // namespace hmm
