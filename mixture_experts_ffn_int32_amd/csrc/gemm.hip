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
//   Small  64 x 256 x 64, 8 waves as 2 x 4,  32 x 64 per wave (expert remainders, small experts;
//          eight waves: one workgroup fits a CU by LDS, and four waves left each SIMD one)
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
#include "gemm_bf16.h"

namespace hmm {

int act_grad_dw_cols(int64_t I, bool narrow) {
  const int64_t bn = narrow ? Narrow::BN : Big::BN;  // Big and Small share BN
  return (int)((I + bn - 1) / bn);
}

namespace {
// per-job policy arguments
template <class A>
void fill_gmm1(A& a, const Gmm1Job& j, int nnt) {
  a.g = j.g; a.x = j.x; a.w1 = j.w1; a.tw = j.tw; a.T = j.g.T; a.H = j.H; a.I = j.I; a.h = j.h; a.a = j.a;
  a.aw = j.aw; a.n_ntiles = nnt;
}
template <class A>
void fill_gmm2(A& a, const Gmm2Job& j, int nnt) {
  a.g = j.g; a.a = j.a; a.w2 = j.w2; a.S = j.g.S; a.H = j.H; a.I = j.I; a.o = j.o; a.n_ntiles = nnt;
}
template <class A>
void fill_act_grad(A& a, const ActGradJob& j, int nnt) {
  a.g = j.g; a.dy = j.dy; a.w2 = j.w2; a.tw = j.tw; a.h = j.h; a.T = j.g.T; a.H = j.H; a.I = j.I;
  a.dh = j.dh; a.dwpart = j.dwpart; a.dw_cols = j.dw_cols; a.n_ntiles = nnt;
}
template <class A>
void fill_input_grad(A& a, const InputGradJob& j, int nnt) {
  a.g = j.g; a.dh = j.dh; a.w1 = j.w1; a.S = j.g.S; a.H = j.H; a.I = j.I; a.dxp = j.dxp; a.n_ntiles = nnt;
}
template <class C, bool GA, bool GB>
typename Dw<C, GA, GB>::Args dw_args(const DwJob& j) {
  return typename Dw<C, GA, GB>::Args{j.offsets, j.tok_of_row, j.E, j.A, j.B, j.a_rows, j.b_rows, j.M, j.N, j.out,
                                      (int)((j.M + C::BM - 1) / C::BM), (int)((j.N + C::BN - 1) / C::BN), j.order};
}
template <class A>
int64_t dw_blocks(const A& a) { return a.E * 8 * ((a.mt * a.nt + 7) / 8); }

int ntiles_half(int64_t n, int bn) { return (int)((n + bn / 2 - 1) / (bn / 2)); }  // BN/2 gate (+ up) columns
int ntiles_full(int64_t n, int bn) { return (int)((n + bn - 1) / bn); }

// Narrow tiles: the jobs share one launch.  Big tiles: one launch each (the
// paired big-tile kernel runs out of registers, and a big-tile launch of a
// weight gradient already holds many tiles).
template <class C, bool GA, bool GB>
hipError_t launch_dw_jobs(const DwJob* j, int n, hipStream_t stream) {
  typedef Dw<C, GA, GB> P;
  const typename P::Args a0 = dw_args<C, GA, GB>(j[0]);
  if (n == 1) return launch<P>(a0, dw_blocks(a0), stream);
  const typename P::Args a1 = dw_args<C, GA, GB>(j[1]);
  if constexpr (C::BM == Big::BM) {
    const hipError_t e = launch<P>(a0, dw_blocks(a0), stream);
    return e != hipSuccess ? e : launch<P>(a1, dw_blocks(a1), stream);
  } else {
    return launch_pair<P, P>(a0, dw_blocks(a0), a1, dw_blocks(a1), stream);
  }
}
}  // namespace

hipError_t launch_gmm1_swiglu(const Gmm1Job* jobs, int n, hipStream_t stream) {
  return launch_rows_jobs<Gmm1, Narrow>(jobs, n, [](const Gmm1Job& j, int bn) { return ntiles_half(j.I, bn); },
                                        [](auto& a, const Gmm1Job& j, int nnt) { fill_gmm1(a, j, nnt); }, stream);
}

hipError_t launch_gmm2(const Gmm2Job* jobs, int n, hipStream_t stream) {
  return launch_rows_jobs<Gmm2, Narrow>(jobs, n, [](const Gmm2Job& j, int bn) { return ntiles_full(j.H, bn); },
                                        [](auto& a, const Gmm2Job& j, int nnt) { fill_gmm2(a, j, nnt); }, stream);
}

hipError_t launch_act_grad(const ActGradJob* jobs, int n, hipStream_t stream) {
  return launch_rows_jobs<ActGrad, Narrow>(jobs, n, [](const ActGradJob& j, int bn) { return ntiles_full(j.I, bn); },
                                           [](auto& a, const ActGradJob& j, int nnt) { fill_act_grad(a, j, nnt); },
                                           stream);
}

hipError_t launch_input_grad(const InputGradJob* jobs, int n, hipStream_t stream) {
  return launch_rows_jobs<InputGrad, Narrow>(
      jobs, n, [](const InputGradJob& j, int bn) { return ntiles_full(j.H, bn); },
      [](auto& a, const InputGradJob& j, int nnt) { fill_input_grad(a, j, nnt); }, stream);
}

hipError_t launch_dw1(const DwJob* jobs, int n, bool narrow, hipStream_t stream) {
  return narrow ? launch_dw_jobs<Narrow, true, false>(jobs, n, stream)
                : launch_dw_jobs<Big, true, false>(jobs, n, stream);
}

hipError_t launch_dw2(const DwJob* jobs, int n, bool narrow, hipStream_t stream) {
  return narrow ? launch_dw_jobs<Narrow, false, true>(jobs, n, stream)
                : launch_dw_jobs<Big, false, true>(jobs, n, stream);
}

hipError_t launch_act_grad_dw2_narrow(const ActGradJob* ag, const DwJob* dw2, int n, hipStream_t stream) {
  typedef ActGrad<Narrow, true> P1;
  typedef Dw<Narrow, false, true> P2;
  typename P1::Args a[2];
  typename P2::Args d[2];
  int64_t ba[2] = {0, 0}, bd[2] = {0, 0};
  for (int q = 0; q < n; ++q) {
    const int nnt = ntiles_full(ag[q].I, Narrow::BN);
    fill_act_grad(a[q], ag[q], nnt);
    ba[q] = ag[q].g.max_small * nnt;
    d[q] = dw_args<Narrow, false, true>(dw2[q]);
    bd[q] = dw_blocks(d[q]);
  }
  if (n == 1) return launch_pair<P1, P2>(a[0], ba[0], d[0], bd[0], stream);
  return launch_quad<P1, P2, P1, P2>(a[0], ba[0], d[0], bd[0], a[1], ba[1], d[1], bd[1], stream);
}

hipError_t launch_input_grad_dw1_narrow(const InputGradJob* ig, const DwJob* dw1, int n, hipStream_t stream) {
  typedef InputGrad<Narrow, true> P1;
  typedef Dw<Narrow, true, false> P2;
  typename P1::Args a[2];
  typename P2::Args d[2];
  int64_t ba[2] = {0, 0}, bd[2] = {0, 0};
  for (int q = 0; q < n; ++q) {
    const int nnt = ntiles_full(ig[q].H, Narrow::BN);
    fill_input_grad(a[q], ig[q], nnt);
    ba[q] = ig[q].g.max_small * nnt;
    d[q] = dw_args<Narrow, true, false>(dw1[q]);
    bd[q] = dw_blocks(d[q]);
  }
  if (n == 1) return launch_pair<P1, P2>(a[0], ba[0], d[0], bd[0], stream);
  return launch_quad<P1, P2, P1, P2>(a[0], ba[0], d[0], bd[0], a[1], ba[1], d[1], bd[1], stream);
}

}  // namespace hmm
