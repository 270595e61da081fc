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
#include "gemm_bf16.h"

namespace hmm {

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

// Narrow tiling: a routed product and the shared expert's share one launch.
hipError_t launch_gmm1_swiglu_with_shared(const RowGroups& g, const uint16_t* x, const uint16_t* w1,
                                          const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                                          uint16_t* aw, const RowGroups& gs, const uint16_t* w1s, const float* ones,
                                          int64_t Is, uint16_t* hs, uint16_t* as, hipStream_t stream) {
  typedef Gmm1<Narrow, true> P;
  constexpr int HALF = Narrow::BN / 2;
  typename P::Args a1, a2;
  a1.g = g; a1.x = x; a1.w1 = w1; a1.tw = topk_w; a1.T = g.T; a1.H = H; a1.I = I; a1.h = h; a1.a = a; a1.aw = aw;
  a1.n_ntiles = (int)((I + HALF - 1) / HALF);
  a2.g = gs; a2.x = x; a2.w1 = w1s; a2.tw = ones; a2.T = gs.T; a2.H = H; a2.I = Is; a2.h = hs; a2.a = as;
  a2.aw = nullptr; a2.n_ntiles = (int)((Is + HALF - 1) / HALF);
  return launch_pair<P, P>(a1, g.max_small * a1.n_ntiles, a2, gs.max_small * a2.n_ntiles, stream);
}

hipError_t launch_gmm2_with_shared(const RowGroups& g, const uint16_t* a, const uint16_t* w2, int64_t H, int64_t I,
                                   uint16_t* o, const RowGroups& gs, const uint16_t* as, const uint16_t* w2s,
                                   int64_t Is, uint16_t* os, hipStream_t stream) {
  typedef Gmm2<Narrow, true> P;
  typename P::Args a1, a2;
  const int nnt = (int)((H + Narrow::BN - 1) / Narrow::BN);
  a1.g = g; a1.a = a; a1.w2 = w2; a1.S = g.S; a1.H = H; a1.I = I; a1.o = o; a1.n_ntiles = nnt;
  a2.g = gs; a2.a = as; a2.w2 = w2s; a2.S = gs.S; a2.H = H; a2.I = Is; a2.o = os; a2.n_ntiles = nnt;
  return launch_pair<P, P>(a1, g.max_small * nnt, a2, gs.max_small * nnt, stream);
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
