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

namespace {
// ------------------------------------------------------------- routed up-projection
// An up-projection tile that routes the ids itself (launch_route_gmm1_swiglu).
// The four waves count the ids of their chunks (slots [w chunk, (w+1) chunk)) per
// expert with ballots, as the one-workgroup routing does; inclusive scans over
// the experts give every expert's first row and first 64-row tile, so the
// workgroup finds its tile (spread over the XCDs by real_tile, with the real
// tile count in hand), then each wave walks its chunk again for the tile's
// expert alone:
//   row = (first row of the expert) + (its slots in earlier waves) + (its
//         earlier slots in this wave's chunk),
// the stable (expert, slot) order.  The tile's tokens and slots land in LDS and
// take the place of the tables' loads.  The launch also stores the routing's
// tables for the later launches: the tile of column 0 its rows (sorted_slot,
// tok_of_row, row_of_slot) and its table entry, workgroup 0 (tile 0, or none
// when no id is valid) every expert's count and first row, the table's header,
// row_of_slot -1 for the slots whose id is out of range, and the error flags.
struct TileRouteLds {
  static constexpr int NW = Narrow::NTHR / 64;
  int32_t cnt[NW][RT_ONE_MAX_EXPERTS];  // per wave, per expert
  int32_t tot[2][NW];                   // per wave: inclusive rows and tiles over its experts
  int32_t info[3 + NW];                 // expert, first row, rows; first row of each wave's slots
  int32_t tok[TILE_SMALL], slot[TILE_SMALL];
};

struct Gmm1Routed : Gmm1<Narrow, true> {
  typedef Gmm1<Narrow, true> G;
  struct Args : G::Args {
    const int32_t* ids;
    int E, K, nbits, max_big;
    int32_t *counts, *offsets, *sorted_slot, *row_of_slot, *tok_of_row, *tiles, *err, *host_err;
  };
  static_assert(C::BM == TILE_SMALL && C::NTHR >= RT_ONE_MAX_EXPERTS, "one thread per expert, one tile row each");

  __device__ __forceinline__ bool init(const Args& A, int idx) {
    __shared__ TileRouteLds L;
    constexpr int NW = TileRouteLds::NW;
    constexpr int R = ROUTED_MAX_SLOTS / C::NTHR;  // 64-slot rounds per wave at most
    ar = &A;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int S = (int)A.g.S, E = A.E;
    for (int i = lane; i < RT_ONE_MAX_EXPERTS; i += 64) L.cnt[w][i] = 0;  // each wave counts in its own row
    const int chunk = ((S + NW - 1) / NW + 63) / 64 * 64;
    const int s0 = w * chunk;
    int ev[R];  // the id of each of this lane's slots; -1 past S or outside [0, E)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int s = s0 + j * 64 + lane;
      const int v = (j * 64 < chunk && s < S) ? A.ids[s] : -1;
      ev[j] = (v >= 0 && v < E) ? v : -1;
    }
    wave_lds_sync();
    const uint64_t lt_mask = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j * 64 >= chunk) continue;  // the same for every wave
      const int v = ev[j];
      const bool valid = v >= 0;
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < A.nbits; ++bit) {
        const bool set = valid && ((v >> bit) & 1);
        const uint64_t m = __ballot(set);
        peers &= set ? m : ~m;
      }
      // one leader per id; an LDS add, so the rounds do not wait on each other
      if (valid && __popcll(peers & lt_mask) == 0) atomicAdd(&L.cnt[w][v], __popcll(peers));
    }
    __syncthreads();
    // thread x < E: expert x's rows and 64-row tiles, scanned over the experts
    int c = 0;
    if (tid < E)
#pragma unroll
      for (int q = 0; q < NW; ++q) c += L.cnt[q][tid];
    const int nt_x = (c + TILE_SMALL - 1) / TILE_SMALL;
    int ic = c, is = nt_x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int vc = __shfl_up(ic, d), vs = __shfl_up(is, d);
      if (lane >= d) {
        ic += vc;
        is += vs;
      }
    }
    if (lane == 63) {
      L.tot[0][w] = ic;
      L.tot[1][w] = is;
    }
    __syncthreads();
    int ntiles = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      if (q < w) {
        ic += L.tot[0][q];
        is += L.tot[1][q];
      }
      ntiles += L.tot[1][q];
    }
    if (idx == 0) {
      if (tid < E) {
        A.counts[tid] = c;
        A.offsets[tid] = ic - c;
      }
      if (tid == C::NTHR - 1) {  // holds the totals over all experts
        A.offsets[E] = ic;
        A.tiles[0] = 0;
        A.tiles[1] = ntiles;
        A.tiles[2] = TILE_BIG;
        A.tiles[3] = TILE_SMALL;
      }
      int bad = 0;
#pragma unroll
      for (int jj = 0; jj < R; ++jj) {
        const int s = s0 + jj * 64 + lane;
        if (jj * 64 < chunk && s < S && ev[jj] < 0) {
          A.row_of_slot[s] = -1;
          bad = 1;
        }
      }
      bad = __syncthreads_or(bad);
      if (tid == 0) {
        *A.err = bad;
        // the host reads this word only after the launch has completed: no release needed
        if (A.host_err) __hip_atomic_store(A.host_err, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    int j;
    if (!real_tile(idx, ntiles, A.n_ntiles, j, nt)) return false;  // every thread alike
    if (tid < E && j >= is - nt_x && j < is) {  // expert tid holds tile j
      const int first = j - (is - nt_x);
      int b = ic - c;
      L.info[0] = tid;
      L.info[1] = b + first * TILE_SMALL;
      L.info[2] = min(TILE_SMALL, c - first * TILE_SMALL);
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        L.info[3 + q] = b;
        b += L.cnt[q][tid];
      }
    }
    __syncthreads();
    e = L.info[0];
    row0 = L.info[1];
    rows = L.info[2];
    int base = L.info[3 + w];
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
      if (jj * 64 >= chunk) continue;
      const bool mine = ev[jj] == e;
      const uint64_t m = __ballot(mine);
      if (mine) {
        const int r = base + __popcll(m & lt_mask) - row0;
        if (r >= 0 && r < rows) {
          const int s = s0 + jj * 64 + lane;
          L.tok[r] = s / A.K;
          L.slot[r] = s;
        }
      }
      base += __popcll(m);
    }
    __syncthreads();
    if (nt == 0) {
      if (tid < rows) {
        const int p = row0 + tid;
        A.sorted_slot[p] = L.slot[tid];
        A.tok_of_row[p] = L.tok[tid];
        A.row_of_slot[L.slot[tid]] = p;
      }
      if (tid == 0) {
        int32_t* entry = A.tiles + 4 + 2 * A.max_big + 2 * j;
        entry[0] = tile_word(e, rows);
        entry[1] = row0;
      }
    }
    // as Gmm1::init, with the tile's rows from LDS
    slot_own = (tid < rows) ? L.slot[tid] : 0;
    i0 = nt * (C::BN / 2);
    ra_ = make_rsrc(A.x, A.T * A.H * 2);
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int cc = tid + i * C::NTHR;
      const int r = min(cc / C::KCH, rows - 1);
      aoff[i] = (uint32_t)(((int64_t)L.tok[r] * A.H + (cc % C::KCH) * 8) * 2);
    }
    init_b(A);
    return true;
  }
};

}  // namespace

hipError_t launch_route_gmm1_swiglu(const RoutedGmm1Job& j, hipStream_t stream) {
  const Gmm1Job& u = j.up;
  if (u.g.S <= 0) return hipSuccess;
  if (!u.g.narrow || u.g.S > ROUTED_MAX_SLOTS || j.E < 1 || j.E > RT_ONE_MAX_EXPERTS || j.K < 1 ||
      u.g.S % j.K)
    return hipErrorInvalidValue;
  Gmm1Routed::Args a;
  const int nnt = ntiles_half(u.I, Narrow::BN);
  fill_gmm1(a, u, nnt);
  a.ids = j.ids;
  a.E = j.E;
  a.K = j.K;
  a.nbits = 0;
  while ((1 << a.nbits) < j.E) ++a.nbits;
  a.max_big = j.max_big;
  a.counts = j.counts; a.offsets = j.offsets; a.sorted_slot = j.sorted_slot; a.row_of_slot = j.row_of_slot;
  a.tok_of_row = j.tok_of_row; a.tiles = j.tiles; a.err = j.err; a.host_err = j.host_err;
  return launch<Gmm1Routed>(a, u.g.max_small * nnt, stream);
}

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
