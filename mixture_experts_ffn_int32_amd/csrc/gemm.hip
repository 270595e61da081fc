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
// "rows" products take their work from the tile table built by the routing
// (one 128-row tile of one expert per entry; the last tile of an expert is
// ragged).  "reduction" products run one tile per (expert, M-tile, N-tile) and
// reduce over that expert's rows; an expert without rows writes zeros.
//
// Tile: 128 x 128 x 64, 256 threads = 4 waves in 2 x 2, each wave a 64 x 64
// block of 2 x 2 MFMA 32x32 accumulators.  Both operand tiles go through LDS,
// double buffered, with global loads of the next K step issued before the MFMAs
// of the current one.  K-major tiles sit in LDS as [row][k] (row pitch 72
// elements) and are read with ds_read_b128; M/N-major tiles sit as [k][m]
// (pitch 144) and are read with the gfx950 transposing ds_read_b64_tr_b16, so
// no operand is transposed in memory.  Workgroup ids are remapped so that
// consecutive logical tiles land on the same XCD (one L2 each).
#include "device.h"
#include "kernels.h"

namespace hmm {
namespace {

constexpr int BM = GEMM_BM;  // 128
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int NTHR = 256;
constexpr int LDK = BK + 8;      // pitch of a K-major LDS tile (elements)
constexpr int LDMN = BM + 16;    // pitch of an M/N-major LDS tile (elements)
constexpr int TILE_ELEMS = 128 * LDK;  // == 64 * LDMN == 9216
static_assert(TILE_ELEMS == 64 * LDMN, "both LDS tile layouts have the same footprint");
constexpr int CHUNKS = 4;        // 16-byte chunks per thread per operand tile (128*64*2 B / 16 B / 256)

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // nblocks is a multiple of 8; workgroups are dealt to the 8 XCDs round robin
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 zero16() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

// LDS placement of the 16-byte chunk c (0..1023) of a tile
template <bool KMAJ>
__device__ __forceinline__ int lds_chunk_off(int c) {
  if constexpr (KMAJ) return (c >> 3) * LDK + (c & 7) * 8;     // [128 rows][64 k]
  else return (c >> 4) * LDMN + (c & 15) * 8;                  // [64 k][128 cols]
}

// MFMA operand fragment (8 bf16 along k) of a 32-row block starting at row0
template <bool KMAJ>
__device__ __forceinline__ bf16x8 frag(const uint16_t* tile, int row0, int kk, int lane) {
  if constexpr (KMAJ) {
    const uint16_t* p = tile + (row0 + (lane & 31)) * LDK + kk * 16 + 8 * (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    const int k = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int m = row0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const uint16_t* p0 = tile + k * LDMN + m;
    const uint16_t* p1 = p0 + 4 * LDMN;
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
}

// Row and column (within the 128x128 tile) of accumulator element r of block (mb, nb)
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <class P>
__global__ void __launch_bounds__(NTHR, 2) gemm_kernel(const typename P::Args args) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE_ELEMS];
  P pol;
  if (!pol.init(args, xcd_remap(blockIdx.x, gridDim.x))) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = pol.nk;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    u32x4 ra[CHUNKS], rb[CHUNKS];
    pol.load_a(0, ra);
    pol.load_b(0, rb);
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      *reinterpret_cast<u32x4*>(smem + lds_chunk_off<P::A_KMAJ>(c)) = ra[i];
      *reinterpret_cast<u32x4*>(smem + TILE_ELEMS + lds_chunk_off<P::B_KMAJ>(c)) = rb[i];
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      uint16_t* sa = smem + (kt & 1) * 2 * TILE_ELEMS;
      uint16_t* sb = sa + TILE_ELEMS;
      const bool more = kt + 1 < nk;
      if (more) {
        pol.load_a(kt + 1, ra);
        pol.load_b(kt + 1, rb);
      }
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fa[mb] = frag<P::A_KMAJ>(sa, wm * 64 + mb * 32, kk, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) fb[nb] = frag<P::B_KMAJ>(sb, P::ncol0(wn, nb), kk, lane);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
      }
      if (more) {
        uint16_t* na = smem + ((kt + 1) & 1) * 2 * TILE_ELEMS;
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
          const int c = tid + i * NTHR;
          *reinterpret_cast<u32x4*>(na + lds_chunk_off<P::A_KMAJ>(c)) = ra[i];
          *reinterpret_cast<u32x4*>(na + TILE_ELEMS + lds_chunk_off<P::B_KMAJ>(c)) = rb[i];
        }
      }
      __syncthreads();
    }
  }
  pol.epilogue(acc, wm, wn, lane, smem);
}

// Column base of the 32-wide accumulator block nb of wave column wn (plain tiles)
struct PlainCols {
  __device__ static __forceinline__ int ncol0(int wn, int nb) { return wn * 64 + nb * 32; }
};

// ------------------------------------------------------------- row-grouped base
// Tile j of the routing's table: expert e, permuted rows [row0, row0 + rows).
struct RowTile {
  int e, row0, rows, n0, nk;
  __device__ __forceinline__ bool init_rows(const RowGroups& g, int logical, int n_ntiles) {
    const int j = logical / n_ntiles;
    const int nt = logical - j * n_ntiles;
    if (j >= g.tiles[0]) return false;
    e = g.tiles[2 + 2 * j];
    row0 = g.tiles[3 + 2 * j];
    rows = min(BM, g.offsets[e + 1] - row0);
    n0 = nt * BN;
    return true;
  }
};

// ------------------------------------------------------------- gmm1 + SwiGLU
struct Gmm1 : RowTile {
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  struct Args {
    RowGroups g;
    const uint16_t* x;
    const uint16_t* w1;
    const float* tw;
    int64_t H, I;
    uint16_t *h, *a, *aw;
    int n_ntiles;
  };
  const Args* ar;
  const uint16_t* arow[CHUNKS];
  const uint16_t* bbase;
  int i0;
  // the B tile holds 64 gate columns then the 64 matching up columns
  __device__ static __forceinline__ int ncol0(int wn, int nb) { return nb * 64 + wn * 32; }
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!init_rows(A.g, logical, A.n_ntiles)) return false;
    i0 = n0 / 2;  // 64 gate columns per tile
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int r = min(c >> 3, rows - 1);
      const int tok = A.g.sorted_slot[row0 + r] / A.g.K;
      arow[i] = A.x + (int64_t)tok * A.H + (c & 7) * 8;
    }
    bbase = A.w1 + (int64_t)e * A.H * 2 * A.I;
    nk = (int)(A.H / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[CHUNKS]) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = ld16(arow[i] + kt * BK);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[CHUNKS]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int kr = c >> 4, c8 = c & 15;
      const int64_t col = (c8 < 8) ? (i0 + c8 * 8) : (ar->I + i0 + (c8 - 8) * 8);
      r[i] = ld16(bbase + (int64_t)(kt * BK + kr) * 2 * ar->I + col);
    }
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[2][2], int wm, int wn, int lane, uint16_t* smem) {
    float* wrow = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x;
    if (tid < BM) wrow[tid] = (tid < rows) ? ar->tw[ar->g.sorted_slot[row0 + tid]] : 0.f;
    __syncthreads();
    const int64_t I = ar->I;
    const int64_t i = i0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rt = acc_row(wm, mb, r, lane);
        if (rt < rows) {
          const int64_t p = row0 + rt;
          const float g = round_bf(acc[mb][0][r]);
          const float u = round_bf(acc[mb][1][r]);
          const float av = round_bf(g * sigmoidf_(g) * u);
          const float awv = wrow[rt] * av;
          ar->h[p * 2 * I + i] = f2bf(g);
          ar->h[p * 2 * I + I + i] = f2bf(u);
          ar->a[p * I + i] = f2bf(av);
          ar->aw[p * I + i] = f2bf(awv);
        }
      }
  }
};

// ------------------------------------------------------------- gmm2
struct Gmm2 : RowTile, PlainCols {
  static constexpr bool A_KMAJ = true, B_KMAJ = false;
  struct Args {
    RowGroups g;
    const uint16_t* a;
    const uint16_t* w2;
    int64_t H, I;
    uint16_t* o;
    int n_ntiles;
  };
  const Args* ar;
  const uint16_t* arow[CHUNKS];
  const uint16_t* bbase;
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!init_rows(A.g, logical, A.n_ntiles)) return false;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int r = min(c >> 3, rows - 1);
      arow[i] = A.a + (int64_t)(row0 + r) * A.I + (c & 7) * 8;
    }
    bbase = A.w2 + (int64_t)e * A.I * A.H;
    nk = (int)(A.I / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[CHUNKS]) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = ld16(arow[i] + kt * BK);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[CHUNKS]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int kr = c >> 4, c8 = c & 15;
      const int64_t col = min((int64_t)(n0 + c8 * 8), ar->H - 8);
      r[i] = ld16(bbase + (int64_t)(kt * BK + kr) * ar->H + col);
    }
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[2][2], int wm, int wn, int lane, uint16_t*) {
    const int64_t H = ar->H;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t col = n0 + ncol0(wn, nb) + (lane & 31);
      if (col >= H) continue;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rt = acc_row(wm, mb, r, lane);
          if (rt < rows) ar->o[(int64_t)(row0 + rt) * H + col] = f2bf(acc[mb][nb][r]);
        }
    }
  }
};

// ------------------------------------------------------------- act_grad + SwiGLUGrad
struct ActGrad : RowTile, PlainCols {
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  struct Args {
    RowGroups g;
    const uint16_t* dy;
    const uint16_t* w2;
    const float* tw;
    const uint16_t* h;
    const uint16_t* a;
    int64_t H, I;
    uint16_t* dh;
    float* dwpart;
    int dw_cols;
    int n_ntiles;
  };
  const Args* ar;
  const uint16_t* arow[CHUNKS];
  const uint16_t* brow[CHUNKS];
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!init_rows(A.g, logical, A.n_ntiles)) return false;
    const int tid = threadIdx.x;
    const uint16_t* w2e = A.w2 + (int64_t)e * A.I * A.H;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int r = min(c >> 3, rows - 1);
      const int tok = A.g.sorted_slot[row0 + r] / A.g.K;
      arow[i] = A.dy + (int64_t)tok * A.H + (c & 7) * 8;
      const int64_t n = min((int64_t)(n0 + (c >> 3)), A.I - 1);
      brow[i] = w2e + n * A.H + (c & 7) * 8;
    }
    nk = (int)(A.H / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[CHUNKS]) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = ld16(arow[i] + kt * BK);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[CHUNKS]) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = ld16(brow[i] + kt * BK);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[2][2], int wm, int wn, int lane, uint16_t* smem) {
    float* wrow = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x;
    if (tid < BM) wrow[tid] = (tid < rows) ? ar->tw[ar->g.sorted_slot[row0 + tid]] : 0.f;
    __syncthreads();
    const int64_t I = ar->I;
    const int nt = n0 / BN;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rt = acc_row(wm, mb, r, lane);
        const bool rv = rt < rows;
        const int64_t p = row0 + (rv ? rt : 0);
        const float wp = wrow[rt];
        float part = 0.f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int64_t i = n0 + ncol0(wn, nb) + (lane & 31);
          if (rv && i < I) {
            const float G = acc[mb][nb][r];
            const float g = bf2f(ar->h[p * 2 * I + i]);
            const float u = bf2f(ar->h[p * 2 * I + I + i]);
            const float av = bf2f(ar->a[p * I + i]);
            part += G * av;
            const float dA = wp * G;
            const float s = sigmoidf_(g);
            const float dg = dA * u * s * (1.f + g * (1.f - s));
            const float du = dA * g * s;
            ar->dh[p * 2 * I + i] = f2bf(dg);
            ar->dh[p * 2 * I + I + i] = f2bf(du);
          }
        }
        // fixed-order butterfly over the 32 columns held by this half-wave
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 8);
        part += __shfl_xor(part, 4);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 1);
        if (rv && (lane & 31) == 0) ar->dwpart[p * ar->dw_cols + nt * 2 + wn] = part;
      }
  }
};

// ------------------------------------------------------------- input_grad
struct InputGrad : RowTile, PlainCols {
  static constexpr bool A_KMAJ = true, B_KMAJ = true;
  struct Args {
    RowGroups g;
    const uint16_t* dh;
    const uint16_t* w1;
    int64_t H, I;
    uint16_t* dxp;
    int n_ntiles;
  };
  const Args* ar;
  const uint16_t* arow[CHUNKS];
  const uint16_t* brow[CHUNKS];
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    if (!init_rows(A.g, logical, A.n_ntiles)) return false;
    const int tid = threadIdx.x;
    const uint16_t* w1e = A.w1 + (int64_t)e * A.H * 2 * A.I;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int r = min(c >> 3, rows - 1);
      arow[i] = A.dh + (int64_t)(row0 + r) * 2 * A.I + (c & 7) * 8;
      const int64_t n = min((int64_t)(n0 + (c >> 3)), A.H - 1);
      brow[i] = w1e + n * 2 * A.I + (c & 7) * 8;
    }
    nk = (int)(2 * A.I / BK);
    return true;
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[CHUNKS]) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = ld16(arow[i] + kt * BK);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[CHUNKS]) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = ld16(brow[i] + kt * BK);
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[2][2], int wm, int wn, int lane, uint16_t*) {
    const int64_t H = ar->H;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t col = n0 + ncol0(wn, nb) + (lane & 31);
      if (col >= H) continue;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rt = acc_row(wm, mb, r, lane);
          if (rt < rows) ar->dxp[(int64_t)(row0 + rt) * H + col] = f2bf(acc[mb][nb][r]);
        }
    }
  }
};

// ------------------------------------------------------------- weight gradients
// C[e][m][n] = sum over the expert's rows p of A[p][m] * B[p][n]; both operands
// are read along their row (m or n contiguous) and transposed by the LDS read.
struct DwBase : PlainCols {
  static constexpr bool A_KMAJ = false, B_KMAJ = false;
  int e, m0, n0, nk, p0, p1;
  __device__ __forceinline__ bool init_dw(const int32_t* offsets, int64_t E, int mt_count, int nt_count,
                                          int logical) {
    const int per_e = mt_count * nt_count;
    e = logical / per_e;
    if (e >= E) return false;
    const int rest = logical - e * per_e;
    m0 = (rest / nt_count) * BM;
    n0 = (rest % nt_count) * BN;
    p0 = offsets[e];
    p1 = offsets[e + 1];
    nk = (p1 - p0 + BK - 1) / BK;
    return true;
  }
};

template <bool GATHER_A, bool GATHER_B>
struct Dw : DwBase {
  struct Args {
    const int32_t* offsets;
    const int32_t* sorted_slot;
    int K;
    int64_t E;
    const uint16_t* A;  // [rows or tokens][M]
    const uint16_t* B;  // [rows or tokens][N]
    int64_t M, N;
    uint16_t* C;        // [E][M][N]
    int mt, nt;
  };
  const Args* ar;
  __device__ __forceinline__ bool init(const Args& A, int logical) {
    ar = &A;
    return init_dw(A.offsets, A.E, A.mt, A.nt, logical);
  }
  template <bool GATHER>
  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int64_t c0, int kt, u32x4 (&r)[CHUNKS]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + i * NTHR;
      const int kr = c >> 4, c8 = c & 15;
      const int p = p0 + kt * BK + kr;
      const int64_t col = c0 + c8 * 8;
      if (p < p1 && col < ld) {
        const int64_t row = GATHER ? (int64_t)(ar->sorted_slot[p] / ar->K) : (int64_t)p;
        r[i] = ld16(base + row * ld + col);
      } else {
        r[i] = zero16();
      }
    }
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[CHUNKS]) { load<GATHER_A>(ar->A, ar->M, m0, kt, r); }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[CHUNKS]) { load<GATHER_B>(ar->B, ar->N, n0, kt, r); }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[2][2], int wm, int wn, int lane, uint16_t*) {
    const int64_t M = ar->M, N = ar->N;
    uint16_t* C = ar->C + (int64_t)e * M * N;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t col = n0 + ncol0(wn, nb) + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + acc_row(wm, mb, r, lane);
          if (m < M) C[m * N + col] = f2bf(acc[mb][nb][r]);
        }
    }
  }
};

inline int64_t round8(int64_t n) { return (n + 7) / 8 * 8; }

template <class P>
hipError_t launch(const typename P::Args& args, int64_t logical_blocks, hipStream_t stream) {
  if (logical_blocks <= 0) return hipSuccess;
  const int64_t g = round8(logical_blocks);
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel<P>, dim3((unsigned)g), dim3(NTHR), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

int act_grad_dw_cols(int64_t I) { return (int)(2 * ((I + BN - 1) / BN)); }

hipError_t launch_gmm1_swiglu(const RowGroups& g, const uint16_t* x, const uint16_t* w1, const float* topk_w,
                              int64_t H, int64_t I, uint16_t* h, uint16_t* a, uint16_t* aw, hipStream_t stream) {
  Gmm1::Args A{g, x, w1, topk_w, H, I, h, a, aw, (int)(I / 64)};
  return launch<Gmm1>(A, g.max_tiles * A.n_ntiles, stream);
}

hipError_t launch_gmm2(const RowGroups& g, const uint16_t* a, const uint16_t* w2, int64_t H, int64_t I,
                       uint16_t* o, hipStream_t stream) {
  Gmm2::Args A{g, a, w2, H, I, o, (int)((H + BN - 1) / BN)};
  return launch<Gmm2>(A, g.max_tiles * A.n_ntiles, stream);
}

hipError_t launch_act_grad(const RowGroups& g, const uint16_t* dy, const uint16_t* w2, const float* topk_w,
                           const uint16_t* h, const uint16_t* a, int64_t H, int64_t I, uint16_t* dh,
                           float* dwpart, int dw_cols, hipStream_t stream) {
  ActGrad::Args A{g, dy, w2, topk_w, h, a, H, I, dh, dwpart, dw_cols, (int)((I + BN - 1) / BN)};
  return launch<ActGrad>(A, g.max_tiles * A.n_ntiles, stream);
}

hipError_t launch_input_grad(const RowGroups& g, const uint16_t* dh, const uint16_t* w1, int64_t H, int64_t I,
                             uint16_t* dxp, hipStream_t stream) {
  InputGrad::Args A{g, dh, w1, H, I, dxp, (int)((H + BN - 1) / BN)};
  return launch<InputGrad>(A, g.max_tiles * A.n_ntiles, stream);
}

hipError_t launch_dw1(const int32_t* offsets, const int32_t* sorted_slot, int K, int64_t E, const uint16_t* x,
                      const uint16_t* dh, int64_t H, int64_t I, uint16_t* dw1, hipStream_t stream) {
  typedef Dw<true, false> P;
  P::Args A{offsets, sorted_slot, K, E, x, dh, H, 2 * I, dw1, (int)((H + BM - 1) / BM), (int)((2 * I + BN - 1) / BN)};
  return launch<P>(A, E * A.mt * A.nt, stream);
}

hipError_t launch_dw2(const int32_t* offsets, const int32_t* sorted_slot, int K, int64_t E, const uint16_t* aw,
                      const uint16_t* dy, int64_t H, int64_t I, uint16_t* dw2, hipStream_t stream) {
  typedef Dw<false, true> P;
  P::Args A{offsets, sorted_slot, K, E, aw, dy, I, H, dw2, (int)((I + BM - 1) / BM), (int)((H + BN - 1) / BN)};
  return launch<P>(A, E * A.mt * A.nt, stream);
}

}  // namespace hmm
