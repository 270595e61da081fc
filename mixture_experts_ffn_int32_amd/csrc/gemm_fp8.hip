// FP8 (E4M3) up-projection with the SwiGLU epilogue, for the FP8 forward
// variant: per-token dynamic quantisation of the tokens (MoeDistributeDispatchV2,
// case 3) and per-(expert, column) quantisation of the up-projection weight
// feed v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 block scales); the float32
// accumulator is dequantised with the row and column factors before the bf16
// rounding of h, then a = silu(g) u and aw = w a as in the bf16 product.
//
// Same structure as the bf16 products: the routing's big (256-row) and small
// (64-row) tile tables, or 64x64 tiles on small problems; LDS double buffered
// with loads three K steps (of 128 bytes) ahead; grouped rasterisation with the
// XCD remap.  A (tokens, K-major, gathered) sits in LDS as [row][k] (pitch 144
// bytes) and is read 32 bytes per lane with two ds_read_b128; B (weights,
// N-major) sits as [k][n] (pitch BN+32 bytes, so the 8 k rows a 32-lane pass
// of ds_read_b64_tr_b8 touches fall in distinct banks) and is read with four
// transposing reads of 8 k each.  Lane l of a 32x32x64 operand holds row/column
// l % 32 and, in the instruction's own k order, k = 16 (l / 32) + 0..15 in bytes
// 0..15 and k = 32 + 16 (l / 32) + 0..15 in bytes 16..31: the instruction's
// first 32-k scale block is bytes 0..15 of both lane halves (checked on the GPU
// with one nonzero position at a time).
//
// MX variant (MoeDistributeDispatchV2 case 5): tokens and weights carry one
// E8M0 exponent per 32 elements along the hidden dimension, which is exactly
// the 32 k values one lane holds in one instruction, so the exponents go to the
// instruction's per-lane scale operands (lane l scales the instruction's k block
// l / 32, which is block 2 kk + l / 32 of the step's four: that byte of the
// step's exponent word of the lane's row or column), and the accumulator needs
// no dequantisation.  The exponents of a step (one 32-bit word per tile row and
// per tile column) are staged in LDS behind the operand tiles.
#include "device.h"
#include "gemm_common.h"
#include "kernels.h"

namespace hmm {
namespace {

constexpr int BKB = 128;   // k per step (bytes = fp8 elements)
constexpr int LDKB = 144;  // pitch of a K-major LDS tile (bytes)

// SETS: register sets of prefetched global data (2: loads run three K steps
// ahead of the MFMAs, 1: two steps; the 256x256 tile has no registers for two).
template <int BM_, int BN_, int WM_, int WN_, int SETS_>
struct F8Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, SETS = SETS_;
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MB = TM / 32, NB = TN / 32;
  static constexpr int CA = BM * BKB / 16 / NTHR;
  static constexpr int CB = BN * BKB / 16 / NTHR;
  static constexpr int LDB = BN + 32;
  // B N-major ([k][n], pitch LDB) or K-major ([n][k], pitch LDKB, the backward's weights)
  static constexpr int A_BYTES = BM * LDKB, B_BYTES = (BKB * LDB > BN * LDKB) ? BKB * LDB : BN * LDKB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(CA >= 1 && CB >= 1 && STAGE % 16 == 0, "tile shape");
};
typedef F8Cfg<256, 256, 2, 4, 1> Big8;
typedef F8Cfg<64, 256, 1, 4, 2> Small8;
typedef F8Cfg<64, 64, 2, 2, 2> Narrow8;
// per group: eight waves on a 64x256 tile, two per SIMD, so one wave's rescaling
// of its step sums overlaps the other's matrix instructions
typedef F8Cfg<64, 256, 2, 4, 2> Group8;

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <class C>
__device__ __forceinline__ int acc_row8(int wm, int mb, int r, int lane) {
  return wm * C::TM + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Row tile j of one of the routing's tables: expert, first row, rows, N tile, for
// workgroup ``idx`` of the launch.  Tiles of 256 columns (large problems) and
// launches of more than SPREAD_MIN_TILES tiles spread the table's real tiles over
// the XCDs (real_tile; the count is loaded before the entry); the others take the
// XCD-remapped index over the table's capacity (the grid) and load the count and
// the entry together.
template <class C, bool SMALL>
__device__ __forceinline__ bool f8_row_tile(const RowGroups& g, int idx, int n_ntiles, int& e, int& row0,
                                            int& rows, int& nt) {
  const int R = SMALL ? (int)g.max_small : (int)g.max_big;
  const int cap = R * n_ntiles;
  const int32_t* tab = g.tiles + 4 + (SMALL ? 2 * g.max_big : 0);
  int j;
  int32_t w;
  if (C::BN > 64 || cap > SPREAD_MIN_TILES) {
    const int cnt = min((int)g.tiles[SMALL ? 1 : 0], R);  // clamped: entries j < cnt are in bounds
    if (!real_tile(idx, cnt, n_ntiles, j, nt)) return false;
    w = tab[2 * j];
    row0 = tab[2 * j + 1];
  } else {
    const int logical = xcd_remap(idx, (cap + 7) & ~7);
    if (logical >= cap) return false;
    raster(logical, R, n_ntiles, j, nt);
    const int cnt = g.tiles[SMALL ? 1 : 0];
    w = tab[2 * j];
    row0 = tab[2 * j + 1];
    if (j >= cnt) return false;
  }
  e = tile_expert(w);
  rows = min(C::BM, tile_rows(w));
  return true;
}

// Q: 0 per-token scales (applied in the epilogue), 1 MX block exponents (fed to
// the instruction), 2 per-group float descales (applied to each K step's sums)
template <class C, bool SMALL, int Q = 0>
struct Gmm1F8 {
  static constexpr bool MX = Q == 1;
  static constexpr bool GROUP = Q == 2;
  struct Args {
    RowGroups g;
    const uint8_t* xq;   // [T][H] E4M3
    const float* dsx;    // [T] (per-token mode)
    const uint8_t* wq;   // [E][H][2I] E4M3
    const float* dsw;    // [E][2I] (per-token mode)
    const float* tw;
    int64_t T, H, I;
    uint16_t *h, *a, *aw;
    int n_ntiles;
    const uint8_t* xs = nullptr;  // [T][H/32] E8M0 (MX mode)
    const uint8_t* ws = nullptr;  // [E][2I][H/32] E8M0 (MX mode)
    const float* gsx = nullptr;   // [T][H/128] token descales (per-group mode)
    const float* gsw = nullptr;   // [E][H/128][2I] weight descales (per-group mode)
  };
  // MX: one exponent word per tile row and column per step; per group: one float
  // descale per tile row and column per step (a K step is one 128-deep group)
  static constexpr bool MX_ = MX;
  static constexpr bool GROUP_ = GROUP;
  static constexpr bool STAGED = MX || GROUP;
  static constexpr bool B_KMAJ_ = false;  // weights [H][2I]: N-major
  static constexpr int SCR = STAGED ? (C::BM + C::BN + C::NTHR - 1) / C::NTHR : 1;
  static constexpr int SC_BYTES = STAGED ? (C::BM + C::BN) * 4 : 0;
  const Args* ar;
  int e, row0, rows, nt, i0, nk;
  rsrc_t ra_, rb_, rsx_, rsw_;
  uint32_t aoff[C::CA], boff[C::CB], soff[SCR];

  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    const RowGroups& g = A.g;
    if (!f8_row_tile<C, SMALL>(g, idx, A.n_ntiles, e, row0, rows, nt)) return false;
    i0 = nt * (C::BN / 2);
    const int tid = threadIdx.x;
    ra_ = make_rsrc(A.xq, A.T * A.H);
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int c = tid + i * C::NTHR;
      const int p = row0 + min(c >> 3, rows - 1);
      aoff[i] = (uint32_t)((int64_t)g.tok_of_row[p] * A.H + (c & 7) * 16);
    }
    rb_ = make_rsrc(A.wq + (int64_t)e * A.H * 2 * A.I, A.H * 2 * A.I);
    constexpr int CPR = C::BN / 16, HALF = C::BN / 32;
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int c = tid + i * C::NTHR;
      const int kr = c / CPR, c16 = c % CPR;
      const int64_t gi = min((int64_t)(i0 + (c16 % HALF) * 16), A.I - 16);  // gate column (clamped)
      const int64_t col = (c16 < HALF) ? gi : A.I + gi;
      boff[i] = (uint32_t)(kr * 2 * A.I + col);
    }
    nk = (int)(A.H / BKB);
    if constexpr (GROUP) {
      static_assert(BKB == 128, "a K step is one quantisation group");
      const int64_t ng = A.H / BKB;
      rsx_ = make_rsrc(A.gsx, A.T * ng * 4);
      rsw_ = make_rsrc(A.gsw + (int64_t)e * ng * 2 * A.I, ng * 2 * A.I * 4);
#pragma unroll
      for (int j = 0; j < SCR; ++j) {
        const int idx = tid + j * C::NTHR;
        if (idx < C::BM) {
          soff[j] = (uint32_t)((int64_t)g.tok_of_row[row0 + min(idx, rows - 1)] * ng * 4);
        } else {
          const int n = min(idx - C::BM, C::BN - 1);
          const int64_t gi = min((int64_t)(i0 + n % (C::BN / 2)), A.I - 1);
          soff[j] = (uint32_t)(((n < C::BN / 2) ? gi : A.I + gi) * 4);
        }
      }
    }
    if constexpr (MX) {
      const int64_t nb = A.H / 32;  // exponent bytes per token row / weight column
      rsx_ = make_rsrc(A.xs, A.T * nb);
      rsw_ = make_rsrc(A.ws + (int64_t)e * 2 * A.I * nb, 2 * A.I * nb);
#pragma unroll
      for (int j = 0; j < SCR; ++j) {
        const int idx = tid + j * C::NTHR;
        if (idx < C::BM) {
          soff[j] = (uint32_t)((int64_t)g.tok_of_row[row0 + min(idx, rows - 1)] * nb);
        } else {
          const int n = min(idx - C::BM, C::BN - 1);
          const int64_t gi = min((int64_t)(i0 + n % (C::BN / 2)), A.I - 1);
          soff[j] = (uint32_t)(((n < C::BN / 2) ? gi : A.I + gi) * nb);
        }
      }
    }
    return true;
  }
  // MX: the exponent words of step kt (four blocks of 32 k) of this thread's rows / columns
  __device__ __forceinline__ void load_s(int kt, uint32_t (&r)[SCR]) {
    if constexpr (GROUP) {
      // group kt: the token descale at word kt of the row, the weight's at row kt of [H/128][2I]
      const int tid = threadIdx.x;
#pragma unroll
      for (int j = 0; j < SCR; ++j) {
        const int idx = tid + j * C::NTHR;
        if (idx < C::BM)
          r[j] = __builtin_amdgcn_raw_buffer_load_b32(rsx_, (int)soff[j], kt * 4, 0);
        else if (idx < C::BM + C::BN)
          r[j] = __builtin_amdgcn_raw_buffer_load_b32(rsw_, (int)soff[j], (int)(kt * 2 * ar->I * 4), 0);
      }
    }
    if constexpr (MX) {
      const int tid = threadIdx.x;
#pragma unroll
      for (int j = 0; j < SCR; ++j) {
        const int idx = tid + j * C::NTHR;
        if (idx < C::BM)
          r[j] = __builtin_amdgcn_raw_buffer_load_b32(rsx_, (int)soff[j], kt * 4, 0);
        else if (idx < C::BM + C::BN)
          r[j] = __builtin_amdgcn_raw_buffer_load_b32(rsw_, (int)soff[j], kt * 4, 0);
      }
    }
  }
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * BKB);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
    const uint32_t so = (uint32_t)(kt * BKB * 2 * ar->I);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], so);
  }

  // g, u = bf16(acc * dsx[token] * dsw[column]) staged in LDS, then as the bf16
  // product's epilogue: 8 columns of one row per thread, 16-byte stores.
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint8_t* smemb) {
    constexpr int LD = C::BN + 8;
    static_assert(C::BM * LD * 2 + (2 * C::BM + C::BN) * 4 <= 2 * C::STAGE, "staging must fit");
    uint16_t* smem = reinterpret_cast<uint16_t*>(smemb);
    float* wrow = reinterpret_cast<float*>(smemb + C::BM * LD * 2);
    float* rsc = wrow + C::BM;
    float* csc = rsc + C::BM;
    const int tid = threadIdx.x;
    const int64_t I = ar->I;
    // per-token mode: the row and column descales; MX: the instruction applied the
    // block exponents already; per group: every K step applied its descales
    for (int t = tid; t < C::BM; t += C::NTHR) {
      const bool v = t < rows;
      wrow[t] = v ? ar->tw[ar->g.sorted_slot[row0 + t]] : 0.f;
      rsc[t] = STAGED ? 1.f : (v ? ar->dsx[ar->g.tok_of_row[row0 + t]] : 0.f);
    }
    for (int t = tid; t < C::BN; t += C::NTHR) {
      const int64_t gi = i0 + (t % (C::BN / 2));
      const int64_t col = (t < C::BN / 2) ? gi : I + gi;
      csc[t] = STAGED ? 1.f : ((gi < I) ? ar->dsw[(int64_t)e * 2 * I + col] : 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row8<C>(wm, mb, r, lane);
          const int col = wn * C::TN + nb * 32 + (lane & 31);
          smem[row * LD + col] = f2bf(acc[mb][nb][r] * rsc[row] * csc[col]);
        }
    __syncthreads();
    constexpr int CPR = C::BN / 16;
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
      store16_stream(ar->a + p * I + i, pack8(av));
      store16_stream(ar->aw + p * I + i, pack8(aw));
    }
  }
};

template <class C, class P>
__device__ __forceinline__ void store_scales(uint8_t* st, const uint32_t (&rs)[P::SCR]) {
  if constexpr (P::STAGED) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < P::SCR; ++j) {
      const int idx = tid + j * C::NTHR;
      if (idx < C::BM + C::BN) reinterpret_cast<uint32_t*>(st + C::STAGE)[idx] = rs[j];
    }
  }
}

template <class C, class P>
__device__ __forceinline__ void store_stage8(uint8_t* st, const u32x4 (&ra)[C::CA], const u32x4 (&rb)[C::CB],
                                             int part = 0, int nparts = 1) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = part; i < C::CA; i += nparts) {
    const int c = tid + i * C::NTHR;
    *reinterpret_cast<u32x4*>(st + (c >> 3) * LDKB + (c & 7) * 16) = ra[i];
  }
#pragma unroll
  for (int i = part; i < C::CB; i += nparts) {
    const int c = tid + i * C::NTHR;
    if constexpr (P::B_KMAJ_)
      *reinterpret_cast<u32x4*>(st + C::A_BYTES + (c >> 3) * LDKB + (c & 7) * 16) = rb[i];
    else
      *reinterpret_cast<u32x4*>(st + C::A_BYTES + (c / (C::BN / 16)) * C::LDB + (c % (C::BN / 16)) * 16) = rb[i];
  }
}

template <class P>
__global__ void __launch_bounds__(P::NTHR_, 1) gemm_fp8_kernel(const typename P::Args args) {
  typedef typename P::Cc C;
  constexpr int ST = C::STAGE + P::SC_BYTES;  // one LDS stage: operand tiles, then the MX exponents
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * ST];
  P pol;
  if (!pol.init(args, (int)blockIdx.x)) return;  // init maps the workgroup onto its tile (f8_row_tile)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int nk = pol.nk;
  f32x16 acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    constexpr int AHEAD = C::SETS + 1;  // K steps between a load and its MFMAs
    // Inside the loops every load and LDS store is unconditional (the last steps
    // run in a tail), so the waits at the top of the loop can count on the loads
    // issued after the ones they wait for (see gemm_core.h).
    const auto kc = [nk](int k) { return k < nk ? k : nk - 1; };
    u32x4 ra0[C::CA], rb0[C::CB], ra1[C::SETS == 2 ? C::CA : 1], rb1[C::SETS == 2 ? C::CB : 1];
    uint32_t rs0[P::SCR], rs1[P::SCR];
    pol.load_s(0, rs0);
    pol.load_a(0, ra0);
    pol.load_b(0, rb0);
    if constexpr (C::SETS == 2) {
      pol.load_s(kc(1), rs1);
      pol.load_a(kc(1), ra1);
      pol.load_b(kc(1), rb1);
    }
    store_stage8<C, P>(smem, ra0, rb0);
    store_scales<C, P>(smem, rs0);
    pol.load_s(kc(AHEAD - 1), rs0);
    pol.load_a(kc(AHEAD - 1), ra0);
    pol.load_b(kc(AHEAD - 1), rb0);
    __syncthreads();
    // With two register sets the next stage's LDS stores are spread over the
    // MFMA slices of the step (see gemm_core.h) and the loads follow the last
    // slice.  With one (the 256x256 tile) that would keep the set live across the
    // MFMAs and spill: there the stores come first and the loads right after.
    constexpr bool SPREAD = C::SETS == 2;
    auto step = [&](int kt, auto& nxa, auto& nxb, auto& nxs, bool full) {
      const bool st_ok = full || kt + 1 < nk;
      uint8_t* dst = smem + ((kt + 1) & 1) * ST;
      if constexpr (!SPREAD) {
        if (st_ok) {
          store_stage8<C, P>(dst, nxa, nxb);
          store_scales<C, P>(dst, nxs);
        }
        if (full || kt + AHEAD < nk) {
          pol.load_s(kt + AHEAD, nxs);
          pol.load_a(kt + AHEAD, nxa);
          pol.load_b(kt + AHEAD, nxb);
        }
      } else {
        if (st_ok) store_scales<C, P>(dst, nxs);
      }
      const uint8_t* sa = smem + (kt & 1) * ST;
      const uint8_t* sb = sa + C::A_BYTES;
      const uint32_t* scl = reinterpret_cast<const uint32_t*>(sa + C::STAGE);
      // per group: this step's sums go to tmp, then into acc times the row's and the
      // column's descale (float32 products and sum, in group order)
      f32x16 tmp[P::GROUP_ ? C::MB : 1][P::GROUP_ ? C::NB : 1];
      if constexpr (P::GROUP_) {
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
          for (int j = 0; j < C::NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmp[i][j][r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < BKB / 64; ++kk) {
        // B fragments for the whole wave tile, then one A fragment at a time
        // (keeps the live fragment registers at NB + 1 operands)
        const int sh = 8 * (2 * kk + (lane >> 5));  // this lane's block among the step's four
        i32x8 fb[C::NB];
        int bsc[C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          if constexpr (P::B_KMAJ_) {
            // K-major B: read like the A fragments (same k order)
            const uint8_t* pb = sb + (wn * C::TN + nb * 32 + (lane & 31)) * LDKB + kk * 64 + 16 * (lane >> 5);
            const u32x4 lo = *reinterpret_cast<const u32x4*>(pb);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(pb + 32);
            fb[nb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          } else {
            const int i = lane & 15;
            const int n = wn * C::TN + nb * 32 + 16 * ((lane >> 4) & 1) + 8 * (i & 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int k = kk * 64 + 32 * (q >> 1) + 16 * (lane >> 5) + 8 * (q & 1) + (i >> 1);
              const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sb + k * C::LDB + n));
              fb[nb][2 * q] = v[0];
              fb[nb][2 * q + 1] = v[1];
            }
          }
          bsc[nb] = P::MX_ ? (int)(scl[C::BM + wn * C::TN + nb * 32 + (lane & 31)] >> sh) : 127;
        }
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const uint8_t* p = sa + (wm * C::TM + mb * 32 + (lane & 31)) * LDKB + kk * 64 + 16 * (lane >> 5);
          const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 32);
          const i32x8 fa = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          const int asc = P::MX_ ? (int)(scl[wm * C::TM + mb * 32 + (lane & 31)] >> sh) : 127;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) {
            if constexpr (P::GROUP_)
              tmp[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[nb], tmp[mb][nb], 0, 0, 0, asc, 0,
                                                                            bsc[nb]);
            else
              acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[nb], acc[mb][nb], 0, 0, 0, asc,
                                                                            0, bsc[nb]);
          }
        }
        if (SPREAD && st_ok) store_stage8<C, P>(dst, nxa, nxb, kk, BKB / 64);
      }
      if constexpr (P::GROUP_) {
        const float* gsc = reinterpret_cast<const float*>(scl);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const float cs = gsc[C::BM + wn * C::TN + nb * 32 + (lane & 31)];
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float rsv = gsc[acc_row8<C>(wm, mb, r, lane)];
              acc[mb][nb][r] = __builtin_fmaf(tmp[mb][nb][r], rsv * cs, acc[mb][nb][r]);
            }
        }
      }
      if (SPREAD && (full || kt + AHEAD < nk)) {
        pol.load_s(kt + AHEAD, nxs);
        pol.load_a(kt + AHEAD, nxa);
        pol.load_b(kt + AHEAD, nxb);
      }
      __syncthreads();
    };
    if constexpr (C::SETS == 2) {
      int kt = 0;
      for (; kt + AHEAD + 1 < nk; kt += 2) {
        step(kt, ra1, rb1, rs1, true);
        step(kt + 1, ra0, rb0, rs0, true);
      }
      if (kt < nk) step(kt, ra1, rb1, rs1, false);
      if (kt + 1 < nk) step(kt + 1, ra0, rb0, rs0, false);
      if (kt + 2 < nk) step(kt + 2, ra1, rb1, rs1, false);
      if (kt + 3 < nk) step(kt + 3, ra0, rb0, rs0, false);
    } else {
      int kt = 0;
      for (; kt + AHEAD < nk; ++kt) step(kt, ra0, rb0, rs0, true);
      for (; kt < nk; ++kt) step(kt, ra0, rb0, rs0, false);
    }
  }
  pol.epilogue(acc, wm, wn, lane, smem);
}

// ---------------------------------------------------------------- FP8 backward
// The dX chain's products on E4M3 (per-row dynamic scales of every operand): the
// row operand A is K-major as in the up-projection, the weight operand B is
// K-major too (a weight row of [I][H] or [H][2I] is contiguous along K).

// Row tile j of one of the routing's tables: expert, first row, rows, N tile.

// shared by both backward products: no per-step scales, K-major weights
template <class C>
struct F8BwdBase {
  typedef C Cc;
  static constexpr int NTHR_ = C::NTHR;
  static constexpr bool MX_ = false, GROUP_ = false, STAGED = false, B_KMAJ_ = true;
  static constexpr int SCR = 1, SC_BYTES = 0;
  int e, row0, rows, nt, n0, nk;
  rsrc_t ra_, rb_;
  uint32_t aoff[C::CA], boff[C::CB];
  __device__ __forceinline__ void load_s(int, uint32_t (&)[SCR]) {}
  __device__ __forceinline__ void load_a(int kt, u32x4 (&r)[C::CA]) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) r[i] = bload(ra_, aoff[i], kt * BKB);
  }
  __device__ __forceinline__ void load_b(int kt, u32x4 (&r)[C::CB]) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) r[i] = bload(rb_, boff[i], kt * BKB);
  }
  // B rows n0 + (c >> 3) (clamped to N - 1) of a [N][K] weight slice
  __device__ __forceinline__ void b_rows(int64_t K, int64_t N) {
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int c = threadIdx.x + i * C::NTHR;
      boff[i] = (uint32_t)(min((int64_t)(n0 + (c >> 3)), N - 1) * K + (c & 7) * 16);
    }
  }
  // the accumulators times the row's and the column's descale (staged in LDS)
  __device__ __forceinline__ void scale(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, const float* rsc,
                                        const float* csc) const {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const float cs = csc[wn * C::TN + nb * 32 + (lane & 31)];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][nb][r] = acc[mb][nb][r] * rsc[acc_row8<C>(wm, mb, r, lane)] * cs;
      }
  }
};

// act_grad: G = (dYq[tok] . W2q[e]^T) dsy[tok] dsw2[e][i], then SwiGLUGrad -> dH and
// the d_topk_weights partials, as the bf16 product's epilogue
template <class C, bool SMALL>
struct ActGradF8 : F8BwdBase<C> {
  typedef F8BwdBase<C> B_;
  using B_::e; using B_::row0; using B_::rows; using B_::nt; using B_::n0; using B_::nk;
  struct Args {
    RowGroups g;
    const uint8_t* dyq;  // [T][H] E4M3
    const float* dsy;    // [T]
    const uint8_t* w2q;  // [E][I][H] E4M3 (rows i)
    const float* dsw;    // [E][I]
    const float* tw;
    const uint16_t* h;
    int64_t T, H, I;
    uint16_t* dh;
    float* dwpart;
    int dw_cols;
    int n_ntiles;
  };
  const Args* ar;
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!f8_row_tile<C, SMALL>(A.g, idx, A.n_ntiles, e, row0, rows, nt)) return false;
    n0 = nt * C::BN;
    this->ra_ = make_rsrc(A.dyq, A.T * A.H);
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int c = threadIdx.x + i * C::NTHR;
      const int p = row0 + min(c >> 3, rows - 1);
      this->aoff[i] = (uint32_t)((int64_t)A.g.tok_of_row[p] * A.H + (c & 7) * 16);
    }
    this->rb_ = make_rsrc(A.w2q + (int64_t)e * A.I * A.H, A.I * A.H);
    this->b_rows(A.H, A.I);
    nk = (int)(A.H / BKB);
    return true;
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint8_t* smemb) {
    static_assert((sgrad_lds_floats<C>() + 2 * C::BM + C::BN) * 4 <= 2 * C::STAGE, "staging must fit");
    float* gst = reinterpret_cast<float*>(smemb);
    float* wrow = gst + sgrad_lds_floats<C>();
    float* rsc = wrow + C::BM;
    float* csc = rsc + C::BM;
    for (int t = threadIdx.x; t < C::BM; t += C::NTHR) {
      const bool v = t < rows;
      wrow[t] = v ? ar->tw[ar->g.sorted_slot[row0 + t]] : 0.f;
      rsc[t] = v ? ar->dsy[ar->g.tok_of_row[row0 + t]] : 0.f;
    }
    for (int t = threadIdx.x; t < C::BN; t += C::NTHR)
      csc[t] = (n0 + t < ar->I) ? ar->dsw[(int64_t)e * ar->I + n0 + t] : 0.f;
    __syncthreads();
    this->scale(acc, wm, wn, lane, rsc, csc);
    // the 256x256 tile (one register set) has no registers for the prefetch
    swiglu_grad_epilogue<C, C::SETS == 2>(acc, wm, wn, lane, gst, wrow, rows, row0, n0, ar->I, ar->h, ar->dh,
                                          ar->dwpart, ar->dw_cols);
  }
};

// input_grad: dXp = bf16((dHq[p] . W1q[e]^T) dsh[p] dsw1[e][h])
template <class C, bool SMALL>
struct InputGradF8 : F8BwdBase<C> {
  typedef F8BwdBase<C> B_;
  using B_::e; using B_::row0; using B_::rows; using B_::nt; using B_::n0; using B_::nk;
  struct Args {
    RowGroups g;
    const uint8_t* dhq;  // [S][2I] E4M3
    const float* dsh;    // [S]
    const uint8_t* w1q;  // [E][H][2I] E4M3 (rows h)
    const float* dsw;    // [E][H]
    int64_t S, H, I;
    uint16_t* dxp;
    int n_ntiles;
  };
  const Args* ar;
  __device__ __forceinline__ bool init(const Args& A, int idx) {
    ar = &A;
    if (!f8_row_tile<C, SMALL>(A.g, idx, A.n_ntiles, e, row0, rows, nt)) return false;
    n0 = nt * C::BN;
    const int64_t K = 2 * A.I;
    this->ra_ = make_rsrc(A.dhq, A.S * K);
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int c = threadIdx.x + i * C::NTHR;
      this->aoff[i] = (uint32_t)((int64_t)(row0 + min(c >> 3, rows - 1)) * K + (c & 7) * 16);
    }
    this->rb_ = make_rsrc(A.w1q + (int64_t)e * A.H * K, A.H * K);
    this->b_rows(K, A.H);
    nk = (int)(K / BKB);
    return true;
  }
  __device__ __forceinline__ void epilogue(f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint8_t* smemb) {
    constexpr int LD = C::BN + 8;
    static_assert(C::BM * LD * 2 + (C::BM + C::BN) * 4 <= 2 * C::STAGE, "staging must fit");
    uint16_t* st = reinterpret_cast<uint16_t*>(smemb);
    float* rsc = reinterpret_cast<float*>(smemb + C::BM * LD * 2);
    float* csc = rsc + C::BM;
    const int64_t H = ar->H;
    for (int t = threadIdx.x; t < C::BM; t += C::NTHR) rsc[t] = t < rows ? ar->dsh[row0 + t] : 0.f;
    for (int t = threadIdx.x; t < C::BN; t += C::NTHR)
      csc[t] = (n0 + t < H) ? ar->dsw[(int64_t)e * H + n0 + t] : 0.f;
    __syncthreads();
    this->scale(acc, wm, wn, lane, rsc, csc);
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st[acc_row8<C>(wm, mb, r, lane) * LD + wn * C::TN + nb * 32 + (lane & 31)] = f2bf(acc[mb][nb][r]);
    __syncthreads();
    constexpr int CPR = C::BN / 8;
    for (int c = threadIdx.x; c < C::BM * CPR; c += C::NTHR) {
      const int row = c / CPR, c8 = c % CPR;
      const int64_t col = n0 + c8 * 8;
      if (row < rows && col < H)
        store16_stream(ar->dxp + (int64_t)(row0 + row) * H + col, *reinterpret_cast<const u32x4*>(st + row * LD + c8 * 8));
    }
  }
};

template <class C, bool SMALL, int Q = 0>
struct Gmm1F8K : Gmm1F8<C, SMALL, Q> {
  typedef C Cc;
  static constexpr int NTHR_ = C::NTHR;
};

template <class T>
struct TypeTag8 {
  typedef T type;
};

template <class P>
hipError_t launch8(const typename P::Args& args, int64_t logical_blocks, hipStream_t stream) {
  if (logical_blocks <= 0) return hipSuccess;
  const int64_t g = (logical_blocks + 7) / 8 * 8;
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_fp8_kernel<P>, dim3((unsigned)g), dim3(P::NTHR_), 0, stream, args);
  return hipGetLastError();
}

template <class C, bool SMALL, int Q>
hipError_t launch_one(const RowGroups& g, const uint8_t* xq, const float* dsx, const uint8_t* wq, const float* dsw,
                      const uint8_t* xs, const uint8_t* ws, const float* tw, int64_t H, int64_t I, uint16_t* h,
                      uint16_t* a, uint16_t* aw, hipStream_t stream) {
  typedef Gmm1F8K<C, SMALL, Q> P;
  const int nnt = (int)((I + C::BN / 2 - 1) / (C::BN / 2));
  typename P::Args A{g, xq, dsx, wq, dsw, tw, g.T, H, I, h, a, aw, nnt, xs, ws};
  if constexpr (Q == 2) {
    A.gsx = dsx;
    A.gsw = dsw;
  }
  return launch8<P>(A, (SMALL ? g.max_small : g.max_big) * nnt, stream);
}

template <int Q>
hipError_t launch_all(const RowGroups& g, const uint8_t* xq, const float* dsx, const uint8_t* wq, const float* dsw,
                      const uint8_t* xs, const uint8_t* ws, const float* tw, int64_t H, int64_t I, uint16_t* h,
                      uint16_t* a, uint16_t* aw, hipStream_t stream) {
  if constexpr (Q == 2) {
    // per group: 64-row tiles only (two accumulator sets)
    if (!g.narrow) return hipErrorInvalidValue;
    return launch_one<Group8, true, Q>(g, xq, dsx, wq, dsw, xs, ws, tw, H, I, h, a, aw, stream);
  } else {
    if (g.narrow) return launch_one<Narrow8, true, Q>(g, xq, dsx, wq, dsw, xs, ws, tw, H, I, h, a, aw, stream);
    hipError_t e = launch_one<Big8, false, Q>(g, xq, dsx, wq, dsw, xs, ws, tw, H, I, h, a, aw, stream);
    if (e != hipSuccess) return e;
    return launch_one<Small8, true, Q>(g, xq, dsx, wq, dsw, xs, ws, tw, H, I, h, a, aw, stream);
  }
}

// big then small tiles (or narrow), one launch each
template <template <class, bool> class P, class Fill>
hipError_t launch_bwd8(const RowGroups& g, int64_t n_cols, Fill fill, hipStream_t stream) {
  auto one = [&](auto tag, bool small) -> hipError_t {
    typedef typename decltype(tag)::type PP;
    typename PP::Args a{};
    const int nnt = (int)((n_cols + PP::Cc::BN - 1) / PP::Cc::BN);
    fill(a, nnt);
    return launch8<PP>(a, (small ? g.max_small : g.max_big) * nnt, stream);
  };
  if (g.narrow) return one(TypeTag8<P<Narrow8, true>>{}, true);
  const hipError_t e = one(TypeTag8<P<Big8, false>>{}, false);
  return e != hipSuccess ? e : one(TypeTag8<P<Small8, true>>{}, true);
}

}  // namespace

hipError_t launch_act_grad_fp8(const RowGroups& g, const uint8_t* dyq, const float* dsy, const uint8_t* w2q,
                               const float* dsw2, const float* topk_w, const uint16_t* h, int64_t H, int64_t I,
                               uint16_t* dh, float* dwpart, int dw_cols, hipStream_t stream) {
  return launch_bwd8<ActGradF8>(g, I, [&](auto& A, int nnt) {
    A.g = g; A.dyq = dyq; A.dsy = dsy; A.w2q = w2q; A.dsw = dsw2; A.tw = topk_w; A.h = h;
    A.T = g.T; A.H = H; A.I = I; A.dh = dh; A.dwpart = dwpart; A.dw_cols = dw_cols; A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_input_grad_fp8(const RowGroups& g, const uint8_t* dhq, const float* dsh, const uint8_t* w1q,
                                 const float* dsw1, int64_t H, int64_t I, uint16_t* dxp, hipStream_t stream) {
  return launch_bwd8<InputGradF8>(g, H, [&](auto& A, int nnt) {
    A.g = g; A.dhq = dhq; A.dsh = dsh; A.w1q = w1q; A.dsw = dsw1; A.S = g.S; A.H = H; A.I = I; A.dxp = dxp;
    A.n_ntiles = nnt;
  }, stream);
}

hipError_t launch_gmm1_fp8(const RowGroups& g, const uint8_t* xq, const float* dsx, const uint8_t* wq,
                           const float* dsw, const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                           uint16_t* aw, hipStream_t stream) {
  return launch_all<0>(g, xq, dsx, wq, dsw, nullptr, nullptr, topk_w, H, I, h, a, aw, stream);
}

hipError_t launch_gmm1_group(const RowGroups& g, const uint8_t* xq, const float* dsx, const uint8_t* wq,
                             const float* dsw, const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                             uint16_t* aw, hipStream_t stream) {
  return launch_all<2>(g, xq, dsx, wq, dsw, nullptr, nullptr, topk_w, H, I, h, a, aw, stream);
}

hipError_t launch_gmm1_mx(const RowGroups& g, const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, const float* topk_w, int64_t H, int64_t I, uint16_t* h, uint16_t* a,
                          uint16_t* aw, hipStream_t stream) {
  return launch_all<1>(g, xq, nullptr, wq, nullptr, xs, ws, topk_w, H, I, h, a, aw, stream);
}

}  // namespace hmm
