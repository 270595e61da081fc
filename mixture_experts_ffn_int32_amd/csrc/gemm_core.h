// The main loop shared by the row-grouped and weight-gradient bf16 products:
// tile shapes, LDS layouts and fragment reads, the software pipeline, the LDS
// staged epilogue, the row-tile base and the launch helpers.  Every kernel file
// that includes it gets its own instantiations (anonymous namespace).
#pragma once

#include "device.h"
#include "gemm_common.h"
#include "kernels.h"

namespace hmm {
namespace {

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = BK_;                    // K step
  static constexpr int LDK = BK + 8;                // pitch of a K-major LDS tile (elements)
  static constexpr int KCH = BK / 8;                // 16-byte chunks per K-major row
  static constexpr int NTHR = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int MB = TM / 32, NB = TN / 32;  // 32x32 accumulator blocks per wave
  static constexpr int CA = BM * BK / 8 / NTHR;     // 16-byte chunks of A per thread per K step
  static constexpr int CB = BN * BK / 8 / NTHR;
  static constexpr int LDA_MN = BM + 32, LDB_MN = BN + 32;
  static constexpr int A_ELEMS = (BM * LDK > BK * LDA_MN) ? BM * LDK : BK * LDA_MN;
  static constexpr int B_ELEMS = (BN * LDK > BK * LDB_MN) ? BN * LDK : BK * LDB_MN;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static_assert(CA >= 1 && CB >= 1 && MB >= 1 && NB >= 1, "tile too small for the workgroup");
};
typedef Cfg<256, 256, 2, 4> Big;
typedef Cfg<64, 256, 2, 4> Small;
typedef Cfg<64, 64, 2, 2> Narrow;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS placement of 16-byte chunk c of a tile with R rows (K-major) or R columns (M/N-major)
template <class C, bool KMAJ, int R>
__device__ __forceinline__ int lds_chunk_off(int c) {
  if constexpr (KMAJ) return (int)((unsigned)c / C::KCH) * C::LDK + (int)((unsigned)c % C::KCH) * 8;  // [R rows][BK k]
  else return (c / (R / 8)) * (R + 32) + (c % (R / 8)) * 8;              // [BK k][R cols]
}

// MFMA operand fragment (8 bf16 along k) of a 32-row block starting at row0
template <class C, bool KMAJ, int R>
__device__ __forceinline__ bf16x8 frag(const uint16_t* tile, int row0, int kk, int lane) {
  if constexpr (KMAJ) {
    const uint16_t* p = tile + (row0 + (lane & 31)) * C::LDK + kk * 16 + 8 * (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(p);
  } else {
    constexpr int LD = R + 32;
    const int k = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int m = row0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const uint16_t* p0 = tile + k * LD + m;
    const uint16_t* p1 = p0 + 4 * LD;
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
}

// Row (within the tile) of accumulator element r of block mb of wave row wm
template <class C>
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * C::TM + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <class C, class P>
__device__ __forceinline__ void store_stage(uint16_t* st, const u32x4 (&ra)[C::CA], const u32x4 (&rb)[C::CB]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::CA; ++i)
    *reinterpret_cast<u32x4*>(st + lds_chunk_off<C, P::A_KMAJ, C::BM>(tid + i * C::NTHR)) = ra[i];
#pragma unroll
  for (int i = 0; i < C::CB; ++i)
    *reinterpret_cast<u32x4*>(st + C::A_ELEMS + lds_chunk_off<C, P::B_KMAJ, C::BN>(tid + i * C::NTHR)) = rb[i];
}

// The main loop of every bf16 product for tile ``idx`` (the index the policy's
// init takes); false if that tile does not exist.  The whole workgroup calls it.
template <class P>
__device__ __forceinline__ bool gemm_tile(const typename P::Args& args, int idx, uint16_t* smem) {
  typedef typename P::C C;
  P pol;
  if (!pol.init(args, idx)) return false;
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
    // Gathered operands take two phases per K step: fetch(k) issues the loads of
    // step k's row indices into the Raw set, index(k) turns them into offsets one
    // step later, so in the steady state no index load is waited for right after
    // it is issued (the memory counter is in order: such a wait would drain the
    // data loads issued before it too).  Inside the loop every load and LDS store
    // is unconditional (the last steps run in a tail after it): with a load under
    // a condition, the wait before the LDS stores at the top of the loop would
    // have to assume it was skipped and drain every load in flight.
    u32x4 ra0[C::CA], rb0[C::CB], ra1[C::CA], rb1[C::CB];
    typename P::Raw rw;
    const auto kc = [nk](int k) { return k < nk ? k : nk - 1; };
    pol.fetch(0, rw);
    pol.index(0, rw);
    pol.load_a(0, ra0);
    pol.load_b(0, rb0);
    pol.fetch(kc(1), rw);
    pol.index(kc(1), rw);
    pol.load_a(kc(1), ra1);
    pol.load_b(kc(1), rb1);
    store_stage<C, P>(smem, ra0, rb0);
    pol.fetch(kc(2), rw);
    pol.index(kc(2), rw);
    pol.load_a(kc(2), ra0);
    pol.load_b(kc(2), rb0);
    pol.fetch(kc(3), rw);
    __syncthreads();
    // one K step: turn the indices of step kt+3 (fetched one step ago) into
    // offsets and fetch those of step kt+4; multiply step kt, and after each of
    // its four 16-deep slices park a quarter of step kt+1 (register set `nx`) in
    // the other LDS buffer (so the stores are spread over the MFMAs instead of one
    // burst that the fragment reads of every wave would queue behind); then
    // refill `nx` with step kt+3.  ``full``: all of those steps exist (the loop),
    // else each is checked (the tail).
    auto step = [&](int kt, u32x4 (&nxa)[C::CA], u32x4 (&nxb)[C::CB], bool full) {
      // the backend's MFMA / LDS interleaving for small GEMM loops, where the
      // policy asks for it (measured: the bf16 row-grouped products 1-6% faster;
      // the weight gradients and the float32-mode products spill with it)
      if constexpr (P::SCHED_HINT) __builtin_amdgcn_iglp_opt(0);
      const bool st_ok = full || kt + 1 < nk, ld_ok = full || kt + 3 < nk;
      if (ld_ok) {
        pol.index(kt + 3, rw);
        pol.fetch(kc(kt + 4), rw);
      }
      uint16_t* dst = smem + ((kt + 1) & 1) * C::STAGE;
      const uint16_t* sa = smem + (kt & 1) * C::STAGE;
      const uint16_t* sb = sa + C::A_ELEMS;
      constexpr int NKK = C::BK / 16;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        bf16x8 fa[C::MB], fb[C::NB];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) fa[mb] = frag<C, P::A_KMAJ, C::BM>(sa, wm * C::TM + mb * 32, kk, lane);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) fb[nb] = frag<C, P::B_KMAJ, C::BN>(sb, P::ncol0(wn, nb), kk, lane);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
        if (st_ok) {
          const int t = threadIdx.x;
#pragma unroll
          for (int i = kk; i < C::CA; i += NKK)
            *reinterpret_cast<u32x4*>(dst + lds_chunk_off<C, P::A_KMAJ, C::BM>(t + i * C::NTHR)) = nxa[i];
#pragma unroll
          for (int i = kk; i < C::CB; i += NKK)
            *reinterpret_cast<u32x4*>(dst + C::A_ELEMS + lds_chunk_off<C, P::B_KMAJ, C::BN>(t + i * C::NTHR)) = nxb[i];
        }
      }
      if (ld_ok) {
        pol.load_a(kt + 3, nxa);
        pol.load_b(kt + 3, nxb);
      }
      __syncthreads();
    };
    // register set 1 holds odd steps, set 0 even steps; the loop runs while both
    // of its steps have a step 3 ahead, the tail (at most 4 steps) after it
    int kt = 0;
    for (; kt + 4 < nk; kt += 2) {
      step(kt, ra1, rb1, true);
      step(kt + 1, ra0, rb0, true);
    }
    if (kt < nk) step(kt, ra1, rb1, false);
    if (kt + 1 < nk) step(kt + 1, ra0, rb0, false);
    if (kt + 2 < nk) step(kt + 2, ra1, rb1, false);
    if (kt + 3 < nk) step(kt + 3, ra0, rb0, false);
  }
  pol.epilogue(acc, wm, wn, lane, smem);
  return true;
}

// ... for workgroup ``bid`` of its launch part (every policy's init maps the
// workgroup index onto its tiles and the XCDs itself)
template <class P>
__device__ __forceinline__ void gemm_body(const typename P::Args& args, int bid, uint16_t* smem) {
  (void)gemm_tile<P>(args, bid, smem);
}

template <class P>
__global__ void __launch_bounds__(P::C::NTHR, 1) gemm_kernel(const typename P::Args args) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * P::C::STAGE];
  gemm_body<P>(args, blockIdx.x, smem);
}

// Two independent products in one launch (small problems, where each fills only
// part of the chip): workgroups [0, n1) run P1, the others P2.  n1 is a multiple
// of 8, so both parts keep their workgroup-to-XCD mapping.
template <class P1, class P2>
__global__ void __launch_bounds__(P1::C::NTHR, 1) gemm_pair_kernel(const typename P1::Args a1, int n1,
                                                                   const typename P2::Args a2) {
  static_assert(P1::C::NTHR == P2::C::NTHR, "one workgroup size");
  constexpr int S1 = 2 * P1::C::STAGE, S2 = 2 * P2::C::STAGE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S1 > S2 ? S1 : S2];
  if ((int)blockIdx.x < n1)
    gemm_body<P1>(a1, blockIdx.x, smem);
  else
    gemm_body<P2>(a2, blockIdx.x - n1, smem);
}

// Four independent products in one launch (small problems with a shared
// expert): workgroups [s1, s2) run P2, [s2, s3) P3, [s3, end) P4, the first s1
// P1; every start is a multiple of 8.
template <class P1, class P2, class P3, class P4>
__global__ void __launch_bounds__(P1::C::NTHR, 1) gemm_quad_kernel(const typename P1::Args a1, int s1,
                                                                   const typename P2::Args a2, int s2,
                                                                   const typename P3::Args a3, int s3,
                                                                   const typename P4::Args a4) {
  static_assert(P1::C::NTHR == P2::C::NTHR && P1::C::NTHR == P3::C::NTHR && P1::C::NTHR == P4::C::NTHR,
                "one workgroup size");
  constexpr int S1 = 2 * P1::C::STAGE, S2 = 2 * P2::C::STAGE, S3 = 2 * P3::C::STAGE, S4 = 2 * P4::C::STAGE;
  constexpr int S12 = S1 > S2 ? S1 : S2, S34 = S3 > S4 ? S3 : S4;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S12 > S34 ? S12 : S34];
  const int b = blockIdx.x;
  if (b < s1)
    gemm_body<P1>(a1, b, smem);
  else if (b < s2)
    gemm_body<P2>(a2, b - s1, smem);
  else if (b < s3)
    gemm_body<P3>(a3, b - s2, smem);
  else
    gemm_body<P4>(a4, b - s3, smem);
}

// Plain epilogue: the tile's results, rounded to bf16, are staged in LDS as a
// [BM][BN] tile and written out as 16-byte row chunks (rows < valid_rows,
// columns < ncols), so every global store is a full, coalesced vector.
// A routing array element; with ``coh`` read at the device-wide coherence point
// (an agent-scope load, sc1: the array was written in the same launch, maybe on
// another XCD, and this XCD's L2 may still hold an older copy).
__device__ __forceinline__ int32_t get(const int32_t* p, bool coh) {
  return coh ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
}

// A 16-byte store of a result: streaming, or with ``coh`` to the device-wide
// coherence point (sc1, as an agent-scope store), for a consumer on another XCD
// in the same launch.  ``base``/``bytes`` describe the whole output array (below 4 GiB).
__device__ __forceinline__ void put16(uint16_t* base, int64_t bytes, int64_t elem, u32x4 v, bool coh) {
  if (coh)
    __builtin_amdgcn_raw_buffer_store_b128(v, make_rsrc(base, bytes), (uint32_t)(elem * 2), 0, 16);
  else
    store16_stream(base + elem, v);
}

template <class C, class P>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane, uint16_t* smem,
                                           uint16_t* out, int64_t ld, int64_t row_base, int valid_rows,
                                           int64_t col_base, int64_t ncols, bool coh = false, int64_t out_rows = 0) {
  constexpr int LD = C::BN + 8;
  static_assert(C::BM * LD <= 2 * C::STAGE, "staging tile must fit in the LDS buffers");
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        smem[acc_row<C>(wm, mb, r, lane) * LD + P::ncol0(wn, nb) + (lane & 31)] = f2bf(acc[mb][nb][r]);
  __syncthreads();
  constexpr int CPR = C::BN / 8;
  for (int c = threadIdx.x; c < C::BM * CPR; c += C::NTHR) {
    const int row = c / CPR, c8 = c % CPR;
    const int64_t col = col_base + c8 * 8;
    if (row < valid_rows && col < ncols)
      put16(out, out_rows * ld * 2, (row_base + row) * ld + col, *reinterpret_cast<const u32x4*>(smem + row * LD + c8 * 8),
            coh);
  }
}

// Column base (within the tile) of accumulator block nb of wave column wn
template <class C>
struct PlainCols {
  __device__ static __forceinline__ int ncol0(int wn, int nb) { return wn * C::TN + nb * 32; }
};

// ------------------------------------------------------------- row-grouped base
// Tile j of one of the routing's tables: expert e, permuted rows [row0, row0 + rows).
template <class Cc, bool SMALL>
struct RowTile {
  typedef Cc C;
  // init takes the workgroup index of its launch part.  Tiles of 256 columns
  // (large problems, many rounds of workgroups) and launches of more than
  // SPREAD_MIN_TILES tiles spread the table's real tiles over the XCDs
  // (real_tile; the count is loaded before the entry).  The others take the
  // XCD-remapped index over the table's capacity (the launch part's size) and load
  // the count and the entry together; inside the fused forward (coh) the index is
  // that kernel's own tile index, used as is.
  static constexpr bool SCHED_HINT = true;  // see gemm_tile
  int e, row0, rows, n0, nk, nt;
  struct Raw {};  // K-major rows are fixed for the whole tile: no per-step indices
  __device__ __forceinline__ void fetch(int, Raw&) {}
  __device__ __forceinline__ void index(int, Raw&) {}
  __device__ __forceinline__ bool init_rows(const RowGroups& g, int idx, int n_ntiles) {
    const int R = SMALL ? (int)g.max_small : (int)g.max_big;
    const int cap = R * n_ntiles;
    const int32_t* tab = g.tiles + 4 + (SMALL ? 2 * g.max_big : 0);
    int j;
    int32_t w;
    if (C::BN > 64 || (!g.coh && cap > SPREAD_MIN_TILES)) {
      // the count is at most the capacity R; clamped anyway, so entries j < cnt
      // are in bounds whatever the table holds
      const int cnt = min(get(g.tiles + (SMALL ? 1 : 0), g.coh), R);
      if (!real_tile(idx, cnt, n_ntiles, j, nt)) return false;
      w = get(tab + 2 * j, g.coh);
      row0 = get(tab + 2 * j + 1, g.coh);
    } else {
      const int logical = g.coh ? idx : xcd_remap(idx, (cap + 7) & ~7);
      if (logical >= cap) return false;
      raster(logical, R, n_ntiles, j, nt);
      // the count and the entry are loaded together (entries j < R are in bounds;
      // one past the count holds stale data and is not used)
      const int cnt = get(g.tiles + (SMALL ? 1 : 0), g.coh);
      w = get(tab + 2 * j, g.coh);
      row0 = get(tab + 2 * j + 1, g.coh);
      if (j >= cnt) return false;
    }
    e = tile_expert(w);
    rows = min(C::BM, tile_rows(w));
    n0 = nt * C::BN;
    if constexpr (EARLY_SLOT) {
      const int t = threadIdx.x;
      slot_own = (t < C::BM && t < rows) ? get(g.sorted_slot + row0 + t, g.coh) : 0;
    }
    return true;
  }
  // Small tiles: thread t < BM loads the routing slot of row t with the tile's
  // other row indices, so the epilogue's weight load no longer waits for a
  // dependent index load (a few microseconds of a small problem's launch).
  static constexpr bool EARLY_SLOT = C::BM <= 64;
  static_assert(!EARLY_SLOT || C::NTHR >= C::BM, "one thread per row of a small tile");
  int slot_own;
  // topk weight of the tile's row t (0 past the expert's rows); on small tiles
  // only for t == threadIdx.x
  __device__ __forceinline__ float row_weight(const float* tw, const RowGroups& g, int t) const {
    if (t >= rows) return 0.f;
    if constexpr (EARLY_SLOT) return tw[slot_own];
    else return tw[get(g.sorted_slot + row0 + t, g.coh)];
  }
  // K-major A rows of this tile: byte offset of chunk i (the tile's rows past the
  // expert's end repeat its last row; their results are not stored)
  template <bool GATHER>
  __device__ __forceinline__ void a_rows(const RowGroups& g, int64_t ld, uint32_t (&off)[C::CA]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int c = tid + i * C::NTHR;
      const int p = row0 + min((int)((unsigned)c / C::KCH), rows - 1);
      const int64_t row = GATHER ? (int64_t)get(g.tok_of_row + p, g.coh) : (int64_t)p;
      off[i] = (uint32_t)((row * ld + (int)((unsigned)c % C::KCH) * 8) * 2);
    }
  }
  // K-major B rows n0 + r (clamped to N - 1), offsets within the expert's slice
  __device__ __forceinline__ void b_rows(int64_t ld, int64_t N, uint32_t (&off)[C::CB]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int c = tid + i * C::NTHR;
      const int64_t n = min((int64_t)(n0 + (int)((unsigned)c / C::KCH)), N - 1);
      off[i] = (uint32_t)((n * ld + (int)((unsigned)c % C::KCH) * 8) * 2);
    }
  }
};

inline int64_t round8(int64_t n) { return (n + 7) / 8 * 8; }
template <class T>
struct TypeTag {
  typedef T type;
};

template <class P>
hipError_t launch(const typename P::Args& args, int64_t logical_blocks, hipStream_t stream) {
  if (logical_blocks <= 0) return hipSuccess;
  const int64_t g = round8(logical_blocks);
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel<P>, dim3((unsigned)g), dim3(P::C::NTHR), 0, stream, args);
  return hipGetLastError();
}

template <class P1, class P2>
hipError_t launch_pair(const typename P1::Args& a1, int64_t blocks1, const typename P2::Args& a2, int64_t blocks2,
                       hipStream_t stream) {
  if (blocks1 <= 0) return launch<P2>(a2, blocks2, stream);
  if (blocks2 <= 0) return launch<P1>(a1, blocks1, stream);
  const int64_t g1 = round8(blocks1), g = g1 + round8(blocks2);
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_pair_kernel<P1, P2>), dim3((unsigned)g), dim3(P1::C::NTHR), 0, stream, a1, (int)g1, a2);
  return hipGetLastError();
}

template <class P1, class P2, class P3, class P4>
hipError_t launch_quad(const typename P1::Args& a1, int64_t b1, const typename P2::Args& a2, int64_t b2,
                       const typename P3::Args& a3, int64_t b3, const typename P4::Args& a4, int64_t b4,
                       hipStream_t stream) {
  const int64_t s1 = round8(b1), s2 = s1 + round8(b2), s3 = s2 + round8(b3), g = s3 + round8(b4);
  if (g <= 0) return hipSuccess;
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_quad_kernel<P1, P2, P3, P4>), dim3((unsigned)g), dim3(P1::C::NTHR), 0, stream, a1, (int)s1,
                     a2, (int)s2, a3, (int)s3, a4);
  return hipGetLastError();
}

// A row-grouped product over n <= 2 jobs (the routed experts and the shared
// expert), which share every launch: big tiles, then small tiles; in narrow mode
// one launch of 64x64 tiles.  ntiles(job, BN) gives a job's N-tile count and
// fill(args, job, nnt) its policy arguments.
template <template <class, bool> class P, class NarrowC, class Job, class NTiles, class Fill>
hipError_t launch_rows_jobs(const Job* j, int n, NTiles ntiles, Fill fill, hipStream_t stream) {
  auto args = [&](auto tag, bool big, typename decltype(tag)::type::Args (&a)[2], int64_t (&blocks)[2]) {
    typedef typename decltype(tag)::type PP;
    for (int q = 0; q < n; ++q) {
      const int nnt = ntiles(j[q], PP::C::BN);
      fill(a[q], j[q], nnt);
      blocks[q] = (big ? j[q].g.max_big : j[q].g.max_small) * nnt;
    }
  };
  if (j[0].g.narrow) {
    typedef P<NarrowC, true> PN;
    typename PN::Args a[2];
    int64_t b[2] = {0, 0};
    args(TypeTag<PN>{}, false, a, b);
    return n == 1 ? launch<PN>(a[0], b[0], stream) : launch_pair<PN, PN>(a[0], b[0], a[1], b[1], stream);
  }
  // big and small tiles in one launch (both shapes have 8 waves): the small
  // tiles come last and fill the CUs the big tiles' last round leaves idle
  typedef P<Big, false> PB;
  typedef P<Small, true> PS;
  static_assert(Big::NTHR == Small::NTHR, "one workgroup size");
  typename PB::Args ab[2];
  typename PS::Args as[2];
  int64_t bb[2] = {0, 0}, bs[2] = {0, 0};
  args(TypeTag<PB>{}, true, ab, bb);
  args(TypeTag<PS>{}, false, as, bs);
  if (n == 1) return launch_pair<PB, PS>(ab[0], bb[0], as[0], bs[0], stream);
  return launch_quad<PB, PB, PS, PS>(ab[0], bb[0], ab[1], bb[1], as[0], bs[0], as[1], bs[1], stream);
}

// big-tile launch, then small-tile launch, of a row-grouped product (n_ntiles
// is a function of the tile width); in narrow mode one launch of 64x64 tiles
template <template <class, bool> class P, class NarrowC, class ArgsFill, class NTiles>
hipError_t launch_rows_c(const RowGroups& g, NTiles n_ntiles, ArgsFill fill, hipStream_t stream) {
  if (g.narrow) {
    typedef P<NarrowC, true> PN;
    typename PN::Args an;
    fill(an, n_ntiles(NarrowC::BN));
    return launch<PN>(an, g.max_small * n_ntiles(NarrowC::BN), stream);
  }
  typedef P<Big, false> PB;
  typedef P<Small, true> PS;
  typename PB::Args ab;
  fill(ab, n_ntiles(Big::BN));
  hipError_t e = launch<PB>(ab, g.max_big * n_ntiles(Big::BN), stream);
  if (e != hipSuccess) return e;
  typename PS::Args as;
  fill(as, n_ntiles(Small::BN));
  return launch<PS>(as, g.max_small * n_ntiles(Small::BN), stream);
}

}  // namespace
}  // namespace hmm
