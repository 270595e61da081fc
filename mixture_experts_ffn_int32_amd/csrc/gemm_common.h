// Helpers shared by the grouped-product kernels (bf16 and FP8): workgroup to
// XCD mapping, tile rasterisation, buffer resources, the act_grad epilogue.
#pragma once

#include "device.h"

namespace hmm {

constexpr int GROUP_M = 8;  // row tiles per rasterisation group

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // nblocks is a multiple of 8; workgroups are dealt to the 8 XCDs round robin
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

// logical index -> (row tile r, column tile c) of an R x C grid, walking groups
// of GROUP_M row tiles column by column (a bijection on [0, R*C))
__device__ __forceinline__ void raster(int idx, int R, int C, int& r, int& c) {
  const int per_group = GROUP_M * C;
  const int g = idx / per_group;
  const int first = g * GROUP_M;
  const int gsz = min(GROUP_M, R - first);
  const int w = idx - g * per_group;
  r = first + w % gsz;
  c = w / gsz;
}

// Workgroup ``bid`` of a launch part (whose first workgroup sits on XCD 0 and
// whose size is a multiple of 8 and at least cnt * C) -> tile (row tile r, column
// tile c) of the cnt x C tiles a routing table really holds.  Each XCD takes an
// equal contiguous share of them in raster order, however much of the table's
// capacity (which sizes the launch) they fill; a share of the capacity instead
// would leave the XCDs past the real tiles idle.  False past the XCD's share.
__device__ __forceinline__ bool real_tile(int bid, int cnt, int C, int& r, int& c) {
  const int n = cnt * C;
  const int share = (n + 7) >> 3;
  const int i = bid >> 3;
  const int logical = (bid & 7) * share + i;
  if (i >= share || logical >= n) return false;
  raster(logical, cnt, C, r, c);
  return true;
}

// Row-grouped launches of more than this many tiles (the table's capacity times
// the column tiles) spread the real tiles with real_tile even on 64x64 tiles;
// smaller ones run in about one round of workgroups, where the extra dependent
// load of the count would cost more than the balance gains.
constexpr int SPREAD_MIN_TILES = 1024;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// buffer resource over [base, base + bytes); bytes < 2^32
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// the same at the device-wide coherence point (sc1), for data written earlier in the same launch
__device__ __forceinline__ u32x4 bload_coh(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 16));
}

// ------------------------------------------------------------- act_grad epilogue
// SwiGLUGrad of one tile of G (fp32 accumulators), wave by wave: each wave stages
// one 32-row block of its own G at a time in a private LDS block (32 x (TN + 4)
// floats), then its lanes take 8 consecutive columns of one row each, read g and
// u as 16-byte chunks, write dH = [dg | du] as 16-byte chunks and add their share
// of sum_i G a.  No workgroup barrier separates the blocks, and each wave loads a
// block's g and u while it computes the block before (PF).  a = bf16(silu(g) u)
// is recomputed from g and u with the forward epilogue's float operations, so it
// is the forward's a bit for bit, without a third load.  The row sums are reduced
// in a fixed order (8-lane butterfly inside a wave column, then the wave columns in
// order, through LDS): one partial per (row, N tile) into dwpart (if not NULL).  wrow [BM] holds the
// rows' topk weights (0 past the tile's rows), written by the caller before the
// call (the first barrier here publishes it).  Shared by the bf16 and FP8 products.
//
// LDS: the waves' staging blocks, then the row sums [BM][WN]; the caller's own
// arrays (wrow, ...) go after sgrad_lds_floats<C>() floats.
template <class C>
constexpr int sgrad_lds_floats() { return (C::NTHR / 64) * 32 * (C::TN + 4) + C::BM * C::WN; }

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// PF: load each block's g and u one block ahead (two blocks of chunks in
// registers); without, right before the block (for tiles with no registers to spare).
template <class C, bool PF = true>
__device__ __forceinline__ void swiglu_grad_epilogue(const f32x16 (&acc)[C::MB][C::NB], int wm, int wn, int lane,
                                                     float* lds, const float* wrow, int rows, int64_t row0,
                                                     int64_t n0, int64_t I, const uint16_t* hbuf,
                                                     uint16_t* dhbuf, float* dwpart, int dw_cols) {
  constexpr int LDF = C::TN + 4;                      // float pitch of a staged block
  constexpr int CPR = C::TN / 8;                      // 8-column chunks per row of a wave tile
  constexpr int KP = 32 * CPR / 64;                   // chunks per lane per 32-row block
  static_assert(32 * CPR % 64 == 0 && 64 % CPR == 0 && C::TM % 32 == 0, "chunk mapping");
  float* gst = lds + (threadIdx.x >> 6) * 32 * LDF;   // this wave's staging block
  float* rsum = lds + (C::NTHR / 64) * 32 * LDF;      // [BM][WN]
  // g and u of a block, as 16-byte chunks; the loads are unconditional, at a
  // clamped row and column for lanes past the tile's rows or past I (results
  // unused), so no wait has to assume a skipped load and drain the others.
  u32x4 hb[2][2 * KP];
  auto load_block = [&](int mb, u32x4 (&buf)[2 * KP]) {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int c = lane + 64 * k;
      const int row = min(wm * C::TM + mb * 32 + c / CPR, rows - 1);
      const int64_t i = min(n0 + wn * C::TN + (c % CPR) * 8, I - 8);
      const uint16_t* q = hbuf + (row0 + row) * 2 * I + i;
      buf[2 * k] = *reinterpret_cast<const u32x4*>(q);
      buf[2 * k + 1] = *reinterpret_cast<const u32x4*>(q + I);
    }
  };
  if constexpr (PF) load_block(0, hb[0]);
  __syncthreads();  // wrow is published, and the main loop is done with the LDS
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    if constexpr (PF) {
      if (mb + 1 < C::MB) load_block(mb + 1, hb[(mb + 1) & 1]);
    } else {
      load_block(mb, hb[mb & 1]);
    }
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        gst[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * LDF + nb * 32 + (lane & 31)] = acc[mb][nb][r];
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int c = lane + 64 * k;
      const int rr = c / CPR, c8 = c % CPR;
      const int row = wm * C::TM + mb * 32 + rr;
      const int64_t i = n0 + wn * C::TN + c8 * 8;
      float s = 0.f;
      if (row < rows && i < I) {
        const int64_t p = row0 + row;
        float g[8], u[8], av[8], dg[8], du[8];
        unpack8(hb[mb & 1][2 * k], g);
        unpack8(hb[mb & 1][2 * k + 1], u);
        const float w = wrow[row];
        const float* G = gst + rr * LDF + c8 * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float sg = sigmoidf_(g[j]);
          av[j] = round_bf(g[j] * sg * u[j]);  // as the up-projection's epilogue forms a
          s += G[j] * av[j];
          const float dA = w * G[j];
          dg[j] = dA * u[j] * sg * (1.f + g[j] * (1.f - sg));
          du[j] = dA * g[j] * sg;
        }
        store16_stream(dhbuf + p * 2 * I + i, pack8(dg));
        store16_stream(dhbuf + p * 2 * I + I + i, pack8(du));
      }
      // the CPR lanes of a row are consecutive: fixed-order butterfly
#pragma unroll
      for (int d = CPR / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d);
      if (c8 == 0) rsum[row * C::WN + wn] = s;
    }
    wave_lds_sync();  // every lane has read the block before the next one is staged
  }
  __syncthreads();
  if (dwpart) {
    for (int t = threadIdx.x; t < rows && t < C::BM; t += C::NTHR) {
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < C::WN; ++q) part += rsum[t * C::WN + q];
      dwpart[(row0 + t) * dw_cols + n0 / C::BN] = part;
    }
  }
}

}  // namespace hmm
