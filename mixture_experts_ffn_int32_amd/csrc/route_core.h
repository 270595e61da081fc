// Routing of a small problem (S <= RT_ONE_MAX_SLOTS, E <= RT_ONE_MAX_EXPERTS) by
// ONE workgroup of NT threads, for the one-workgroup routing kernel and for the
// fused small-problem forward.  Same results as route_hist + route_scan +
// route_scatter (the stable (expert, slot) order).
#pragma once

#include "device.h"
#include "kernels.h"

namespace hmm {

// The same steps in ONE workgroup, for S <= RT_ONE_MAX_SLOTS and E <=
// RT_ONE_MAX_EXPERTS.  Wave w owns a contiguous chunk of slots and walks it 64
// slots at a time; a ballot multisplit over the id bits gives every slot its
// rank among the equal ids of its 64 and their count, so each wave keeps exact
// per-expert counts of its chunk in LDS without atomics.  Prefix sums over the
// waves (per expert) and over the experts then give every slot its row:
//   row = offsets[e] + (slots of e in earlier waves) + (earlier slots of e in
//   this wave's chunk) + rank,
// which is the stable (expert, slot) order.  Four barriers in all.
template <int NT>
struct RouteLds {
  static constexpr int NW = NT / 64;
  int32_t cntw[NW][RT_ONE_MAX_EXPERTS];  // per wave counts, then their exclusive prefix
  int32_t offs[RT_ONE_MAX_EXPERTS];
  int32_t wtot[3][RT_ONE_MAX_EXPERTS / 64];
};

// A routing output written by route_block: with COH the store goes to the
// device-wide coherence point (an agent-scope store; no L2 write-back needed
// before another XCD may read it), else a plain store.
template <bool COH>
__device__ __forceinline__ void put(int32_t* p, int32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

template <int NT, bool COH = false>
__device__ __forceinline__ void route_block(RouteLds<NT>& L, const int32_t* __restrict__ ids, int64_t S, int E, int K,
                                            int nbits, int max_big, int big_on, int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                                            int32_t* __restrict__ row_of_slot, int32_t* __restrict__ tok_of_row,
                                            int32_t* __restrict__ tiles, int32_t* __restrict__ err,
                                            int32_t* __restrict__ host_err) {
  constexpr int NW = NT / 64;
  constexpr int R = RT_ONE_MAX_SLOTS / NT;     // 64-slot rounds per wave at most
  constexpr int SW = RT_ONE_MAX_EXPERTS / 64;  // waves that hold one expert each in the scan
  static_assert(RT_ONE_MAX_EXPERTS % 64 == 0 && SW <= NW, "scan layout");
  int32_t (&cntw)[NW][RT_ONE_MAX_EXPERTS] = L.cntw;
  int32_t (&offs)[RT_ONE_MAX_EXPERTS] = L.offs;
  int32_t (&wtot)[3][SW] = L.wtot;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  for (int i = tid; i < NW * RT_ONE_MAX_EXPERTS; i += NT) (&cntw[0][0])[i] = 0;
  __syncthreads();

  // phase 1: per-wave counts; every slot keeps (id, rank, count of its id in its 64)
  const int64_t chunk = ((S + NW - 1) / NW + 63) / 64 * 64;
  const int64_t s0 = (int64_t)w * chunk;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ev[R], rc[R];  // id; rank | count << 8 (both <= 64)
  int bad = 0;
  // every round's id load is issued before the first ballot needs one, so the
  // wave waits for its loads once, not once per round
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t s = s0 + j * 64 + lane;
    ev[j] = ((j * 64 < chunk) && s < S) ? ids[s] : -1;
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    rc[j] = 0;
    if (j * 64 >= chunk) continue;  // past the chunk (the same for every wave): no ballots
    const int64_t s = s0 + j * 64 + lane;
    const bool in = s < S;
    int e = ev[j];
    const bool valid = in && e >= 0 && e < E;
    bad |= (in && !valid);
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    if (!valid) {
      peers = 0;
      e = in ? -2 : -1;  // -2: a real slot with an invalid id
    }
    ev[j] = e;
    const int rk = __popcll(peers & lt_mask), cn = __popcll(peers);
    rc[j] = rk | (cn << 8);
    if (valid && rk == 0) cntw[w][e] += cn;  // one leader per distinct id: no conflicts
  }
  bad = __syncthreads_or(bad);
  if (tid == 0) {
    put<COH>(err, bad);
    // the host only reads this word after the kernel has completed: no release needed
    if (host_err) __hip_atomic_store(host_err, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }

  // per expert: exclusive prefix over the waves, total count
  int c = 0;
  if (tid < E) {
    int v[NW];  // all reads issued before the first write
#pragma unroll
    for (int q = 0; q < NW; ++q) v[q] = cntw[q][tid];
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      cntw[q][tid] = c;
      c += v[q];
    }
  }
  // offsets and tile tables (the rule of route_scan): inclusive scans over the experts,
  // inside each wave with shuffles, then across the SW waves through LDS
  const int rem = big_on ? c % TILE_BIG : c;
  const int nbig = (tid < E && big_on) ? c / TILE_BIG + (rem > TILE_BIG / 2 ? 1 : 0) : 0;
  const int nsmall = (tid < E && !(big_on && rem > TILE_BIG / 2)) ? (rem + TILE_SMALL - 1) / TILE_SMALL : 0;
  int ic = c, ib = nbig, is = nsmall;
  if (w < SW) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int vc = __shfl_up(ic, d), vb = __shfl_up(ib, d), vs = __shfl_up(is, d);
      if (lane >= d) {
        ic += vc;
        ib += vb;
        is += vs;
      }
    }
    if (lane == 63) {
      wtot[0][w] = ic;
      wtot[1][w] = ib;
      wtot[2][w] = is;
    }
  }
  __syncthreads();
  if (w < SW) {
    for (int q = 0; q < w; ++q) {
      ic += wtot[0][q];
      ib += wtot[1][q];
      is += wtot[2][q];
    }
    if (tid < E) {
      const int off = ic - c;
      const int b0 = ib - nbig;
      const int sm0 = is - nsmall;
      put<COH>(counts + tid, c);
      put<COH>(offsets + tid, off);
      offs[tid] = off;
      for (int i = 0; i < nbig; ++i) {
        put<COH>(tiles + 4 + 2 * (b0 + i), tile_word(tid, min(TILE_BIG, c - i * TILE_BIG)));
        put<COH>(tiles + 4 + 2 * (b0 + i) + 1, off + i * TILE_BIG);
      }
      int32_t* small = tiles + 4 + 2 * max_big;
      const int srow = off + nbig * TILE_BIG;
      for (int i = 0; i < nsmall; ++i) {
        put<COH>(small + 2 * (sm0 + i), tile_word(tid, min(TILE_SMALL, c - nbig * TILE_BIG - i * TILE_SMALL)));
        put<COH>(small + 2 * (sm0 + i) + 1, srow + i * TILE_SMALL);
      }
    }
    if (tid == SW * 64 - 1) {  // holds the totals over all experts
      put<COH>(offsets + E, ic);
      put<COH>(tiles, ib);
      put<COH>(tiles + 1, is);
      put<COH>(tiles + 2, TILE_BIG);
      put<COH>(tiles + 3, TILE_SMALL);
    }
  }
  __syncthreads();

  // phase 2: rows; cntw[w][e] runs through the earlier slots of e in this chunk
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * 64 >= chunk) continue;
    const int64_t s = s0 + j * 64 + lane;
    const int e = ev[j];
    const int rk = rc[j] & 0xff, cn = rc[j] >> 8;
    if (e >= 0) {
      const int row = offs[e] + cntw[w][e] + rk;
      put<COH>(sorted_slot + row, (int32_t)s);
      put<COH>(tok_of_row + row, (int32_t)(s / K));
      put<COH>(row_of_slot + s, row);
    } else if (e == -2) {
      put<COH>(row_of_slot + s, -1);
    }
    // every lane has read cntw before a leader updates it (the wave runs in lockstep,
    // and the read above precedes this write in program order)
    if (e >= 0 && rk == 0) cntw[w][e] += cn;
  }
}

}  // namespace hmm
