// Routing: top-k expand, per-expert int32 histogram, exclusive prefix offsets,
// stable scatter of slots into expert order, and the tile table of the grouped
// products.  (HyperMegaMoE RFC section 4.1: each token expands into K expert
// slots; section 3.1: offsets are built inside the operator; section 6.2:
// slots are sorted by expert and un-sorted afterwards.)
//
// Slot s = t*K + k.  Three kernels, all integer and deterministic (a small
// problem runs the same steps in one workgroup, route_one):
//   route_hist     one block per RT_SLOTS slots: LDS histogram -> blockhist[b][e]
//   route_scan     one block: counts, per-block bases, offsets, tile tables
//   route_scatter  one block per RT_SLOTS slots: stable rank inside the block
//                  (wave multisplit over the id bits with ballots, then a
//                  fixed-order sum over the waves) -> sorted_slot, row_of_slot,
//                  and the token of every permuted row (tok_of_row)
#include "device.h"
#include "kernels.h"
#include "route_core.h"

namespace hmm {

// The shared expert's tables (RFC section 6.1: the shared expert runs through
// the same grouped products as one more group), written by the routing launch
// alongside the routed tables: one expert that holds every token, in token
// order, with the tile table of one expert with T rows under route_scan's rule.
__device__ __forceinline__ void shared_counts(const SharedTables& st, int64_t& nbig, int64_t& nsmall) {
  const int64_t rem = st.big_on ? st.T % TILE_BIG : st.T;
  const bool big_tail = st.big_on && rem > TILE_BIG / 2;
  nbig = st.big_on ? st.T / TILE_BIG + (big_tail ? 1 : 0) : 0;
  nsmall = big_tail ? 0 : (rem + TILE_SMALL - 1) / TILE_SMALL;
}
// entry i of the row arrays and tile lists (i < T; #big and #small are at most T)
__device__ __forceinline__ void shared_entry(const SharedTables& st, int64_t i) {
  int64_t nbig, nsmall;
  shared_counts(st, nbig, nsmall);
  if (i >= st.T) return;
  st.idx[i] = (int32_t)i;
  st.ones[i] = 1.f;
  if (i < nbig) {
    st.tiles[4 + 2 * i] = tile_word(0, (int)min((int64_t)TILE_BIG, st.T - i * TILE_BIG));
    st.tiles[4 + 2 * i + 1] = (int32_t)(i * TILE_BIG);
  }
  if (i < nsmall) {
    int32_t* small = st.tiles + 4 + 2 * (int64_t)st.max_big;
    const int64_t r0 = nbig * TILE_BIG + i * TILE_SMALL;
    small[2 * i] = tile_word(0, (int)min((int64_t)TILE_SMALL, st.T - r0));
    small[2 * i + 1] = (int32_t)r0;
  }
}
__device__ __forceinline__ void shared_header(const SharedTables& st) {
  int64_t nbig, nsmall;
  shared_counts(st, nbig, nsmall);
  st.offsets[0] = 0;
  st.offsets[1] = (int32_t)st.T;
  st.tiles[0] = (int32_t)nbig;
  st.tiles[1] = (int32_t)nsmall;
  st.tiles[2] = TILE_BIG;
  st.tiles[3] = TILE_SMALL;
}

__global__ void __launch_bounds__(RT_THREADS) route_hist(const int32_t* __restrict__ ids, int64_t S, int E,
                                                         int32_t* __restrict__ blockhist,
                                                         int32_t* __restrict__ blockerr, const SharedTables st) {
  __shared__ int32_t hist[MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += RT_THREADS) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RT_SLOTS;
  int bad = 0;
#pragma unroll
  for (int r = 0; r < RT_SLOTS / RT_THREADS; ++r) {
    const int64_t s = base + r * RT_THREADS + tid;
    if (s < S) {
      const int e = ids[s];
      if (e >= 0 && e < E)
        atomicAdd(&hist[e], 1);
      else
        bad = 1;
    }
  }
  bad = __syncthreads_or(bad);
  for (int e = tid; e < E; e += RT_THREADS) blockhist[(int64_t)blockIdx.x * E + e] = hist[e];
  if (tid == 0) blockerr[blockIdx.x] = bad;
  // the shared expert's entries of this block's range (T <= S: the blocks cover them)
  if (st.idx)
    for (int r = 0; r < RT_SLOTS / RT_THREADS; ++r) shared_entry(st, base + r * RT_THREADS + tid);
}

// One block of RT_SCAN_THREADS threads (>= E).  Besides counts and offsets it
// builds the tile table of the row-grouped products: each expert's rows are
// covered by TILE_BIG-row tiles, and a remainder of at most TILE_BIG/2 rows by
// TILE_SMALL-row tiles (a larger remainder gets one more, partly filled, big
// tile).  With big_on = 0 (small problems) every row goes to TILE_SMALL-row
// tiles.  Layout: tiles[0] = #big, tiles[1] = #small, then max_big entries
// (expert | rows << 16, first row) from tiles[4], then the small entries from
// tiles[4 + 2*max_big].
__global__ void __launch_bounds__(RT_SCAN_THREADS) route_scan(const int32_t* __restrict__ blockhist,
                                                              const int32_t* __restrict__ blockerr, int nblk,
                                                              int E, int max_big, int big_on,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ blockbase,
                                                              int32_t* __restrict__ tiles,
                                                              int32_t* __restrict__ err,
                                                              int32_t* __restrict__ host_err,
                                                              const SharedTables st) {
  __shared__ int32_t scan_c[RT_SCAN_THREADS];
  __shared__ int32_t scan_b[RT_SCAN_THREADS];
  __shared__ int32_t scan_s[RT_SCAN_THREADS];
  const int e = threadIdx.x;
  if (st.idx && e == 0) shared_header(st);
  int c = 0;
  if (e < E) {
    // the per-block counts of expert e, 16 loads in flight at a time
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = (b0 + j < nblk) ? blockhist[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < nblk) blockbase[(int64_t)(b0 + j) * E + e] = c;
        c += v[j];
      }
    }
  }
  const int rem = big_on ? c % TILE_BIG : c;
  const int nbig = big_on ? c / TILE_BIG + (rem > TILE_BIG / 2 ? 1 : 0) : 0;
  const int nsmall = (big_on && rem > TILE_BIG / 2) ? 0 : (rem + TILE_SMALL - 1) / TILE_SMALL;
  scan_c[e] = (e < E) ? c : 0;
  scan_b[e] = (e < E) ? nbig : 0;
  scan_s[e] = (e < E) ? nsmall : 0;
  __syncthreads();
  // inclusive Hillis-Steele scans over the E experts (integers: order-free)
  for (int d = 1; d < E; d <<= 1) {
    const int vc = (e >= d) ? scan_c[e - d] : 0;
    const int vb = (e >= d) ? scan_b[e - d] : 0;
    const int vs = (e >= d) ? scan_s[e - d] : 0;
    __syncthreads();
    scan_c[e] += vc;
    scan_b[e] += vb;
    scan_s[e] += vs;
    __syncthreads();
  }
  if (e < E) {
    const int off = scan_c[e] - c;
    const int b0 = scan_b[e] - nbig;
    const int s0 = scan_s[e] - nsmall;
    counts[e] = c;
    offsets[e] = off;
    for (int i = 0; i < nbig; ++i) {
      tiles[4 + 2 * (b0 + i)] = tile_word(e, min(TILE_BIG, c - i * TILE_BIG));
      tiles[4 + 2 * (b0 + i) + 1] = off + i * TILE_BIG;
    }
    int32_t* small = tiles + 4 + 2 * max_big;
    const int srow = off + nbig * TILE_BIG;
    for (int i = 0; i < nsmall; ++i) {
      small[2 * (s0 + i)] = tile_word(e, min(TILE_SMALL, c - nbig * TILE_BIG - i * TILE_SMALL));
      small[2 * (s0 + i) + 1] = srow + i * TILE_SMALL;
    }
  }
  if (e == E - 1) {  // holds the totals over all experts
    offsets[E] = scan_c[e];
    tiles[0] = scan_b[e];
    tiles[1] = scan_s[e];
    tiles[2] = TILE_BIG;
    tiles[3] = TILE_SMALL;
  }
  int bad = 0;
  for (int b = e; b < nblk; b += RT_SCAN_THREADS) bad |= blockerr[b];
  bad = __syncthreads_or(bad);
  if (e == 0) {
    *err = bad;
    // the host only reads this word after the kernel has completed: no release needed
    if (host_err) __hip_atomic_store(host_err, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ void __launch_bounds__(RT_THREADS) route_scatter(const int32_t* __restrict__ ids, int64_t S, int E,
                                                            int nbits, const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ blockbase,
                                                            int K, int32_t* __restrict__ sorted_slot,
                                                            int32_t* __restrict__ row_of_slot,
                                                            int32_t* __restrict__ tok_of_row) {
  __shared__ int32_t running[MAX_EXPERTS];
  __shared__ int32_t wcnt[RT_THREADS / 64][MAX_EXPERTS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  for (int e = tid; e < E; e += RT_THREADS) {
    running[e] = offsets[e] + blockbase[(int64_t)blockIdx.x * E + e];
#pragma unroll
    for (int q = 0; q < RT_THREADS / 64; ++q) wcnt[q][e] = 0;
  }
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RT_SLOTS;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < RT_SLOTS / RT_THREADS; ++r) {
    const int64_t s = base + r * RT_THREADS + tid;
    int e = -1;
    bool valid = false;
    if (s < S) {
      e = ids[s];
      valid = (e >= 0 && e < E);
      if (!valid) row_of_slot[s] = -1;
    }
    // lanes of this wave holding the same expert id
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    if (!valid) peers = 0;
    const int rank = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    const int tag = (r + 1) << 16;
    if (valid && rank == 0) wcnt[w][e] = tag | cnt;
    __syncthreads();
    if (valid) {
      int row = running[e] + rank;
      for (int q = 0; q < w; ++q) {
        const int v = wcnt[q][e];
        if ((v >> 16) == r + 1) row += v & 0xffff;
      }
      sorted_slot[row] = (int32_t)s;
      tok_of_row[row] = (int32_t)(s / K);
      row_of_slot[s] = row;
    }
    __syncthreads();
    if (valid && rank == 0) atomicAdd(&running[e], cnt);
    __syncthreads();
  }
}

__global__ void __launch_bounds__(RT_ONE_THREADS) route_one(const int32_t* __restrict__ ids, int64_t S, int E,
                                                            int K, int nbits, int max_big, int big_on,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_slot,
                                                            int32_t* __restrict__ row_of_slot,
                                                            int32_t* __restrict__ tok_of_row,
                                                            int32_t* __restrict__ tiles, int32_t* __restrict__ err,
                                                            int32_t* __restrict__ host_err, const SharedTables st) {
  __shared__ RouteLds<RT_ONE_THREADS> lds;
  if (st.idx) {  // the shared expert's tables first: their stores overlap the routing
    if (threadIdx.x == 0) shared_header(st);
    for (int64_t i = threadIdx.x; i < st.T; i += RT_ONE_THREADS) shared_entry(st, i);
  }
  route_block<RT_ONE_THREADS>(lds, ids, S, E, K, nbits, max_big, big_on, counts, offsets, sorted_slot, row_of_slot,
                              tok_of_row, tiles, err, host_err);
}

// The experts ranked by descending row count, ties by id (a permutation: every
// expert gets a distinct rank).  One block of RT_SCAN_THREADS >= E threads;
// thread e counts the experts that go before it.
__global__ void __launch_bounds__(RT_SCAN_THREADS) expert_order(const int32_t* __restrict__ counts, int E,
                                                                int32_t* __restrict__ order) {
  __shared__ int32_t c[RT_SCAN_THREADS];
  const int e = threadIdx.x;
  if (e < E) c[e] = counts[e];
  __syncthreads();
  if (e >= E) return;
  const int32_t ce = c[e];
  int rank = 0;
  for (int f = 0; f < E; ++f) {
    const int32_t cf = c[f];
    rank += (cf > ce || (cf == ce && f < e)) ? 1 : 0;
  }
  order[rank] = e;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_expert_order(const int32_t* counts, int E, int32_t* order, hipStream_t stream) {
  if (E <= 0 || E > RT_SCAN_THREADS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_order, dim3(1), dim3(RT_SCAN_THREADS), 0, stream, counts, E, order);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* ids, int64_t S, int E, int K, int max_big, int big_on, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slot, int32_t* row_of_slot, int32_t* tok_of_row,
                        int32_t* tiles, int32_t* err, int32_t* blockhist, int32_t* blockbase, int32_t* blockerr,
                        int32_t* host_err, const SharedTables& st, hipStream_t stream) {
  const int nblk = (int)((S + RT_SLOTS - 1) / RT_SLOTS);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (S <= RT_ONE_MAX_SLOTS && E <= RT_ONE_MAX_EXPERTS) {
    hipLaunchKernelGGL(route_one, dim3(1), dim3(RT_ONE_THREADS), 0, stream, ids, S, E, K, nbits, max_big, big_on,
                       counts, offsets, sorted_slot, row_of_slot, tok_of_row, tiles, err, host_err, st);
    return hipGetLastError();
  }
  if (nblk > 0) {
    hipLaunchKernelGGL(route_hist, dim3(nblk), dim3(RT_THREADS), 0, stream, ids, S, E, blockhist, blockerr, st);
  }
  hipLaunchKernelGGL(route_scan, dim3(1), dim3(RT_SCAN_THREADS), 0, stream, blockhist, blockerr, nblk, E, max_big,
                     big_on, counts, offsets, blockbase, tiles, err, host_err, st);
  if (nblk > 0) {
    hipLaunchKernelGGL(route_scatter, dim3(nblk), dim3(RT_THREADS), 0, stream, ids, S, E, nbits, offsets,
                       blockbase, K, sorted_slot, row_of_slot, tok_of_row);
  }
  return hipGetLastError();
}

}  // namespace hmm
