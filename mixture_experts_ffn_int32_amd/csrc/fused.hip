// The fused small-problem forward: ONE launch runs the routing, the
// up-projection + SwiGLU tiles, the down-projection tiles and the weighted
// combine, with tile-ready counters between them instead of kernel boundaries
// (RFC section 6.1: a persistent kernel whose tiles start as soon as the tiles
// they read are done; section 5.1: the first tile's latency and the gaps
// between stages dominate small problems).
//
// Work items, in dependency order:
//   0                      the routing (one workgroup, route_core.h)
//   1 .. n1                up-projection tiles (64x64, the small tile table)
//   n1+1 .. n1+n2          down-projection tiles; tile (row tile j, column tile)
//                          waits until all up-projection tiles of row tile j are done
//   then                   combine items of ct tokens; they wait for every
//                          down-projection tile
// Workgroup b takes items b, b + G, b + 2G, ... in increasing order, and every
// wait is for an item of a smaller index.  With all G workgroups resident (G is
// at most the number of CUs) the oldest unfinished item never waits, so the
// kernel always progresses.  Every wait is nevertheless bounded: after about a
// second (or the host's lower test limit) it gives up, stores 1 into the
// caller's pinned host status word, and its workgroup skips every item it has
// left (it never reads routing tables it has not seen published, so nothing
// it touches is out of bounds).  The results are then incomplete; the host
// waits for the launch, reads the word and returns an error.
//
// Counters live in the caller's workspace.  They are reset by the routing item
// of each call before it publishes its per-call epoch in the flag word; no
// item reads a counter before it has seen that epoch.  Everything one item
// writes for another (the routing arrays, a, o) is stored at the device-wide
// coherence point (agent-scope stores, sc1), so publishing needs only the
// completion of those stores before the counter update, not an L2 write-back
// (an agent-scope release fence walks the whole L2: about 15 us on MI355X),
// and every read of such data is an agent-scope (sc1) read too, so no
// consumer has to invalidate its L2 (which would throw away the cached
// weights of every other tile on that XCD).
#include "gemm_bf16.h"
#include "route_core.h"

namespace hmm {
namespace {

typedef Gmm1<Narrow, true> FG1;
typedef Gmm2<Narrow, true, true> FG2;
constexpr int FT = Narrow::NTHR;
constexpr uint32_t SPIN_CAP = 1u << 20;  // polls (an L2 round trip and s_sleep each): about a second
uint32_t g_spin_cap = SPIN_CAP;          // the host's limit for the next launches (tests lower it)

struct FusedFwdArgs {
  const int32_t* ids;
  int64_t S;
  int E, K, nbits, max_small;
  int32_t *counts, *offsets, *sorted_slot, *row_of_slot, *tok_of_row, *tiles, *err, *host_err;
  typename FG1::Args g1;
  int n1, nnt1;
  typename FG2::Args g2;
  int n2, nnt2;
  const float* tw;
  const uint16_t* o;
  uint16_t* y;
  int64_t T, H;
  int ncomb, ct;
  uint32_t* sync;  // [0] epoch flag, [1] down-projection tiles done, [4 + j] up tiles done of row tile j
  uint32_t epoch;
  uint32_t spin_cap;     // polls before a wait gives up
  uint32_t* host_status; // pinned host word: 1 once a wait has given up (the host clears it)
};

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the whole workgroup waits until *word == target; false if the wait gave up
// (then the host status word holds 1)
__device__ __forceinline__ bool block_wait(const uint32_t* word, uint32_t target, const FusedFwdArgs& A, int* flag) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    bool ok = true;
    while (load_agent(word) != target) {
      if (++spins > A.spin_cap) {
        __hip_atomic_store(A.host_status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *flag = ok;
  }
  __syncthreads();
  const bool ok = *flag != 0;
  __syncthreads();  // the flag is reused by the next wait
  return ok;
}

// every thread's coherent stores have completed (reached the coherence point)
__device__ __forceinline__ void stores_done() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// publish this workgroup's coherent stores, then add one to *word
__device__ __forceinline__ void block_signal_add(uint32_t* word) {
  stores_done();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void combine_item(const FusedFwdArgs& A, int it) {
  const int64_t cpr = A.H >> 3;
  const int64_t t0 = (int64_t)it * A.ct, t1 = min(A.T, t0 + A.ct);
  const rsrc_t o_rsrc = make_rsrc(A.o, A.S * A.H * 2);
  for (int64_t idx = threadIdx.x; idx < (t1 - t0) * cpr; idx += FT) {
    const int64_t t = t0 + idx / cpr, c = idx % cpr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < A.K; ++k) {
      const int64_t s = t * A.K + k;
      const int r = get(A.row_of_slot + s, true);
      if (r < 0) continue;
      const float wk = A.tw[s];
      float v[8];
      unpack8(bload_coh(o_rsrc, (uint32_t)(((int64_t)r * A.H + c * 8) * 2), 0), v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(wk, v[j], acc[j]);
    }
    *reinterpret_cast<u32x4*>(A.y + t * A.H + c * 8) = pack8(acc);
  }
}

__global__ void __launch_bounds__(FT, 1) fused_forward(const FusedFwdArgs A) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Narrow::STAGE];
  static_assert(sizeof(RouteLds<FT>) <= sizeof(smem), "routing LDS fits in the product buffers");
  const int tid = threadIdx.x;
  __shared__ int wait_flag;
  const int total = 1 + A.n1 + A.n2 + A.ncomb;
  bool routed = false;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    if (item == 0) {
      route_block<FT, true>(*reinterpret_cast<RouteLds<FT>*>(smem), A.ids, A.S, A.E, A.K, A.nbits, 0, 0, A.counts,
                            A.offsets, A.sorted_slot, A.row_of_slot, A.tok_of_row, A.tiles, A.err, A.host_err);
      for (int i = tid; i < A.max_small; i += FT)
        __hip_atomic_store(A.sync + 4 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) __hip_atomic_store(A.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      stores_done();
      if (tid == 0) __hip_atomic_store(A.sync, A.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      routed = true;
      continue;
    }
    if (!routed) {
      if (!block_wait(A.sync, A.epoch, A, &wait_flag)) return;  // the tables are not published
      routed = true;
    }
    int it = item - 1;
    if (it < A.n1) {
      int j, nt;
      raster(it, A.max_small, A.nnt1, j, nt);
      if (gemm_tile<FG1>(A.g1, it, smem)) block_signal_add(A.sync + 4 + j);
      __syncthreads();
      continue;
    }
    it -= A.n1;
    if (it < A.n2) {
      int j, nt;
      raster(it, A.max_small, A.nnt2, j, nt);
      if (j < get(A.tiles + 1, true)) {
        if (!block_wait(A.sync + 4 + j, (uint32_t)A.nnt1, A, &wait_flag)) return;
        if (gemm_tile<FG2>(A.g2, it, smem)) block_signal_add(A.sync + 1);
      }
      __syncthreads();
      continue;
    }
    it -= A.n2;
    if (!block_wait(A.sync + 1, (uint32_t)(get(A.tiles + 1, true) * A.nnt2), A, &wait_flag)) return;
    combine_item(A, it);
  }
}

}  // namespace

void set_fused_spin_cap(uint32_t polls) { g_spin_cap = polls ? polls : SPIN_CAP; }

int64_t fused_forward_sync_words(int64_t S, int64_t E) { return 4 + max_small_tiles(S, E, true); }

hipError_t launch_fused_forward(const int32_t* ids, int64_t T, int64_t H, int64_t I, int E, int K, const uint16_t* x,
                                const uint16_t* w1, const uint16_t* w2, const float* topk_w, uint16_t* y,
                                int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* row_of_slot,
                                int32_t* tok_of_row, int32_t* tiles, int32_t* err, int32_t* host_err, uint16_t* h,
                                uint16_t* a, uint16_t* aw, uint16_t* o, uint32_t* sync, uint32_t epoch,
                                uint32_t* host_status, int max_groups, hipStream_t stream) {
  const int64_t S = T * K;
  FusedFwdArgs A{};
  A.ids = ids;
  A.S = S;
  A.E = E;
  A.K = K;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  A.nbits = nbits;
  A.max_small = (int)max_small_tiles(S, E, true);
  A.counts = counts; A.offsets = offsets; A.sorted_slot = sorted_slot; A.row_of_slot = row_of_slot;
  A.tok_of_row = tok_of_row; A.tiles = tiles; A.err = err; A.host_err = host_err;
  const RowGroups g{tiles, offsets, sorted_slot, tok_of_row, 0, A.max_small, T, S, true, true};
  A.nnt1 = (int)((I + Narrow::BN / 2 - 1) / (Narrow::BN / 2));
  A.g1.g = g; A.g1.x = x; A.g1.w1 = w1; A.g1.tw = topk_w; A.g1.T = T; A.g1.H = H; A.g1.I = I;
  A.g1.h = h; A.g1.a = a; A.g1.aw = aw; A.g1.n_ntiles = A.nnt1; A.g1.coh = true;
  A.n1 = A.max_small * A.nnt1;
  A.nnt2 = (int)((H + Narrow::BN - 1) / Narrow::BN);
  A.g2.g = g; A.g2.a = a; A.g2.w2 = w2; A.g2.S = S; A.g2.H = H; A.g2.I = I; A.g2.o = o; A.g2.n_ntiles = A.nnt2;
  A.g2.coh = true;
  A.n2 = A.max_small * A.nnt2;
  A.tw = topk_w; A.o = o; A.y = y; A.T = T; A.H = H;
  const int64_t per = 4 * FT / (H / 8);  // about four 8-column chunks per thread
  A.ct = (int)(per < 1 ? 1 : per);
  A.ncomb = (int)((T + A.ct - 1) / A.ct);
  A.sync = sync;
  A.epoch = epoch;
  A.spin_cap = g_spin_cap;
  A.host_status = host_status;
  const int64_t total = 1 + (int64_t)A.n1 + A.n2 + A.ncomb;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  const int grid = (int)(total < max_groups ? total : max_groups);
  hipLaunchKernelGGL(fused_forward, dim3(grid), dim3(FT), 0, stream, A);
  return hipGetLastError();
}

}  // namespace hmm
