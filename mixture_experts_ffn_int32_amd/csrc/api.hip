// Host side of libhmm: validation, buffer layouts and the kernel sequences of
// the forward and backward calls declared in include/hmm.h.
#include <hip/hip_runtime.h>

#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/hmm.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

hmm_status fail(hmm_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hmm_status fail(hmm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hmm_status hip_fail(hipError_t e, const char* what) {
  return fail(HMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
inline size_t up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }

struct Dims {
  int64_t T, H, I, E, K, S;
  int64_t Is;  // shared expert's intermediate size (0: none)
  bool shared;
  bool small;  // small-problem mode (narrow tiles; see kernels.h)
  bool fp8;    // FP8 E4M3 up-projection (per-token scales, or MX block exponents)
  bool mx;     // ... with MX block exponents
  bool group;  // ... with per-group (128 along H) float scales
  bool f32;    // float32 outputs (accuracy mode)
  bool fused;  // small problem whose forward runs as one fused launch (fused.hip)
  bool fp8bwd; // the backward's act_grad and input_grad on E4M3 (HMM_FLAG_FP8_BACKWARD)
  uint32_t flags;
};

hmm_status validate(const hmm_problem* p, Dims* d) {
  if (!p) return fail(HMM_ERR_NULL_POINTER, "problem is NULL");
  if (p->shared_I != 0 && (p->shared_I < 64 || p->shared_I > 65536 || p->shared_I % 64))
    return fail(HMM_ERR_BAD_SHAPE, "shared_I must be 0 or a multiple of 64 in [64, 65536] (got %u)", p->shared_I);
  if (p->T < 0) return fail(HMM_ERR_BAD_SHAPE, "T must be >= 0 (got %lld)", (long long)p->T);
  if (p->K < 1 || p->K > 16) return fail(HMM_ERR_BAD_SHAPE, "K must be in [1, 16] (got %lld)", (long long)p->K);
  if (p->E < 1 || p->E > hmm::MAX_EXPERTS)
    return fail(HMM_ERR_BAD_SHAPE, "E must be in [1, %d] (got %lld)", hmm::MAX_EXPERTS, (long long)p->E);
  if (p->H < 64 || p->H > 65536 || p->H % 64)
    return fail(HMM_ERR_BAD_SHAPE, "H must be a multiple of 64 in [64, 65536] (got %lld)", (long long)p->H);
  if (p->I < 64 || p->I > 65536 || p->I % 64)
    return fail(HMM_ERR_BAD_SHAPE, "I must be a multiple of 64 in [64, 65536] (got %lld)", (long long)p->I);
  if (p->T > (int64_t)0x7fffffff / p->K)
    return fail(HMM_ERR_BAD_SHAPE, "T*K must stay below 2^31 (T=%lld, K=%lld)", (long long)p->T, (long long)p->K);
  if (p->flags & ~(HMM_FLAG_VALIDATE_IDS | HMM_FLAG_TILES_LARGE | HMM_FLAG_TILES_NARROW | HMM_FLAG_FUSED_FORWARD |
                   HMM_FLAG_SERIAL_BACKWARD | HMM_FLAG_FP8_BACKWARD))
    return fail(HMM_ERR_BAD_SHAPE, "unknown flag bits 0x%x", p->flags);
  if ((p->flags & HMM_FLAG_TILES_LARGE) && (p->flags & HMM_FLAG_TILES_NARROW))
    return fail(HMM_ERR_BAD_SHAPE, "HMM_FLAG_TILES_LARGE and HMM_FLAG_TILES_NARROW are exclusive");
  if (p->out_dtype != HMM_BF16 && p->out_dtype != HMM_F32)
    return fail(HMM_ERR_BAD_DTYPE, "out_dtype must be HMM_BF16 or HMM_F32 (got %d)", p->out_dtype);
  if (p->gmm1_dtype != HMM_BF16 && p->gmm1_dtype != HMM_FP8_E4M3 && p->gmm1_dtype != HMM_MXFP8_E4M3 &&
      p->gmm1_dtype != HMM_FP8_E4M3_GROUP)
    return fail(HMM_ERR_BAD_DTYPE,
                "gmm1_dtype must be HMM_BF16, HMM_FP8_E4M3, HMM_MXFP8_E4M3 or HMM_FP8_E4M3_GROUP (got %d)",
                p->gmm1_dtype);
  {
    // every array a product reads through a buffer resource must stay below 4 GiB
    // (the float32-output mode reads [hi | lo] operands of twice the width)
    const int64_t S = p->T * p->K, lim = (int64_t)0xFFFFFF00, w = (p->out_dtype == HMM_F32) ? 2 : 1;
    const int64_t Is = p->shared_I;
    const int64_t ext[] = {p->T * p->H * 2 * w, S * 2 * p->I * 2 * w, S * p->H * 2 * w, p->H * 2 * p->I * 2,
                           p->T * 2 * Is * 2 * w, p->H * 2 * Is * 2};
    for (int64_t x : ext)
      if (x > lim) return fail(HMM_ERR_UNSUPPORTED, "an operand array exceeds 4 GiB (%lld bytes)", (long long)x);
  }
  if (p->out_dtype == HMM_F32 && p->gmm1_dtype != HMM_BF16)
    return fail(HMM_ERR_UNSUPPORTED, "out_dtype HMM_F32 is implemented with gmm1_dtype HMM_BF16 only");
  if (p->gmm1_dtype != HMM_BF16 && p->H % 128)
    return fail(HMM_ERR_BAD_SHAPE, "an FP8 gmm1_dtype needs H to be a multiple of 128 (got %lld)", (long long)p->H);
  if ((p->flags & HMM_FLAG_FP8_BACKWARD) && p->out_dtype == HMM_F32)
    return fail(HMM_ERR_UNSUPPORTED, "HMM_FLAG_FP8_BACKWARD is implemented with bf16 outputs only");
  if ((p->flags & HMM_FLAG_FP8_BACKWARD) && p->H % 128)
    return fail(HMM_ERR_BAD_SHAPE, "HMM_FLAG_FP8_BACKWARD needs H to be a multiple of 128 (got %lld)", (long long)p->H);
  d->T = p->T;
  d->H = p->H;
  d->I = p->I;
  d->E = p->E;
  d->K = p->K;
  d->S = p->T * p->K;
  d->Is = p->shared_I;
  d->shared = p->shared_I != 0;
  d->fp8 = p->gmm1_dtype == HMM_FP8_E4M3 || p->gmm1_dtype == HMM_MXFP8_E4M3 || p->gmm1_dtype == HMM_FP8_E4M3_GROUP;
  d->mx = p->gmm1_dtype == HMM_MXFP8_E4M3;
  d->group = p->gmm1_dtype == HMM_FP8_E4M3_GROUP;
  d->f32 = p->out_dtype == HMM_F32;
  d->small = (p->flags & HMM_FLAG_TILES_NARROW) ? true
             : (p->flags & HMM_FLAG_TILES_LARGE) ? false
             : hmm::small_mode(d->S, d->H, d->I);
  d->fused = d->small && !d->fp8 && !d->f32 && !d->shared && d->S > 0 && d->S <= hmm::RT_ONE_MAX_SLOTS &&
             d->E <= hmm::RT_ONE_MAX_EXPERTS && (p->flags & HMM_FLAG_FUSED_FORWARD);
  d->fp8bwd = (p->flags & HMM_FLAG_FP8_BACKWARD) != 0;
  d->flags = p->flags;
  return HMM_OK;
}

bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15u) != 0; }

// A pointer to an array that may legitimately be empty may be NULL.
hmm_status need(const void* ptr, bool nonempty, const char* name) {
  if (!ptr && nonempty) return fail(HMM_ERR_NULL_POINTER, "%s is NULL", name);
  if (ptr && misaligned(ptr)) return fail(HMM_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return HMM_OK;
}

int64_t n_route_blocks(const Dims& d) { return (d.S + hmm::RT_SLOTS - 1) / hmm::RT_SLOTS; }
int64_t tile_ints(const Dims& d) { return hmm::tile_table_ints(d.S, d.E, d.small); }
hmm::RowGroups row_groups(const Dims& d, const int32_t* tiles, const int32_t* offsets, const int32_t* sorted_slot,
                          const int32_t* tok_of_row) {
  return hmm::RowGroups{tiles, offsets, sorted_slot, tok_of_row, hmm::max_big_tiles(d.S, d.E, d.small),
                        hmm::max_small_tiles(d.S, d.E, d.small), d.T, d.S, d.small};
}
// The shared expert as a grouped problem of its own: one expert, all T tokens
// in token order (idx is both its sorted_slot and its tok_of_row), the same
// tiling mode as the routed experts.
int64_t shared_tile_ints(const Dims& d) { return hmm::tile_table_ints(d.T, 1, d.small); }
hmm::RowGroups shared_groups(const Dims& d, const int32_t* tiles, const int32_t* offsets, const int32_t* idx) {
  return hmm::RowGroups{tiles, offsets, idx, idx, hmm::max_big_tiles(d.T, 1, d.small),
                        hmm::max_small_tiles(d.T, 1, d.small), d.T, d.T, d.small};
}

hmm_saved_layout saved_layout(const Dims& d) {
  hmm_saved_layout L{};
  size_t o = 0;
  L.counts = o;        o += up(d.E * 4);
  L.offsets = o;       o += up((d.E + 1) * 4);
  L.sorted_slot = o;   o += up(d.S * 4);
  L.row_of_slot = o;   o += up(d.S * 4);
  L.tok_of_row = o;    o += up(d.S * 4);
  L.tiles = o;         o += up(tile_ints(d) * 4);
  // float32-output mode: h float32, a and aw as bf16 [hi | lo] pairs (twice as wide)
  const int64_t hb = d.f32 ? 4 : 2, ab = d.f32 ? 4 : 2;
  L.h = o;             o += up(d.S * 2 * d.I * hb);
  L.a = o;             o += up(d.S * d.I * ab);
  L.aw = o;            o += up(d.S * d.I * ab);
  L.id_error = o;      o += up(4);
  // shared expert (all zero-sized without one)
  const int64_t Ts = d.shared ? d.T : 0;
  L.shared_offsets = o; o += d.shared ? up(2 * 4) : 0;
  L.shared_idx = o;     o += up(Ts * 4);
  L.shared_ones = o;    o += up(Ts * 4);
  L.shared_tiles = o;   o += d.shared ? up(shared_tile_ints(d) * 4) : 0;
  L.shared_h = o;       o += up(Ts * 2 * d.Is * hb);
  L.shared_a = o;       o += up(Ts * d.Is * ab);
  L.total = o;
  return L;
}

// routing scratch: per-block histograms and bases, per-block error bits
struct RouteScratch {
  size_t blockhist, blockbase, blockerr, total;
};
RouteScratch route_scratch(const Dims& d, size_t base) {
  RouteScratch r{};
  const int64_t nb = n_route_blocks(d);
  size_t o = base;
  r.blockhist = o; o += up(nb * d.E * 4);
  r.blockbase = o; o += up(nb * d.E * 4);
  r.blockerr = o;  o += up(nb * 4 + 4);
  r.total = o;
  return r;
}

// Forward scratch: routing scratch, the expert outputs o [S,H] and, for the FP8
// up-projection, the quantised operands with their descales and the column
// maxima of the weight quantisation.
struct FwdWork {
  RouteScratch rs;
  size_t o, os, xq, dsx, wq, dsw, pmax, xs, ws, sync, ntiles, total;
};
FwdWork fwd_work(const Dims& d) {
  FwdWork w{};
  w.rs = route_scratch(d, 0);
  size_t o = w.rs.total;
  w.o = o; o += up(d.S * d.H * (d.f32 ? 4 : 2));
  if (d.shared) {
    w.os = o; o += up(d.T * d.H * (d.f32 ? 4 : 2));  // the shared expert's output rows
  }
  if (d.fp8) {
    w.xq = o;   o += up(d.T * d.H);
    w.wq = o;   o += up(d.E * d.H * 2 * d.I);
  }
  if (d.mx) {  // E8M0 block exponents: [T][H/32] and [E][2I][H/32]
    w.xs = o;   o += up(d.T * (d.H / 32));
    w.ws = o;   o += up(d.E * 2 * d.I * (d.H / 32));
  } else if (d.group) {  // float32 descales: [T][H/128] and [E][H/128][2I]
    w.dsx = o;  o += up(d.T * (d.H / 128) * 4);
    w.dsw = o;  o += up(d.E * (d.H / 128) * 2 * d.I * 4);
    if (!d.small) {  // the per-group product's own 64-row tile table
      w.ntiles = o; o += up(hmm::tile_table_ints(d.S, d.E, true) * 4);
    }
  } else if (d.fp8) {
    w.dsx = o;  o += up(d.T * 4);
    w.dsw = o;  o += up(d.E * 2 * d.I * 4);
    w.pmax = o; o += up(hmm::quant_cols_chunks(d.H) * d.E * 2 * d.I * 4);
  }
  if (d.fused) {
    w.sync = o; o += up(hmm::fused_forward_sync_words(d.S, d.E) * 4);  // tile-ready counters
  }
  w.total = o;
  return w;
}

// Backward scratch: dH, dXp, the d_topk_weights partials and, in the float32-output
// mode, dY as a bf16 [hi | lo] pair (dH is then a pair too and dXp float32).
struct BwdWork {
  size_t dy2, dh, dxp, dwpart, dhs, dxs, total;
  // FP8 backward: E4M3 codes and float32 descales of dY [T][H], W2 rows [E*I][H],
  // dH [S][2I] and W1 rows [E*H][2I]
  size_t dyq, dsy, w2q, dsw2, dhq, dsh, w1q, dsw1;
  size_t order;  // [E] int32: the experts by descending row count (weight gradients, large tiling)
  int dw_cols;
};
BwdWork bwd_work(const Dims& d) {
  BwdWork w{};
  w.dw_cols = d.f32 ? hmm::act_grad_f32_dw_cols(d.I, d.small) : hmm::act_grad_dw_cols(d.I, d.small);
  const int64_t wide = d.f32 ? 2 : 1;
  size_t o = 0;
  if (d.f32) {
    w.dy2 = o;  o += up(d.T * 2 * d.H * 2);
  }
  w.dh = o;     o += up(d.S * 2 * d.I * 2 * wide);
  w.dxp = o;    o += up(d.S * d.H * (d.f32 ? 4 : 2));
  w.dwpart = o; o += up(d.S * w.dw_cols * 4);
  if (d.S > 0 && !d.f32 && !d.small) {
    w.order = o; o += up(d.E * 4);
  }
  if (d.shared) {  // the shared expert's dH and dX rows
    w.dhs = o;  o += up(d.T * 2 * d.Is * 2 * wide);
    w.dxs = o;  o += up(d.T * d.H * (d.f32 ? 4 : 2));
  }
  if (d.fp8bwd) {
    w.dyq = o;  o += up(d.T * d.H);
    w.dsy = o;  o += up(d.T * 4);
    w.w2q = o;  o += up(d.E * d.I * d.H);
    w.dsw2 = o; o += up(d.E * d.I * 4);
    w.dhq = o;  o += up(d.S * 2 * d.I);
    w.dsh = o;  o += up(d.S * 4);
    w.w1q = o;  o += up(d.E * d.H * 2 * d.I);
    w.dsw1 = o; o += up(d.E * d.H * 4);
  }
  w.total = o;
  return w;
}

template <class T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }
template <class T>
const T* at(const void* base, size_t off) { return reinterpret_cast<const T*>(static_cast<const char*>(base) + off); }

// ------------------------------------------------------------- stage timing
struct Prof {
  bool on = false;
  int dropped = 0;
  std::vector<hipEvent_t> pool;           // events created so far (reused after a read)
  size_t used = 0;                        // events handed out since the last read
  std::vector<std::pair<std::string, std::pair<size_t, size_t>>> marks;  // name, (start, end) indices
};
constexpr size_t PROF_MAX_EVENTS = 16384;
thread_local Prof g_prof;

hipEvent_t prof_event() {
  Prof& P = g_prof;
  if (P.used == P.pool.size()) {
    if (P.pool.size() >= PROF_MAX_EVENTS) return nullptr;
    // timing-only events: no system-scope fence (cache writeback and invalidate)
    // when recorded, which would add its own cost to every bracketed launch
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    P.pool.push_back(ev);
  }
  return P.pool[P.used++];
}

// Brackets one launch with events when timing is on.
struct Stage {
  const char* name;
  hipStream_t st;
  size_t i0 = 0;
  bool live = false;
  Stage(const char* n, hipStream_t s) : name(n), st(s) {
    if (!g_prof.on) return;
    hipEvent_t e = prof_event();
    if (!e) { ++g_prof.dropped; return; }
    i0 = g_prof.used - 1;
    live = hipEventRecord(e, st) == hipSuccess;
  }
  ~Stage() {
    if (!live) return;
    hipEvent_t e = prof_event();
    if (!e) { ++g_prof.dropped; return; }
    if (hipEventRecord(e, st) == hipSuccess) g_prof.marks.push_back({name, {i0, g_prof.used - 1}});
  }
};

// Per-thread, per-device objects of the id check: a pinned (coherent,
// device-visible) host word that the routing kernel writes, and an event recorded
// after the routing.  Created on first use with that device current.
constexpr int MAX_DEVICES = 64;
constexpr int32_t ID_PENDING = -1;  // the id-check word before the routing has written it
struct DevState {
  bool ready = false;
  int32_t* word = nullptr;
  hipEvent_t id_ev = nullptr;
  uint32_t* fused_status = nullptr;  // pinned: the fused forward stores 1 when a wait gave up
  hipEvent_t fused_ev = nullptr;     // recorded after a fused forward launch
  int cus = 0;  // compute units (the fused kernel's workgroup count: all resident)
  // the backward's second stream (default priority, non-blocking) and its fork,
  // dH-ready and join events; created on the first large backward
  bool side_ready = false;
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, dh_ev = nullptr, join_ev = nullptr;
};
DevState* dev_state() {
  thread_local DevState st[MAX_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  DevState& c = st[dev];
  if (c.ready) return &c;
  bool ok = hipHostMalloc((void**)&c.word, sizeof(int32_t), hipHostMallocCoherent) == hipSuccess;
  ok = ok && hipHostMalloc((void**)&c.fused_status, sizeof(uint32_t), hipHostMallocCoherent) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c.id_ev, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c.fused_ev, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipDeviceGetAttribute(&c.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c.cus > 0;
  if (!ok) {  // release whatever was made; the next call tries again
    if (c.word) (void)hipHostFree(c.word);
    if (c.fused_status) (void)hipHostFree(c.fused_status);
    if (c.id_ev) (void)hipEventDestroy(c.id_ev);
    if (c.fused_ev) (void)hipEventDestroy(c.fused_ev);
    c = DevState{};
    return nullptr;
  }
  c.ready = true;
  return &c;
}

// The backward's side stream and events of the current device (created once);
// nullptr if they cannot be made (the backward then runs on one stream).
DevState* side_state() {
  DevState* c = dev_state();
  if (!c) return nullptr;
  if (c->side_ready) return c;
  bool ok = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c->dh_ev, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    if (c->side) (void)hipStreamDestroy(c->side);
    for (hipEvent_t* e : {&c->fork_ev, &c->dh_ev, &c->join_ev})
      if (*e) (void)hipEventDestroy(*e);
    c->side = nullptr;
    c->fork_ev = c->dh_ev = c->join_ev = nullptr;
    return nullptr;
  }
  c->side_ready = true;
  return c;
}

// Enqueue the routing; with validate_ids the routing also stores its error flag
// into the pinned host word, and an event is recorded after it.  The caller
// waits with finish_id_check (after enqueueing its products, so the GPU never
// idles while the host waits).
hmm_status run_route(const Dims& d, const int32_t* ids, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                     int32_t* row_of_slot, int32_t* tok_of_row, int32_t* tiles, int32_t* err, void* scratch,
                     const RouteScratch& rs, bool validate_ids, const hmm::SharedTables& shared,
                     hipStream_t stream) {
  DevState* c = nullptr;
  if (validate_ids) {
    c = dev_state();
    if (!c) return fail(HMM_ERR_HIP, "could not create the per-device id-check word or event");
    *c->word = ID_PENDING;
  }
  hipError_t e;
  {
    Stage stage("route", stream);
    e = hmm::launch_route(ids, d.S, (int)d.E, (int)d.K, (int)hmm::max_big_tiles(d.S, d.E, d.small), d.small ? 0 : 1,
                          counts, offsets, sorted_slot, row_of_slot, tok_of_row, tiles, err,
                          at<int32_t>(scratch, rs.blockhist), at<int32_t>(scratch, rs.blockbase),
                          at<int32_t>(scratch, rs.blockerr), c ? c->word : nullptr, shared, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "routing launch");
  if (c) {
    e = hipEventRecord(c->id_ev, stream);
    if (e != hipSuccess) return hip_fail(e, "id-validation event");
  }
  return HMM_OK;
}

// The routing and the up-projection in one launch (small bf16 problems without
// a shared expert; launch_route_gmm1_swiglu), with run_route's id check.
hmm_status run_route_gmm1(hmm::RoutedGmm1Job j, bool validate_ids, hipStream_t stream) {
  DevState* c = nullptr;
  if (validate_ids) {
    c = dev_state();
    if (!c) return fail(HMM_ERR_HIP, "could not create the per-device id-check word or event");
    *c->word = ID_PENDING;
  }
  j.host_err = c ? c->word : nullptr;
  hipError_t e;
  {
    Stage stage("route+gmm1_swiglu", stream);
    e = hmm::launch_route_gmm1_swiglu(j, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "routing + gmm1 launch");
  if (c) {
    e = hipEventRecord(c->id_ev, stream);
    if (e != hipSuccess) return hip_fail(e, "id-validation event");
  }
  return HMM_OK;
}

// The routing stores 0 or 1 into the host word as soon as the ids are checked
// (the word holds ID_PENDING until then); the host polls it, and falls back on
// the event recorded after the launch that contains the routing.
hmm_status finish_id_check(const Dims& d) {
  DevState* c = dev_state();
  if (!c) return fail(HMM_ERR_HIP, "id-check state missing");
  volatile int32_t* w = c->word;
  int32_t v = *w;
  for (uint32_t spin = 0; v == ID_PENDING; ++spin) {
    if ((spin & 1023) == 1023) {
      const hipError_t q = hipEventQuery(c->id_ev);
      if (q == hipSuccess) {
        v = *w;
        if (v == ID_PENDING) return fail(HMM_ERR_HIP, "the routing did not report its id check");
        break;
      }
      if (q != hipErrorNotReady) return hip_fail(q, "id-validation wait");
    }
    v = *w;
  }
  if (v) return fail(HMM_ERR_EXPERT_ID_OUT_OF_RANGE, "topk_ids holds a value outside [0, E=%lld)", (long long)d.E);
  return HMM_OK;
}

// A per-call value for the fused kernel's flag word: distinct for 2^32 calls of
// this process and unlikely to be left in a workspace by anything else.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  static const uint32_t salt =
      (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() ^ ((uint32_t)getpid() * 2654435761u);
  const uint32_t e = salt + counter.fetch_add(1) * 2654435761u;
  return e ? e : 1u;
}

}  // namespace

extern "C" {

const char* hmm_status_string(hmm_status s) {
  switch (s) {
    case HMM_OK: return "HMM_OK";
    case HMM_ERR_NULL_POINTER: return "HMM_ERR_NULL_POINTER";
    case HMM_ERR_BAD_SHAPE: return "HMM_ERR_BAD_SHAPE";
    case HMM_ERR_BAD_DTYPE: return "HMM_ERR_BAD_DTYPE";
    case HMM_ERR_MISALIGNED: return "HMM_ERR_MISALIGNED";
    case HMM_ERR_UNSUPPORTED: return "HMM_ERR_UNSUPPORTED";
    case HMM_ERR_WORKSPACE_TOO_SMALL: return "HMM_ERR_WORKSPACE_TOO_SMALL";
    case HMM_ERR_EXPERT_ID_OUT_OF_RANGE: return "HMM_ERR_EXPERT_ID_OUT_OF_RANGE";
    case HMM_ERR_HIP: return "HMM_ERR_HIP";
    case HMM_ERR_TIMEOUT: return "HMM_ERR_TIMEOUT";
  }
  return "HMM_ERR_UNKNOWN";
}

const char* hmm_last_error_message(void) { return g_last_error.c_str(); }

hmm_status hmm_set_fused_spin_limit(uint32_t polls) {
  hmm::set_fused_spin_cap(polls);
  return HMM_OK;
}

const char* hmm_build_info(void) {
  return "libhmm gfx950 (CDNA4) bf16 MFMA 32x32x16 and fp8 e4m3 MFMA 32x32x64; 256x256, 64x256 and 64x64 tiles, "
         "grouped rasterisation";
}

hmm_status hmm_forward_sizes(const hmm_problem* p, size_t* workspace_bytes, size_t* saved_bytes) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (!workspace_bytes || !saved_bytes) return fail(HMM_ERR_NULL_POINTER, "size outputs are NULL");
  *workspace_bytes = fwd_work(d).total;
  *saved_bytes = saved_layout(d).total;
  return HMM_OK;
}

hmm_status hmm_saved_layout_of(const hmm_problem* p, hmm_saved_layout* out) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (!out) return fail(HMM_ERR_NULL_POINTER, "layout output is NULL");
  *out = saved_layout(d);
  return HMM_OK;
}

hmm_status hmm_backward_sizes(const hmm_problem* p, size_t* workspace_bytes) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (!workspace_bytes) return fail(HMM_ERR_NULL_POINTER, "size output is NULL");
  *workspace_bytes = bwd_work(d).total;
  return HMM_OK;
}

hmm_status hmm_route_workspace_size(const hmm_problem* p, size_t* workspace_bytes) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (!workspace_bytes) return fail(HMM_ERR_NULL_POINTER, "size output is NULL");
  RouteScratch rs = route_scratch(d, 0);
  size_t o = rs.total;
  o += up(tile_ints(d) * 4);  // tile table
  o += up(4);                 // error word
  o += up(d.S * 4);           // token of each permuted row
  *workspace_bytes = o;
  return HMM_OK;
}

hmm_status hmm_route(const hmm_problem* p, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                     int32_t* sorted_slot, int32_t* row_of_slot, void* workspace, size_t workspace_bytes,
                     void* stream) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  const bool ne = d.S > 0;
  if ((s = need(topk_ids, ne, "topk_ids")) || (s = need(counts, true, "counts")) ||
      (s = need(offsets, true, "offsets")) || (s = need(sorted_slot, ne, "sorted_slot")) ||
      (s = need(row_of_slot, ne, "row_of_slot")) || (s = need(workspace, true, "workspace")))
    return s;
  size_t need_ws = 0;
  hmm_route_workspace_size(p, &need_ws);
  if (workspace_bytes < need_ws)
    return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need_ws);
  RouteScratch rs = route_scratch(d, 0);
  int32_t* tiles = at<int32_t>(workspace, rs.total);
  int32_t* err = at<int32_t>(workspace, rs.total + up(tile_ints(d) * 4));
  int32_t* tok = at<int32_t>(workspace, rs.total + up(tile_ints(d) * 4) + up(4));
  const bool v = (p->flags & HMM_FLAG_VALIDATE_IDS) != 0;
  s = run_route(d, topk_ids, counts, offsets, sorted_slot, row_of_slot, tok, tiles, err, workspace, rs, v, {},
                (hipStream_t)stream);
  if (s != HMM_OK || !v) return s;
  return finish_id_check(d);
}

namespace {
hmm_status quant_dims(int64_t E, int64_t H, int64_t N) {
  if (E < 1 || H < 8 || N < 8 || H % 8 || N % 8)
    return fail(HMM_ERR_BAD_SHAPE, "quantisation needs E >= 1 and H, N positive multiples of 8 (E=%lld H=%lld N=%lld)",
                (long long)E, (long long)H, (long long)N);
  if (E * H * N > (int64_t)0xFFFFFF00 || E > (int64_t)0x7fffffff)
    return fail(HMM_ERR_UNSUPPORTED, "quantised array exceeds 4 GiB");
  if (N > ((int64_t)1 << 24)) return fail(HMM_ERR_UNSUPPORTED, "N exceeds 2^24 columns (got %lld)", (long long)N);
  return HMM_OK;
}
}  // namespace

hmm_status hmm_quant_rows_fp8(const void* x, int64_t T, int64_t H, uint8_t* xq, float* descale, void* stream) {
  if (T < 0 || T > (int64_t)0x7fffffff) return fail(HMM_ERR_BAD_SHAPE, "T must be in [0, 2^31) (got %lld)", (long long)T);
  hmm_status s = quant_dims(T > 0 ? T : 1, H, 8);
  if (s != HMM_OK) return s;
  const bool ne = T > 0;
  if ((s = need(x, ne, "x")) || (s = need(xq, ne, "xq")) || (s = need(descale, ne, "descale"))) return s;
  Stage stage("quant_x", (hipStream_t)stream);
  const hipError_t e = hmm::launch_quant_rows_fp8((const uint16_t*)x, T, H, xq, descale, (hipStream_t)stream);
  return e == hipSuccess ? HMM_OK : hip_fail(e, "token quantisation launch");
}

hmm_status hmm_quant_cols_workspace_size(int64_t E, int64_t H, int64_t N, size_t* workspace_bytes) {
  hmm_status s = quant_dims(E, H, N);
  if (s != HMM_OK) return s;
  if (!workspace_bytes) return fail(HMM_ERR_NULL_POINTER, "size output is NULL");
  *workspace_bytes = up(hmm::quant_cols_chunks(H) * E * N * 4);
  return HMM_OK;
}

hmm_status hmm_quant_cols_fp8(const void* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, float* descale,
                              void* workspace, size_t workspace_bytes, void* stream) {
  size_t need_ws = 0;
  hmm_status s = hmm_quant_cols_workspace_size(E, H, N, &need_ws);
  if (s != HMM_OK) return s;
  if ((s = need(w, true, "w")) || (s = need(wq, true, "wq")) || (s = need(descale, true, "descale")) ||
      (s = need(workspace, true, "workspace")))
    return s;
  if (workspace_bytes < need_ws)
    return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need_ws);
  Stage stage("quant_w1", (hipStream_t)stream);
  const hipError_t e =
      hmm::launch_quant_cols_fp8((const uint16_t*)w, E, H, N, (float*)workspace, wq, descale, (hipStream_t)stream);
  return e == hipSuccess ? HMM_OK : hip_fail(e, "weight quantisation launch");
}

}  // extern "C"

namespace {

// The forward of hmm_forward and hmm_forward_shared (up_s / down_s: the shared
// expert's weights, used when d.shared).
hmm_status forward_impl(const hmm_problem* p, const Dims& d, const void* x, const int32_t* topk_ids,
                        const float* topk_weights, const void* up_w, const void* down_w, const void* up_s,
                        const void* down_s, void* y, void* saved, size_t saved_bytes, void* workspace,
                        size_t workspace_bytes, void* stream) {
  hmm_status s;
  const bool ne = d.S > 0;
  if ((s = need(x, ne, "x")) || (s = need(topk_ids, ne, "topk_ids")) || (s = need(topk_weights, ne, "topk_weights")) ||
      (s = need(up_w, true, "up_proj_weight")) || (s = need(down_w, true, "down_proj_weight")) ||
      (s = need(up_s, d.shared, "shared_up_proj_weight")) ||
      (s = need(down_s, d.shared, "shared_down_proj_weight")) || (s = need(y, ne, "y")) ||
      (s = need(saved, true, "saved")) || (s = need(workspace, true, "workspace")))
    return s;
  const hmm_saved_layout L = saved_layout(d);
  const FwdWork W = fwd_work(d);
  if (saved_bytes < L.total) return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "saved %zu < %zu bytes", saved_bytes, L.total);
  if (workspace_bytes < W.total)
    return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, W.total);
  hipStream_t st = (hipStream_t)stream;

  int32_t* offsets = at<int32_t>(saved, L.offsets);
  int32_t* sorted_slot = at<int32_t>(saved, L.sorted_slot);
  int32_t* tiles = at<int32_t>(saved, L.tiles);
  int32_t* tok_of_row = at<int32_t>(saved, L.tok_of_row);
  const bool validate_ids = (p->flags & HMM_FLAG_VALIDATE_IDS) != 0;
  if (d.fused) {
    // small problem: routing, both products and the combine in one launch
    DevState* c = dev_state();
    if (!c) return fail(HMM_ERR_HIP, "could not create the per-device id-check word or event");
    if (validate_ids) *c->word = ID_PENDING;
    *c->fused_status = 0;
    hipError_t e;
    {
      Stage stage("fused_forward", st);
      e = hmm::launch_fused_forward(topk_ids, d.T, d.H, d.I, (int)d.E, (int)d.K, (const uint16_t*)x,
                                    (const uint16_t*)up_w, (const uint16_t*)down_w, topk_weights, (uint16_t*)y,
                                    at<int32_t>(saved, L.counts), offsets, sorted_slot,
                                    at<int32_t>(saved, L.row_of_slot), tok_of_row, tiles,
                                    at<int32_t>(saved, L.id_error), validate_ids ? c->word : nullptr,
                                    at<uint16_t>(saved, L.h), at<uint16_t>(saved, L.a), at<uint16_t>(saved, L.aw),
                                    at<uint16_t>(workspace, W.o), at<uint32_t>(workspace, W.sync), next_epoch(),
                                    c->fused_status, c->cus, st);
    }
    if (e != hipSuccess) return hip_fail(e, "fused forward launch");
    e = hipEventRecord(c->fused_ev, st);
    if (e != hipSuccess) return hip_fail(e, "fused forward event");
    if (validate_ids) {
      e = hipEventRecord(c->id_ev, st);
      if (e != hipSuccess) return hip_fail(e, "id-validation event");
      s = finish_id_check(d);
    }
    // the launch's waits are bounded; one that gave up has stored the flag
    e = hipEventSynchronize(c->fused_ev);
    if (e != hipSuccess) return hip_fail(e, "fused forward wait");
    if (*(volatile uint32_t*)c->fused_status)
      return fail(HMM_ERR_TIMEOUT, "fused forward: a tile-ready wait gave up (not all of its %d workgroups were "
                  "resident at once?); y and the saved intermediates are incomplete", c->cus);
    return validate_ids ? s : HMM_OK;
  }
  // the routing launch also writes the shared expert's tables (also for T = 0:
  // the backward's weight gradients read them)
  hmm::SharedTables sh{};
  if (d.shared)
    sh = hmm::SharedTables{d.T, (int)hmm::max_big_tiles(d.T, 1, d.small), d.small ? 0 : 1,
                           at<int32_t>(saved, L.shared_offsets), at<int32_t>(saved, L.shared_idx),
                           at<float>(saved, L.shared_ones), at<int32_t>(saved, L.shared_tiles)};
  // small bf16 problems route inside the up-projection's launch (below)
  const bool route_in_gmm1 = d.small && !d.fp8 && !d.f32 && !d.shared && d.S > 0 &&
                             d.S <= hmm::ROUTED_MAX_SLOTS && d.E <= hmm::RT_ONE_MAX_EXPERTS &&
                             hmm::max_small_tiles(d.S, d.E, true) * ((d.I + 31) / 32) <= hmm::ROUTED_MAX_TILES;
  if (!route_in_gmm1) {
    s = run_route(d, topk_ids, at<int32_t>(saved, L.counts), offsets, sorted_slot, at<int32_t>(saved, L.row_of_slot),
                  tok_of_row, tiles, at<int32_t>(saved, L.id_error), workspace, W.rs, validate_ids, sh, st);
    if (s != HMM_OK) return s;
  }
  hipError_t e;
  const hmm::RowGroups gs =
      d.shared ? shared_groups(d, sh.tiles, sh.offsets, sh.idx) : hmm::RowGroups{};
  if (!ne) return validate_ids ? finish_id_check(d) : HMM_OK;

  hmm::RowGroups g = row_groups(d, tiles, offsets, sorted_slot, tok_of_row);
  const float* ones = at<float>(saved, L.shared_ones);
  if (d.f32) {
    float* h32 = at<float>(saved, L.h);
    float* o32 = at<float>(workspace, W.o);
    uint16_t* a2 = at<uint16_t>(saved, L.a);
    {
      Stage stage("gmm1_swiglu", st);
      e = hmm::launch_gmm1_f32(g, (const uint16_t*)x, (const uint16_t*)up_w, topk_weights, d.H, d.I, h32, a2,
                               at<uint16_t>(saved, L.aw), st);
    }
    if (e != hipSuccess) return hip_fail(e, "gmm1 launch");
    if (d.shared) {
      Stage stage("shared_gmm1", st);
      e = hmm::launch_gmm1_f32(gs, (const uint16_t*)x, (const uint16_t*)up_s, ones, d.H, d.Is,
                               at<float>(saved, L.shared_h), at<uint16_t>(saved, L.shared_a), nullptr, st);
    }
    if (e != hipSuccess) return hip_fail(e, "shared gmm1 launch");
    {
      Stage stage("gmm2", st);
      e = hmm::launch_gmm2_f32(g, a2, (const uint16_t*)down_w, d.H, d.I, o32, st);
    }
    if (e != hipSuccess) return hip_fail(e, "gmm2 launch");
    if (d.shared) {
      Stage stage("shared_gmm2", st);
      e = hmm::launch_gmm2_f32(gs, at<uint16_t>(saved, L.shared_a), (const uint16_t*)down_s, d.H, d.Is,
                               at<float>(workspace, W.os), st);
    }
    if (e != hipSuccess) return hip_fail(e, "shared gmm2 launch");
    {
      Stage stage("combine", st);
      e = hmm::launch_combine_f32(o32, at<int32_t>(saved, L.row_of_slot), topk_weights, d.T, (int)d.K, d.H,
                                  d.shared ? at<float>(workspace, W.os) : nullptr, (float*)y, st);
    }
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return validate_ids ? finish_id_check(d) : HMM_OK;
  }
  uint16_t* h = at<uint16_t>(saved, L.h);
  uint16_t* a = at<uint16_t>(saved, L.a);
  uint16_t* aw = at<uint16_t>(saved, L.aw);
  uint16_t* o = at<uint16_t>(workspace, W.o);
  uint16_t* hs = at<uint16_t>(saved, L.shared_h);
  uint16_t* as = at<uint16_t>(saved, L.shared_a);
  uint16_t* os = d.shared ? at<uint16_t>(workspace, W.os) : nullptr;
  const int nj = d.shared ? 2 : 1;  // jobs per product launch: routed experts, then the shared expert
  if (d.mx) {
    uint8_t* xq = at<uint8_t>(workspace, W.xq);
    uint8_t* wq = at<uint8_t>(workspace, W.wq);
    uint8_t* xs = at<uint8_t>(workspace, W.xs);
    uint8_t* ws = at<uint8_t>(workspace, W.ws);
    {
      Stage stage("quant_x_mx", st);
      e = hmm::launch_quant_rows_mx((const uint16_t*)x, d.T, d.H, xq, xs, st);
    }
    if (e != hipSuccess) return hip_fail(e, "token quantisation launch");
    {
      Stage stage("quant_w1_mx", st);
      e = hmm::launch_quant_cols_mx((const uint16_t*)up_w, d.E, d.H, 2 * d.I, wq, ws, st);
    }
    if (e != hipSuccess) return hip_fail(e, "weight quantisation launch");
    {
      Stage stage("gmm1_mx_swiglu", st);
      e = hmm::launch_gmm1_mx(g, xq, xs, wq, ws, topk_weights, d.H, d.I, h, a, aw, st);
    }
    if (e != hipSuccess) return hip_fail(e, "gmm1 launch");
  } else if (d.group) {
    uint8_t* xq = at<uint8_t>(workspace, W.xq);
    uint8_t* wq = at<uint8_t>(workspace, W.wq);
    float* dsx = at<float>(workspace, W.dsx);
    float* dsw = at<float>(workspace, W.dsw);
    {
      Stage stage("quant_x_group", st);
      e = hmm::launch_quant_rows_group((const uint16_t*)x, d.T, d.H, xq, dsx, st);
    }
    if (e != hipSuccess) return hip_fail(e, "token quantisation launch");
    {
      Stage stage("quant_w1_group", st);
      e = hmm::launch_quant_cols_group((const uint16_t*)up_w, d.E, d.H, 2 * d.I, wq, dsw, st);
    }
    if (e != hipSuccess) return hip_fail(e, "weight quantisation launch");
    // The per-group product runs on 64-row tiles only (two accumulator sets).  With
    // 256-row tiles for the other products a second routing pass, in the narrow
    // mode, writes its tile table (every other array it writes is unchanged).
    hmm::RowGroups gn = g;
    if (!d.small) {
      int32_t* nt = at<int32_t>(workspace, W.ntiles);
      {
        Stage stage("route_narrow", st);
        e = hmm::launch_route(topk_ids, d.S, (int)d.E, (int)d.K, (int)hmm::max_big_tiles(d.S, d.E, true), 0,
                              at<int32_t>(saved, L.counts), offsets, sorted_slot, at<int32_t>(saved, L.row_of_slot),
                              tok_of_row, nt, at<int32_t>(saved, L.id_error), at<int32_t>(workspace, W.rs.blockhist),
                              at<int32_t>(workspace, W.rs.blockbase), at<int32_t>(workspace, W.rs.blockerr), nullptr,
                              hmm::SharedTables{}, st);
      }
      if (e != hipSuccess) return hip_fail(e, "routing launch (64-row tiles)");
      Dims dn = d;
      dn.small = true;
      gn = row_groups(dn, nt, offsets, sorted_slot, tok_of_row);
    }
    {
      Stage stage("gmm1_group_swiglu", st);
      e = hmm::launch_gmm1_group(gn, xq, dsx, wq, dsw, topk_weights, d.H, d.I, h, a, aw, st);
    }
    if (e != hipSuccess) return hip_fail(e, "gmm1 launch");
  } else if (d.fp8) {
    uint8_t* xq = at<uint8_t>(workspace, W.xq);
    uint8_t* wq = at<uint8_t>(workspace, W.wq);
    float* dsx = at<float>(workspace, W.dsx);
    float* dsw = at<float>(workspace, W.dsw);
    {
      Stage stage("quant_x", st);
      e = hmm::launch_quant_rows_fp8((const uint16_t*)x, d.T, d.H, xq, dsx, st);
    }
    if (e != hipSuccess) return hip_fail(e, "token quantisation launch");
    {
      Stage stage("quant_w1", st);
      e = hmm::launch_quant_cols_fp8((const uint16_t*)up_w, d.E, d.H, 2 * d.I, at<float>(workspace, W.pmax), wq, dsw,
                                     st);
    }
    if (e != hipSuccess) return hip_fail(e, "weight quantisation launch");
    {
      Stage stage("gmm1_fp8_swiglu", st);
      e = hmm::launch_gmm1_fp8(g, xq, dsx, wq, dsw, topk_weights, d.H, d.I, h, a, aw, st);
    }
    if (e != hipSuccess) return hip_fail(e, "gmm1 launch");
  }
  if (d.fp8) {
    if (d.shared) {
      // the shared expert's up-projection stays bf16
      const hmm::Gmm1Job js{gs, (const uint16_t*)x, (const uint16_t*)up_s, ones, d.H, d.Is, hs, as, nullptr};
      Stage stage("shared_gmm1", st);
      e = hmm::launch_gmm1_swiglu(&js, 1, st);
    }
    if (e != hipSuccess) return hip_fail(e, "shared gmm1 launch");
  } else if (route_in_gmm1) {
    const hmm::RoutedGmm1Job j{{g, (const uint16_t*)x, (const uint16_t*)up_w, topk_weights, d.H, d.I, h, a, aw},
                               topk_ids, (int)d.E, (int)d.K, (int)hmm::max_big_tiles(d.S, d.E, d.small),
                               at<int32_t>(saved, L.counts), offsets, sorted_slot, at<int32_t>(saved, L.row_of_slot),
                               tok_of_row, tiles, at<int32_t>(saved, L.id_error), nullptr};
    s = run_route_gmm1(j, validate_ids, st);
    if (s != HMM_OK) return s;
  } else {
    const hmm::Gmm1Job jobs[2] = {{g, (const uint16_t*)x, (const uint16_t*)up_w, topk_weights, d.H, d.I, h, a, aw},
                                  {gs, (const uint16_t*)x, (const uint16_t*)up_s, ones, d.H, d.Is, hs, as, nullptr}};
    Stage stage(d.shared ? "gmm1_swiglu+shared" : "gmm1_swiglu", st);
    e = hmm::launch_gmm1_swiglu(jobs, nj, st);
    if (e != hipSuccess) return hip_fail(e, "gmm1 launch");
  }
  {
    const hmm::Gmm2Job jobs[2] = {{g, a, (const uint16_t*)down_w, d.H, d.I, o},
                                  {gs, as, (const uint16_t*)down_s, d.H, d.Is, os}};
    Stage stage(d.shared ? "gmm2+shared" : "gmm2", st);
    e = hmm::launch_gmm2(jobs, nj, st);
  }
  if (e != hipSuccess) return hip_fail(e, "gmm2 launch");
  {
    Stage stage("combine", st);
    e = hmm::launch_combine(o, at<int32_t>(saved, L.row_of_slot), topk_weights, d.T, (int)d.K, d.H, os, (uint16_t*)y,
                            st);
  }
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return validate_ids ? finish_id_check(d) : HMM_OK;
}

// The backward of hmm_backward and hmm_backward_shared.
hmm_status backward_impl(const Dims& d, const void* dy, const void* x, const int32_t* topk_ids,
                         const float* topk_weights, const void* up_w, const void* down_w, const void* up_s,
                         const void* down_s, const void* saved, size_t saved_bytes, void* dx, void* d_up_w,
                         void* d_down_w, void* d_up_s, void* d_down_s, float* d_topk_weights, void* workspace,
                         size_t workspace_bytes, void* stream) {
  hmm_status s;
  const bool ne = d.S > 0;
  if ((s = need(dy, ne, "dy")) || (s = need(x, ne, "x")) || (s = need(topk_ids, ne, "topk_ids")) ||
      (s = need(topk_weights, ne, "topk_weights")) || (s = need(up_w, true, "up_proj_weight")) ||
      (s = need(down_w, true, "down_proj_weight")) || (s = need(up_s, d.shared, "shared_up_proj_weight")) ||
      (s = need(down_s, d.shared, "shared_down_proj_weight")) || (s = need(saved, true, "saved")) ||
      (s = need(dx, ne, "dx")) || (s = need(d_up_w, true, "d_up_proj_weight")) ||
      (s = need(d_down_w, true, "d_down_proj_weight")) || (s = need(d_up_s, d.shared, "d_shared_up_proj_weight")) ||
      (s = need(d_down_s, d.shared, "d_shared_down_proj_weight")) ||
      (s = need(d_topk_weights, ne, "d_topk_weights")))
    return s;
  const hmm_saved_layout L = saved_layout(d);
  const BwdWork W = bwd_work(d);
  if ((s = need(workspace, W.total > 0, "workspace"))) return s;  // T = 0 needs no workspace
  if (saved_bytes < L.total) return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "saved %zu < %zu bytes", saved_bytes, L.total);
  if (workspace_bytes < W.total)
    return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, W.total);
  hipStream_t st = (hipStream_t)stream;

  const int32_t* offsets = at<int32_t>(saved, L.offsets);
  const int32_t* sorted_slot = at<int32_t>(saved, L.sorted_slot);
  const int32_t* row_of_slot = at<int32_t>(saved, L.row_of_slot);
  const int32_t* tok_of_row = at<int32_t>(saved, L.tok_of_row);
  hmm::RowGroups g = row_groups(d, at<int32_t>(saved, L.tiles), offsets, sorted_slot, tok_of_row);
  // the shared expert: one group of all tokens (tables recorded by the forward)
  const int32_t* s_offsets = at<int32_t>(saved, L.shared_offsets);
  const int32_t* s_idx = at<int32_t>(saved, L.shared_idx);
  const float* ones = at<float>(saved, L.shared_ones);
  const hmm::RowGroups gs = d.shared ? shared_groups(d, at<int32_t>(saved, L.shared_tiles), s_offsets, s_idx)
                                     : hmm::RowGroups{};
  const uint16_t* h = at<uint16_t>(saved, L.h);
  const uint16_t* a = at<uint16_t>(saved, L.a);
  const uint16_t* aw = at<uint16_t>(saved, L.aw);
  const uint16_t* as = at<uint16_t>(saved, L.shared_a);
  uint16_t* dh = at<uint16_t>(workspace, W.dh);
  uint16_t* dxp = at<uint16_t>(workspace, W.dxp);
  uint16_t* dhs = d.shared ? at<uint16_t>(workspace, W.dhs) : nullptr;
  float* dwpart = at<float>(workspace, W.dwpart);
  hipError_t e = hipSuccess;
  if (d.f32) {
    uint16_t* dy2 = at<uint16_t>(workspace, W.dy2);
    float* dxp32 = at<float>(workspace, W.dxp);
    float* dxs32 = d.shared ? at<float>(workspace, W.dxs) : nullptr;
    const float* h32 = at<float>(saved, L.h);
    if (ne) {
      {
        Stage stage("split_dy", st);
        e = hmm::launch_split_rows((const float*)dy, d.T, d.H, dy2, st);
      }
      if (e != hipSuccess) return hip_fail(e, "dY split launch");
      {
        Stage stage("act_grad", st);
        e = hmm::launch_act_grad_f32(g, dy2, (const uint16_t*)down_w, topk_weights, h32, a, d.H, d.I, dh, dwpart,
                                     W.dw_cols, st);
      }
      if (e != hipSuccess) return hip_fail(e, "act_grad launch");
      if (d.shared) {
        Stage stage("shared_act_grad", st);
        e = hmm::launch_act_grad_f32(gs, dy2, (const uint16_t*)down_s, ones, at<float>(saved, L.shared_h), as, d.H,
                                     d.Is, dhs, nullptr, 0, st);
      }
      if (e != hipSuccess) return hip_fail(e, "shared act_grad launch");
      {
        Stage stage("input_grad", st);
        e = hmm::launch_input_grad_f32(g, dh, (const uint16_t*)up_w, d.H, d.I, dxp32, st);
      }
      if (e != hipSuccess) return hip_fail(e, "input_grad launch");
      if (d.shared) {
        Stage stage("shared_input_grad", st);
        e = hmm::launch_input_grad_f32(gs, dhs, (const uint16_t*)up_s, d.H, d.Is, dxs32, st);
      }
      if (e != hipSuccess) return hip_fail(e, "shared input_grad launch");
      {
        Stage stage("combine_dx", st);
        e = hmm::launch_combine_dx_f32(dxp32, row_of_slot, d.T, (int)d.K, d.H, dxs32, (float*)dx, dwpart, W.dw_cols,
                                       d_topk_weights, st);
      }
      if (e != hipSuccess) return hip_fail(e, "combine(dX) launch");
    }
    {
      Stage stage("dw2", st);
      e = hmm::launch_dw2_f32(offsets, tok_of_row, d.T, d.S, d.E, aw, dy2, d.H, d.I, (float*)d_down_w, d.small, st);
    }
    if (e != hipSuccess) return hip_fail(e, "W2Grad launch");
    if (d.shared) {
      Stage stage("shared_dw2", st);
      e = hmm::launch_dw2_f32(s_offsets, s_idx, d.T, d.T, 1, as, dy2, d.H, d.Is, (float*)d_down_s, d.small, st);
    }
    if (e != hipSuccess) return hip_fail(e, "shared W2Grad launch");
    {
      Stage stage("dw1", st);
      e = hmm::launch_dw1_f32(offsets, tok_of_row, d.T, d.S, d.E, (const uint16_t*)x, dh, d.H, d.I, (float*)d_up_w,
                              d.small, st);
    }
    if (e != hipSuccess) return hip_fail(e, "W1Grad launch");
    if (d.shared) {
      Stage stage("shared_dw1", st);
      e = hmm::launch_dw1_f32(s_offsets, s_idx, d.T, d.T, 1, (const uint16_t*)x, dhs, d.H, d.Is, (float*)d_up_s,
                              d.small, st);
    }
    return e == hipSuccess ? HMM_OK : hip_fail(e, "shared W1Grad launch");
  }
  uint16_t* dxs = d.shared ? at<uint16_t>(workspace, W.dxs) : nullptr;
  // jobs per product launch: the routed experts, then the shared expert
  const int nj = d.shared ? 2 : 1;
  const hmm::ActGradJob ag[2] = {
      {g, (const uint16_t*)dy, (const uint16_t*)down_w, topk_weights, h, d.H, d.I, dh, dwpart, W.dw_cols},
      {gs, (const uint16_t*)dy, (const uint16_t*)down_s, ones, at<uint16_t>(saved, L.shared_h), d.H, d.Is, dhs,
       nullptr, 0}};
  const hmm::InputGradJob ig[2] = {{g, dh, (const uint16_t*)up_w, d.H, d.I, dxp},
                                   {gs, dhs, (const uint16_t*)up_s, d.H, d.Is, dxs}};
  hmm::DwJob dw2[2] = {
      hmm::dw2_job(offsets, tok_of_row, d.T, d.S, d.E, aw, (const uint16_t*)dy, d.H, d.I, (uint16_t*)d_down_w),
      hmm::dw2_job(s_offsets, s_idx, d.T, d.T, 1, as, (const uint16_t*)dy, d.H, d.Is, (uint16_t*)d_down_s)};
  hmm::DwJob dw1[2] = {
      hmm::dw1_job(offsets, tok_of_row, d.T, d.S, d.E, (const uint16_t*)x, dh, d.H, d.I, (uint16_t*)d_up_w),
      hmm::dw1_job(s_offsets, s_idx, d.T, d.T, 1, (const uint16_t*)x, dhs, d.H, d.Is, (uint16_t*)d_up_s)};
  if (ne && !d.small) {
    // large tiling: the routed weight gradients take the experts longest first
    // (their cost grows with the row count; a large expert last would run alone
    // at the launch's end)
    int32_t* order = at<int32_t>(workspace, W.order);
    {
      Stage stage("expert_order", st);
      e = hmm::launch_expert_order(at<int32_t>(saved, L.counts), (int)d.E, order, st);
    }
    if (e != hipSuccess) return hip_fail(e, "expert order launch");
    dw1[0].order = dw2[0].order = order;
  }
  if (d.fp8bwd) {
    // FP8 backward: dY and the rows of W2 quantised per row, act_grad on E4M3 (dH
    // and the d_topk_weights partials as in bf16), dH and the rows of W1 quantised,
    // input_grad on E4M3; the shared expert's products, the combine and the weight
    // gradients in bf16.  One launch per product, on the caller's stream.
    if (ne) {
      uint8_t* dyq = at<uint8_t>(workspace, W.dyq);
      uint8_t* w2q = at<uint8_t>(workspace, W.w2q);
      uint8_t* dhq = at<uint8_t>(workspace, W.dhq);
      uint8_t* w1q = at<uint8_t>(workspace, W.w1q);
      float* dsy = at<float>(workspace, W.dsy);
      float* dsw2 = at<float>(workspace, W.dsw2);
      float* dsh = at<float>(workspace, W.dsh);
      float* dsw1 = at<float>(workspace, W.dsw1);
      {
        Stage stage("quant_dy", st);
        e = hmm::launch_quant_rows_fp8((const uint16_t*)dy, d.T, d.H, dyq, dsy, st);
      }
      if (e != hipSuccess) return hip_fail(e, "dY quantisation launch");
      {
        Stage stage("quant_w2", st);
        e = hmm::launch_quant_rows_fp8((const uint16_t*)down_w, d.E * d.I, d.H, w2q, dsw2, st);
      }
      if (e != hipSuccess) return hip_fail(e, "W2 quantisation launch");
      {
        Stage stage("act_grad_fp8", st);
        e = hmm::launch_act_grad_fp8(g, dyq, dsy, w2q, dsw2, topk_weights, h, d.H, d.I, dh, dwpart, W.dw_cols, st);
      }
      if (e != hipSuccess) return hip_fail(e, "act_grad launch");
      if (d.shared) {
        Stage stage("shared_act_grad", st);
        e = hmm::launch_act_grad(&ag[1], 1, st);
      }
      if (e != hipSuccess) return hip_fail(e, "shared act_grad launch");
      {
        Stage stage("quant_dh", st);
        e = hmm::launch_quant_rows_fp8(dh, d.S, 2 * d.I, dhq, dsh, st);
      }
      if (e != hipSuccess) return hip_fail(e, "dH quantisation launch");
      {
        Stage stage("quant_w1r", st);
        e = hmm::launch_quant_rows_fp8((const uint16_t*)up_w, d.E * d.H, 2 * d.I, w1q, dsw1, st);
      }
      if (e != hipSuccess) return hip_fail(e, "W1 quantisation launch");
      {
        Stage stage("input_grad_fp8", st);
        e = hmm::launch_input_grad_fp8(g, dhq, dsh, w1q, dsw1, d.H, d.I, dxp, st);
      }
      if (e != hipSuccess) return hip_fail(e, "input_grad launch");
      if (d.shared) {
        Stage stage("shared_input_grad", st);
        e = hmm::launch_input_grad(&ig[1], 1, st);
      }
      if (e != hipSuccess) return hip_fail(e, "shared input_grad launch");
      {
        Stage stage("combine_dx", st);
        e = hmm::launch_combine_dx(dxp, row_of_slot, d.T, (int)d.K, d.H, dxs, (uint16_t*)dx, dwpart, W.dw_cols,
                                   d_topk_weights, st);
      }
      if (e != hipSuccess) return hip_fail(e, "combine(dX) launch");
    }
    {
      Stage stage(d.shared ? "dw2+shared" : "dw2", st);
      e = hmm::launch_dw2(dw2, nj, d.small, st);
    }
    if (e != hipSuccess) return hip_fail(e, "W2Grad launch");
    {
      Stage stage(d.shared ? "dw1+shared" : "dw1", st);
      e = hmm::launch_dw1(dw1, nj, d.small, st);
    }
    return e == hipSuccess ? HMM_OK : hip_fail(e, "W1Grad launch");
  }
  if (ne && d.small) {
    // small problems: each product fills only part of the chip, so the independent
    // ones share a launch (RFC 2.2: W2Grad alongside act_grad, W1Grad alongside the
    // rest of the dX chain), the shared expert's with them
    {
      Stage stage(d.shared ? "act_grad+dw2+shared" : "act_grad+dw2", st);
      e = hmm::launch_act_grad_dw2_narrow(ag, dw2, nj, st);
    }
    if (e != hipSuccess) return hip_fail(e, "act_grad + W2Grad launch");
    {
      Stage stage(d.shared ? "input_grad+dw1+shared" : "input_grad+dw1", st);
      e = hmm::launch_input_grad_dw1_narrow(ig, dw1, nj, st);
    }
    if (e != hipSuccess) return hip_fail(e, "input_grad + W1Grad launch");
    {
      Stage stage("combine_dx", st);
      e = hmm::launch_combine_dx(dxp, row_of_slot, d.T, (int)d.K, d.H, dxs, (uint16_t*)dx, dwpart, W.dw_cols,
                                 d_topk_weights, st);
    }
    return e == hipSuccess ? HMM_OK : hip_fail(e, "combine(dX) launch");
  }
  // The weight gradients run on a second stream beside the dX chain (RFC 2.2:
  // W2Grad alongside act_grad, W1Grad alongside the rest of the dX chain) when
  // the products are short, so neither chain's last wave of tiles leaves the
  // chip idle and the HBM-bound Combine(dX) overlaps matrix work.  W2Grad needs
  // only the forward's aw and dY; W1Grad waits for act_grad's dH.  The caller's
  // stream waits for both.  With act_grad at 4 or more waves of 256-row tiles
  // on the chip, two products sharing the XCDs' L2 caches lose more than the
  // tails gain (measured per step on two streams: 18.25 -> 18.56 ms at T=8192,
  // H=7168, I=2048, E=32, K=8 with one hot expert; 2.37 -> 2.23 ms at T=4000,
  // H=2048, I=768, E=128, K=8 with Zipf routing), so those stay on one stream.
  DevState* side = nullptr;
  if (ne && !(d.flags & HMM_FLAG_SERIAL_BACKWARD)) {
    DevState* c = dev_state();
    const int64_t tiles = ((d.S + hmm::TILE_BIG - 1) / hmm::TILE_BIG) * ((d.I + 255) / 256);
    if (c && tiles < 4 * (int64_t)c->cus) side = side_state();
  }
  if (side) {
    hipStream_t s2 = side->side;
    if ((e = hipEventRecord(side->fork_ev, st)) != hipSuccess || (e = hipStreamWaitEvent(s2, side->fork_ev, 0)))
      return hip_fail(e, "backward fork");
    {
      Stage stage(d.shared ? "dw2+shared" : "dw2", s2);
      e = hmm::launch_dw2(dw2, nj, d.small, s2);
    }
    if (e != hipSuccess) return hip_fail(e, "W2Grad launch");
    {
      Stage stage(d.shared ? "act_grad+shared" : "act_grad", st);
      e = hmm::launch_act_grad(ag, nj, st);
    }
    if (e != hipSuccess) return hip_fail(e, "act_grad launch");
    if ((e = hipEventRecord(side->dh_ev, st)) != hipSuccess || (e = hipStreamWaitEvent(s2, side->dh_ev, 0)))
      return hip_fail(e, "dH event");
    {
      Stage stage(d.shared ? "dw1+shared" : "dw1", s2);
      e = hmm::launch_dw1(dw1, nj, d.small, s2);
    }
    if (e != hipSuccess) return hip_fail(e, "W1Grad launch");
    {
      Stage stage(d.shared ? "input_grad+shared" : "input_grad", st);
      e = hmm::launch_input_grad(ig, nj, st);
    }
    if (e != hipSuccess) return hip_fail(e, "input_grad launch");
    {
      Stage stage("combine_dx", st);
      e = hmm::launch_combine_dx(dxp, row_of_slot, d.T, (int)d.K, d.H, dxs, (uint16_t*)dx, dwpart, W.dw_cols,
                                 d_topk_weights, st);
    }
    if (e != hipSuccess) return hip_fail(e, "combine(dX) launch");
    if ((e = hipEventRecord(side->join_ev, s2)) != hipSuccess || (e = hipStreamWaitEvent(st, side->join_ev, 0)))
      return hip_fail(e, "backward join");
    return HMM_OK;
  }
  if (ne) {
    {
      Stage stage(d.shared ? "act_grad+shared" : "act_grad", st);
      e = hmm::launch_act_grad(ag, nj, st);
    }
    if (e != hipSuccess) return hip_fail(e, "act_grad launch");
    {
      Stage stage(d.shared ? "input_grad+shared" : "input_grad", st);
      e = hmm::launch_input_grad(ig, nj, st);
    }
    if (e != hipSuccess) return hip_fail(e, "input_grad launch");
    {
      Stage stage("combine_dx", st);
      e = hmm::launch_combine_dx(dxp, row_of_slot, d.T, (int)d.K, d.H, dxs, (uint16_t*)dx, dwpart, W.dw_cols,
                                 d_topk_weights, st);
    }
    if (e != hipSuccess) return hip_fail(e, "combine(dX) launch");
  }
  {
    Stage stage(d.shared ? "dw2+shared" : "dw2", st);
    e = hmm::launch_dw2(dw2, nj, d.small, st);
  }
  if (e != hipSuccess) return hip_fail(e, "W2Grad launch");
  {
    Stage stage(d.shared ? "dw1+shared" : "dw1", st);
    e = hmm::launch_dw1(dw1, nj, d.small, st);
  }
  return e == hipSuccess ? HMM_OK : hip_fail(e, "W1Grad launch");
}

}  // namespace

extern "C" {

hmm_status hmm_quant_rows_mx(const void* x, int64_t T, int64_t H, uint8_t* xq, uint8_t* xs, void* stream) {
  if (T < 0 || T > (int64_t)0x7fffffff) return fail(HMM_ERR_BAD_SHAPE, "T must be in [0, 2^31) (got %lld)", (long long)T);
  if (H < 32 || H % 32) return fail(HMM_ERR_BAD_SHAPE, "H must be a positive multiple of 32 (got %lld)", (long long)H);
  hmm_status s = quant_dims(T > 0 ? T : 1, H, 8);
  if (s != HMM_OK) return s;
  const bool ne = T > 0;
  if ((s = need(x, ne, "x")) || (s = need(xq, ne, "xq")) || (s = need(xs, ne, "xs"))) return s;
  Stage stage("quant_x_mx", (hipStream_t)stream);
  const hipError_t e = hmm::launch_quant_rows_mx((const uint16_t*)x, T, H, xq, xs, (hipStream_t)stream);
  return e == hipSuccess ? HMM_OK : hip_fail(e, "token quantisation launch");
}

hmm_status hmm_quant_cols_mx(const void* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, uint8_t* ws, void* stream) {
  hmm_status s = quant_dims(E, H, N);
  if (s != HMM_OK) return s;
  if (H % 32) return fail(HMM_ERR_BAD_SHAPE, "H must be a multiple of 32 (got %lld)", (long long)H);
  if ((s = need(w, true, "w")) || (s = need(wq, true, "wq")) || (s = need(ws, true, "ws"))) return s;
  Stage stage("quant_w1_mx", (hipStream_t)stream);
  const hipError_t e = hmm::launch_quant_cols_mx((const uint16_t*)w, E, H, N, wq, ws, (hipStream_t)stream);
  return e == hipSuccess ? HMM_OK : hip_fail(e, "weight quantisation launch");
}

hmm_status hmm_quant_rows_group(const void* x, int64_t T, int64_t H, uint8_t* xq, float* dsx, void* stream) {
  if (T < 0 || T > (int64_t)0x7fffffff) return fail(HMM_ERR_BAD_SHAPE, "T must be in [0, 2^31) (got %lld)", (long long)T);
  if (H < 128 || H % 128) return fail(HMM_ERR_BAD_SHAPE, "H must be a positive multiple of 128 (got %lld)", (long long)H);
  hmm_status s = quant_dims(T > 0 ? T : 1, H, 8);
  if (s != HMM_OK) return s;
  const bool ne = T > 0;
  if ((s = need(x, ne, "x")) || (s = need(xq, ne, "xq")) || (s = need(dsx, ne, "dsx"))) return s;
  Stage stage("quant_x_group", (hipStream_t)stream);
  const hipError_t e = hmm::launch_quant_rows_group((const uint16_t*)x, T, H, xq, dsx, (hipStream_t)stream);
  return e == hipSuccess ? HMM_OK : hip_fail(e, "token quantisation launch");
}

hmm_status hmm_quant_cols_group(const void* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, float* dsw,
                                void* stream) {
  hmm_status s = quant_dims(E, H, N);
  if (s != HMM_OK) return s;
  if (H % 128) return fail(HMM_ERR_BAD_SHAPE, "H must be a multiple of 128 (got %lld)", (long long)H);
  if ((s = need(w, true, "w")) || (s = need(wq, true, "wq")) || (s = need(dsw, true, "dsw"))) return s;
  Stage stage("quant_w1_group", (hipStream_t)stream);
  const hipError_t e = hmm::launch_quant_cols_group((const uint16_t*)w, E, H, N, wq, dsw, (hipStream_t)stream);
  return e == hipSuccess ? HMM_OK : hip_fail(e, "weight quantisation launch");
}

}  // extern "C"

// ------------------------------------------------------------- no-allocation forward
// hmm_forward_noalloc takes its workspace from this file-scope device array:
// one copy per device, held from the library's load on that device until the
// process ends.  In host code the name is only a host-side stand-in; the
// array's device address comes from hipGetSymbolAddress, once per device, and
// only that address is handed to kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
struct NoallocScratch {
  std::mutex m;
  void* ptr[MAX_DEVICES] = {};
};
NoallocScratch g_noalloc;

// The current device's address of ``scratch`` (looked up on its first use there).
hmm_status noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(HMM_ERR_UNSUPPORTED, "device %d is beyond the %d tracked", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_noalloc.m);
  if (!g_noalloc.ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "address of the no-allocation scratch");
    if (!ptr) return fail(HMM_ERR_HIP, "the no-allocation scratch has no device address");
    g_noalloc.ptr[dev] = ptr;
  }
  *out = g_noalloc.ptr[dev];
  return HMM_OK;
}

// Stage timing off for the guard's lifetime (its events are created on first use).
struct ProfPause {
  bool was = g_prof.on;
  ProfPause() { g_prof.on = false; }
  ~ProfPause() { g_prof.on = was; }
};
}  // namespace

extern "C" {

hmm_status hmm_forward_noalloc(const hmm_problem* p, const void* x, const int32_t* topk_ids,
                               const float* topk_weights, const void* up_w, const void* down_w, void* y, void* saved,
                               size_t saved_bytes, void* stream) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (d.shared) return fail(HMM_ERR_BAD_SHAPE, "shared_I != 0: the no-allocation forward has no shared expert");
  if (p->flags & (HMM_FLAG_VALIDATE_IDS | HMM_FLAG_FUSED_FORWARD))
    return fail(HMM_ERR_UNSUPPORTED, "the no-allocation forward takes neither HMM_FLAG_VALIDATE_IDS nor "
                "HMM_FLAG_FUSED_FORWARD (both need pinned host memory and events created on first use); invalid "
                "ids are dropped and flagged in saved's id_error word");
  const size_t need_bytes = fwd_work(d).total;
  if (need_bytes > NOALLOC_SCRATCH_BYTES)
    return fail(HMM_ERR_WORKSPACE_TOO_SMALL, "the problem needs %zu bytes of forward workspace; the no-allocation "
                "forward holds %zu (use hmm_forward with a workspace)", need_bytes, NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if ((s = noalloc_scratch(&ptr)) != HMM_OK) return s;
  ProfPause pause;
  return forward_impl(p, d, x, topk_ids, topk_weights, up_w, down_w, nullptr, nullptr, y, saved, saved_bytes, ptr,
                      NOALLOC_SCRATCH_BYTES, stream);
}

hmm_status hmm_forward(const hmm_problem* p, const void* x, const int32_t* topk_ids, const float* topk_weights,
                       const void* up_w, const void* down_w, void* y, void* saved, size_t saved_bytes,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (d.shared) return fail(HMM_ERR_BAD_SHAPE, "shared_I != 0: call hmm_forward_shared with the shared weights");
  return forward_impl(p, d, x, topk_ids, topk_weights, up_w, down_w, nullptr, nullptr, y, saved, saved_bytes,
                      workspace, workspace_bytes, stream);
}

hmm_status hmm_forward_shared(const hmm_problem* p, const void* x, const int32_t* topk_ids, const float* topk_weights,
                              const void* up_w, const void* down_w, const void* shared_up_w,
                              const void* shared_down_w, void* y, void* saved, size_t saved_bytes, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  return forward_impl(p, d, x, topk_ids, topk_weights, up_w, down_w, shared_up_w, shared_down_w, y, saved,
                      saved_bytes, workspace, workspace_bytes, stream);
}

hmm_status hmm_backward(const hmm_problem* p, const void* dy, const void* x, const int32_t* topk_ids,
                        const float* topk_weights, const void* up_w, const void* down_w, const void* saved,
                        size_t saved_bytes, void* dx, void* d_up_w, void* d_down_w, float* d_topk_weights,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  if (d.shared) return fail(HMM_ERR_BAD_SHAPE, "shared_I != 0: call hmm_backward_shared with the shared weights");
  return backward_impl(d, dy, x, topk_ids, topk_weights, up_w, down_w, nullptr, nullptr, saved, saved_bytes, dx,
                       d_up_w, d_down_w, nullptr, nullptr, d_topk_weights, workspace, workspace_bytes, stream);
}

hmm_status hmm_backward_shared(const hmm_problem* p, const void* dy, const void* x, const int32_t* topk_ids,
                               const float* topk_weights, const void* up_w, const void* down_w,
                               const void* shared_up_w, const void* shared_down_w, const void* saved,
                               size_t saved_bytes, void* dx, void* d_up_w, void* d_down_w, void* d_shared_up_w,
                               void* d_shared_down_w, float* d_topk_weights, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Dims d;
  hmm_status s = validate(p, &d);
  if (s != HMM_OK) return s;
  return backward_impl(d, dy, x, topk_ids, topk_weights, up_w, down_w, shared_up_w, shared_down_w, saved, saved_bytes,
                       dx, d_up_w, d_down_w, d_shared_up_w, d_shared_down_w, d_topk_weights, workspace,
                       workspace_bytes, stream);
}

hmm_status hmm_profile_enable(int32_t on) {
  g_prof.on = on != 0;
  return HMM_OK;
}

hmm_status hmm_profile_read(hmm_stage_time* out, int32_t max_stages, int32_t* n_stages, int32_t* dropped) {
  if (!n_stages) return fail(HMM_ERR_NULL_POINTER, "n_stages is NULL");
  Prof& P = g_prof;
  std::vector<hmm_stage_time> acc;
  for (auto& m : P.marks) {
    hipEvent_t a = P.pool[m.second.first], b = P.pool[m.second.second];
    hipError_t e = hipEventSynchronize(b);
    if (e != hipSuccess) return hip_fail(e, "profile event wait");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, a, b);
    if (e != hipSuccess) return hip_fail(e, "profile event time");
    hmm_stage_time* slot = nullptr;
    for (auto& x : acc)
      if (m.first == x.name) slot = &x;
    if (!slot) {
      acc.push_back(hmm_stage_time{});
      slot = &acc.back();
      std::snprintf(slot->name, sizeof slot->name, "%s", m.first.c_str());
    }
    slot->launches += 1;
    slot->ms += ms;
  }
  *n_stages = (int32_t)acc.size();
  if (dropped) *dropped = P.dropped;
  if (out)
    for (int32_t i = 0; i < (int32_t)acc.size() && i < max_stages; ++i) out[i] = acc[i];
  P.marks.clear();
  P.used = 0;
  P.dropped = 0;
  return HMM_OK;
}

}  // extern "C"
