// Bandwidth-bound steps of the path:
//   combine      (HyperMegaMoE RFC section 2.1 Combine and 4.1: outputs return to
//                 their token and are summed with the top-k weights; section 2.2
//                 Combine(dX): the same gather without weights)
//                 out[t] = sum_k w[t,k] * rows[row_of_slot[t*K+k]]   (w = 1 if NULL)
//                          (+ extra[t], the shared expert's row, when given)
//                 in float32, k ascending, the extra term last, then one bf16
//                 rounding; no atomics, so the result is deterministic.
//   combine(dX) also finalises d_topk_weights[s] = sum_c dwpart[row_of_slot[s]][c],
//                c ascending, in the threads of each token's first K chunks.
#include "device.h"
#include "kernels.h"

namespace hmm {

constexpr int PW_THREADS = 256;

// 8 consecutive elements of a row: bf16 (one 16-byte load / store) or float32 (two)
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) { unpack8(*reinterpret_cast<const u32x4*>(p), v); }
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = b[j];
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) { *reinterpret_cast<u32x4*>(p) = pack8(v); }
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = (f32x4){v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = (f32x4){v[4], v[5], v[6], v[7]};
}

// Streaming (non-temporal) forms for the combines: every gathered row chunk is
// read once and every output chunk written once, so they bypass the caches'
// normal retention (measured: 15% more bandwidth on the largest workload).
struct Raw8 {  // 8 elements as loaded: bf16 (one vector) or float32 (two)
  u32x4 a, b;
};
__device__ __forceinline__ Raw8 load8_nt(const uint16_t* p) {
  return Raw8{__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)), u32x4{}};
}
__device__ __forceinline__ Raw8 load8_nt(const float* p) {
  return Raw8{__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)),
              __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4))};
}
__device__ __forceinline__ void unraw(const Raw8& r, const uint16_t*, float (&v)[8]) { unpack8(r.a, v); }
__device__ __forceinline__ void unraw(const Raw8& r, const float*, float (&v)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = __uint_as_float(r.a[j]);
    v[4 + j] = __uint_as_float(r.b[j]);
  }
}
__device__ __forceinline__ void store8_nt(uint16_t* p, const float (&v)[8]) {
  __builtin_nontemporal_store(pack8(v), reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float (&v)[8]) {
  __builtin_nontemporal_store((f32x4){v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store((f32x4){v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(p + 4));
}

// One thread per 8 consecutive hidden elements of one token (16-byte loads).
// With dwpart, the thread of chunk k (< K) of a token also finalises slot k of
// that token: dw[s] = sum_c dwpart[row_of_slot[s]][c], c ascending.  T is bf16
// (the default) or float32 (the accuracy mode) for both the rows and the output.
template <bool WEIGHTED, class T_>
__global__ void __launch_bounds__(PW_THREADS) combine_kernel(const T_* __restrict__ rows,
                                                             const int32_t* __restrict__ row_of_slot,
                                                             const float* __restrict__ tw, int64_t T, int K,
                                                             int64_t H, const T_* __restrict__ extra,
                                                             T_* __restrict__ out,
                                                             const float* __restrict__ dwpart, int dw_cols,
                                                             float* __restrict__ dw) {
  const int64_t chunks_per_row = H >> 3;
  const int64_t total = T * chunks_per_row;
  for (int64_t idx = (int64_t)blockIdx.x * PW_THREADS + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * PW_THREADS) {
    const int64_t t = idx / chunks_per_row;
    const int64_t c = idx - t * chunks_per_row;
    // the gathered loads of up to 8 slots are issued before their sums (unrolled
    // with a guard so the chunks stay in registers), slots summed in ascending k
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += 8) {
      Raw8 raw[8];
      float wk[8];
      bool ok[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = k0 + q;
        ok[q] = false;
        wk[q] = 0.f;
        if (k < K) {
          const int64_t s = t * K + k;
          const int r = row_of_slot[s];
          if (r >= 0) {
            ok[q] = true;
            wk[q] = WEIGHTED ? tw[s] : 1.f;
            raw[q] = load8_nt(rows + (int64_t)r * H + c * 8);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (ok[q]) {
          float v[8];
          unraw(raw[q], rows, v);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = WEIGHTED ? __builtin_fmaf(wk[q], v[j], acc[j]) : acc[j] + v[j];
        }
      }
    }
    if (extra) {  // the shared expert's row of this token, weight 1, after the K routed terms
      float v[8];
      unraw(load8_nt(extra + t * H + c * 8), extra, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
    store8_nt(out + t * H + c * 8, acc);
    if (dwpart) {
      for (int64_t k = c; k < K; k += chunks_per_row) {
        const int64_t s = t * K + k;
        const int r = row_of_slot[s];
        float a = 0.f;
        if (r >= 0) {
          const float* p = dwpart + (int64_t)r * dw_cols;
          for (int q = 0; q < dw_cols; ++q) a += p[q];
        }
        dw[s] = a;
      }
    }
  }
}

static unsigned grid_for(int64_t work, int64_t cap) {
  int64_t g = (work + PW_THREADS - 1) / PW_THREADS;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

template <class T_>
hipError_t combine_t(const T_* rows, const int32_t* row_of_slot, const float* topk_w, int64_t T, int K, int64_t H,
                     const T_* extra, T_* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const unsigned g = grid_for(T * (H / 8), 1 << 20);
  hipLaunchKernelGGL((combine_kernel<true, T_>), dim3(g), dim3(PW_THREADS), 0, stream, rows, row_of_slot, topk_w, T,
                     K, H, extra, out, nullptr, 0, nullptr);
  return hipGetLastError();
}

template <class T_>
hipError_t combine_dx_t(const T_* rows, const int32_t* row_of_slot, int64_t T, int K, int64_t H, const T_* extra,
                        T_* dx, const float* dwpart, int dw_cols, float* dw, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const unsigned g = grid_for(T * (H / 8), 1 << 20);
  hipLaunchKernelGGL((combine_kernel<false, T_>), dim3(g), dim3(PW_THREADS), 0, stream, rows, row_of_slot, nullptr,
                     T, K, H, extra, dx, dwpart, dw_cols, dw);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* rows, const int32_t* row_of_slot, const float* topk_w, int64_t T, int K,
                          int64_t H, const uint16_t* extra, uint16_t* out, hipStream_t stream) {
  return combine_t(rows, row_of_slot, topk_w, T, K, H, extra, out, stream);
}
hipError_t launch_combine_dx(const uint16_t* rows, const int32_t* row_of_slot, int64_t T, int K, int64_t H,
                             const uint16_t* extra, uint16_t* dx, const float* dwpart, int dw_cols, float* dw,
                             hipStream_t stream) {
  return combine_dx_t(rows, row_of_slot, T, K, H, extra, dx, dwpart, dw_cols, dw, stream);
}
hipError_t launch_combine_f32(const float* rows, const int32_t* row_of_slot, const float* topk_w, int64_t T, int K,
                              int64_t H, const float* extra, float* out, hipStream_t stream) {
  return combine_t(rows, row_of_slot, topk_w, T, K, H, extra, out, stream);
}
hipError_t launch_combine_dx_f32(const float* rows, const int32_t* row_of_slot, int64_t T, int K, int64_t H,
                                 const float* extra, float* dx, const float* dwpart, int dw_cols, float* dw,
                                 hipStream_t stream) {
  return combine_dx_t(rows, row_of_slot, T, K, H, extra, dx, dwpart, dw_cols, dw, stream);
}

// x float32 [n][H] -> out bf16 [n][2H]: [hi | lo] with hi = bf16(v), lo = bf16(v - hi)
__global__ void __launch_bounds__(PW_THREADS) split_rows_kernel(const float* __restrict__ x, int64_t n, int64_t H,
                                                                uint16_t* __restrict__ out) {
  const int64_t cpr = H >> 3, total = n * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * PW_THREADS + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * PW_THREADS) {
    const int64_t t = idx / cpr, c = idx - t * cpr;
    float v[8], hi[8], lo[8];
    load8(x + t * H + c * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hi[j] = round_bf(v[j]);
      lo[j] = v[j] - hi[j];
    }
    store8(out + t * 2 * H + c * 8, hi);
    store8(out + t * 2 * H + H + c * 8, lo);
  }
}

hipError_t launch_split_rows(const float* x, int64_t n, int64_t H, uint16_t* out, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const unsigned g = grid_for(n * (H / 8), 1 << 20);
  hipLaunchKernelGGL(split_rows_kernel, dim3(g), dim3(PW_THREADS), 0, stream, x, n, H, out);
  return hipGetLastError();
}

}  // namespace hmm
