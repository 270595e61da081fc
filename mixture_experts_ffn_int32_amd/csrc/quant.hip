// Dynamic FP8 E4M3 quantisation for the FP8 up-projection.
//
// MoeDistributeDispatchV2, function description, case 3 (per-token dynamic
// quantisation): a row is taken to float32, its scale is 448 / max|row|
// (448 = the largest E4M3 value), the quantised row is the cast of row * scale,
// and 1 / scale travels with it.  The weight operand of an FP8 product must be
// FP8 as well; it gets the same rule per (expert, output column), the maximum
// taken over the hidden dimension.  An all-zero row or column gets scale 1.
//
// Every decision is taken in float32 exactly as stated: an IEEE division for
// the scale, one float32 product, then the hardware's round-to-nearest-even
// conversion to E4M3 (v_cvt_pk_fp8_f32; |row * scale| never exceeds 448 by
// more than a rounding of the product, which still converts to 448).
#include "device.h"
#include "kernels.h"

namespace hmm {

constexpr int QT = 256;  // threads per quantisation block
constexpr int QH = 256;  // hidden rows per column-maximum chunk

__device__ __forceinline__ float scale_of(float absmax) { return absmax > 0.f ? 448.f / absmax : 1.f; }

// 8 floats * scale -> 8 E4M3 bytes
__device__ __forceinline__ uint2 to_e4m3x8(const float (&v)[8], const float (&s)[8]) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * s[0], v[1] * s[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * s[2], v[3] * s[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * s[4], v[5] * s[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * s[6], v[7] * s[7], hi, true);
  return make_uint2((unsigned)lo, (unsigned)hi);
}

// One block per token row: xq[t] = e4m3(x[t] * scale), dsx[t] = 1 / scale.
__global__ void __launch_bounds__(QT) quant_rows_fp8(const uint16_t* __restrict__ x, int64_t H,
                                                     uint8_t* __restrict__ xq, float* __restrict__ dsx) {
  __shared__ float wmax[QT / 64];
  const int64_t t = blockIdx.x;
  const uint16_t* row = x + t * H;
  float m = 0.f;
  for (int64_t c = threadIdx.x; c < H / 8; c += QT) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(row + c * 8), v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < QT / 64; ++q) m = fmaxf(m, wmax[q]);
  const float sx = scale_of(m);
  if (threadIdx.x == 0) dsx[t] = 1.f / sx;
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = sx;
  for (int64_t c = threadIdx.x; c < H / 8; c += QT) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(row + c * 8), v);
    *reinterpret_cast<uint2*>(xq + t * H + c * 8) = to_e4m3x8(v, s);
  }
}

// Pass 1 of the weight quantisation: per (column chunk of 8, hidden chunk of
// QH rows) the column maxima -> pmax[hc][e][n].  Consecutive threads take
// consecutive column chunks of the same rows (coalesced).
__global__ void __launch_bounds__(QT) quant_cols_max(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                     int64_t N, float* __restrict__ pmax) {
  const int64_t n8s = N / 8;
  const int64_t g = (int64_t)blockIdx.x * QT + threadIdx.x;
  const int64_t HC = (H + QH - 1) / QH;
  if (g >= HC * E * n8s) return;
  const int64_t hc = g / (E * n8s);
  const int64_t rem = g - hc * E * n8s;
  const int64_t e = rem / n8s, n8 = rem - e * n8s;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t h1 = min(H, (hc + 1) * QH);
  for (int64_t h = hc * QH; h < h1; ++h) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(w + (e * H + h) * N + n8 * 8), v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(v[j]));
  }
  float* out = pmax + (hc * E + e) * N + n8 * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = m[j];
}

// Pass 2: column scale from the chunk maxima, then the chunk's rows quantised.
__global__ void __launch_bounds__(QT) quant_cols_apply(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                       int64_t N, const float* __restrict__ pmax,
                                                       uint8_t* __restrict__ wq, float* __restrict__ dsw) {
  const int64_t n8s = N / 8;
  const int64_t g = (int64_t)blockIdx.x * QT + threadIdx.x;
  const int64_t HC = (H + QH - 1) / QH;
  if (g >= HC * E * n8s) return;
  const int64_t hc = g / (E * n8s);
  const int64_t rem = g - hc * E * n8s;
  const int64_t e = rem / n8s, n8 = rem - e * n8s;
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.f;
    for (int64_t q = 0; q < HC; ++q) m = fmaxf(m, pmax[(q * E + e) * N + n8 * 8 + j]);
    s[j] = scale_of(m);
    if (hc == 0) dsw[e * N + n8 * 8 + j] = 1.f / s[j];
  }
  const int64_t h1 = min(H, (hc + 1) * QH);
  for (int64_t h = hc * QH; h < h1; ++h) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(w + (e * H + h) * N + n8 * 8), v);
    *reinterpret_cast<uint2*>(wq + (e * H + h) * N + n8 * 8) = to_e4m3x8(v, s);
  }
}

hipError_t launch_quant_rows_fp8(const uint16_t* x, int64_t T, int64_t H, uint8_t* xq, float* dsx,
                                 hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_fp8, dim3((unsigned)T), dim3(QT), 0, stream, x, H, xq, dsx);
  return hipGetLastError();
}

int64_t quant_cols_chunks(int64_t H) { return (H + QH - 1) / QH; }

hipError_t launch_quant_cols_fp8(const uint16_t* w, int64_t E, int64_t H, int64_t N, float* pmax, uint8_t* wq,
                                 float* dsw, hipStream_t stream) {
  const int64_t work = quant_cols_chunks(H) * E * (N / 8);
  const unsigned blocks = (unsigned)((work + QT - 1) / QT);
  hipLaunchKernelGGL(quant_cols_max, dim3(blocks), dim3(QT), 0, stream, w, E, H, N, pmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_cols_apply, dim3(blocks), dim3(QT), 0, stream, w, E, H, N, pmax, wq, dsw);
  return hipGetLastError();
}

}  // namespace hmm
