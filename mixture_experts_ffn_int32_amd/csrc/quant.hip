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

// ----------------------------------------------------------------------------- MX
// MoeDistributeDispatchV2 case 5 (mx): per block of 32 elements along the
// hidden dimension, shared exponent e = floor(log2 max|x|) - 8 (8: the exponent
// of E4M3's largest value, 448 = 1.75 * 2^8), clamped to E8M0's [-127, 127],
// -127 for an all-zero block; codes = round-to-nearest-even E4M3 of x * 2^-e,
// saturated at +-448 (x * 2^-e reaches up to 2^9).  The exponent is stored as
// its E8M0 byte e + 127.  floor(log2 m) of a positive float is its unbiased
// exponent field (a subnormal m gives -127, which the clamp maps like any
// exponent below -119); x * 2^-e is exact (a power-of-two product whose
// result is either a normal float or, if subnormal, below E4M3's rounding
// threshold 2^-10 either way).
__device__ __forceinline__ int mx_exp(float absmax) {
  const int field = (int)((__float_as_uint(absmax) >> 23) & 0xff);
  const int e = absmax > 0.f ? field - 127 - 8 : -127;
  return min(127, max(-127, e));
}

// 8 values times 2^-e -> 8 saturated E4M3 bytes
__device__ __forceinline__ uint2 mx_codes8(const float (&v)[8], int e) {
  const float s = __builtin_ldexpf(1.f, -e);  // e <= 120 for bf16 data: a normal float
  float c[8], one[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[j] = fminf(448.f, fmaxf(-448.f, v[j] * s));
    one[j] = 1.f;
  }
  return to_e4m3x8(c, one);
}

// x [T][H] -> xq [T][H], xs [T][H/32]; four consecutive threads share a block
__global__ void __launch_bounds__(QT) quant_rows_mx(const uint16_t* __restrict__ x, int64_t chunks, int64_t H,
                                                    uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  // chunks is a multiple of 4 and QT of 4: the four lanes of a block run the same iterations
  for (int64_t c = (int64_t)blockIdx.x * QT + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * QT) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(x + c * 8), v);
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int e = mx_exp(m);
    *reinterpret_cast<uint2*>(xq + c * 8) = mx_codes8(v, e);
    if ((c & 3) == 0) xs[c >> 2] = (uint8_t)(e + 127);
  }
}

// w [E][H][N] -> wq [E][H][N], ws [E][N][H/32]: one thread per (expert, 32-row
// block, 8 columns); consecutive threads take consecutive column chunks.
__global__ void __launch_bounds__(QT) quant_cols_mx(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                    int64_t N, uint8_t* __restrict__ wq, uint8_t* __restrict__ ws) {
  const int64_t n8s = N / 8, hbs = H / 32;
  const int64_t g = (int64_t)blockIdx.x * QT + threadIdx.x;
  if (g >= E * hbs * n8s) return;
  const int64_t e = g / (hbs * n8s);
  const int64_t rem = g - e * hbs * n8s;
  const int64_t hb = rem / n8s, n8 = rem - hb * n8s;
  const uint16_t* base = w + (e * H + hb * 32) * N + n8 * 8;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < 32; ++r) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(base + r * N), v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(v[j]));
  }
  int ex[8];
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ex[j] = mx_exp(m[j]);
    s[j] = __builtin_ldexpf(1.f, -ex[j]);
    ws[(e * N + n8 * 8 + j) * hbs + hb] = (uint8_t)(ex[j] + 127);
  }
  for (int r = 0; r < 32; ++r) {
    float v[8], one[8];
    unpack8(*reinterpret_cast<const u32x4*>(base + r * N), v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = fminf(448.f, fmaxf(-448.f, v[j] * s[j]));
      one[j] = 1.f;
    }
    *reinterpret_cast<uint2*>(wq + (e * H + hb * 32 + r) * N + n8 * 8) = to_e4m3x8(v, one);
  }
}

hipError_t launch_quant_rows_mx(const uint16_t* x, int64_t T, int64_t H, uint8_t* xq, uint8_t* xs,
                                hipStream_t stream) {
  const int64_t chunks = T * (H / 8);
  if (chunks <= 0) return hipSuccess;
  int64_t blocks = (chunks + QT - 1) / QT;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  hipLaunchKernelGGL(quant_rows_mx, dim3((unsigned)blocks), dim3(QT), 0, stream, x, chunks, H, xq, xs);
  return hipGetLastError();
}

hipError_t launch_quant_cols_mx(const uint16_t* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, uint8_t* ws,
                                hipStream_t stream) {
  const int64_t work = E * (H / 32) * (N / 8);
  if (work <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_cols_mx, dim3((unsigned)((work + QT - 1) / QT)), dim3(QT), 0, stream, w, E, H, N, wq, ws);
  return hipGetLastError();
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
