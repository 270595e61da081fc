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

// 448 / max|x| in float32; an all-zero row or group gets 1.  Below a largest
// value of about 1.3e-36 (bf16 holds values down to ~9e-41) the quotient
// overflows: it is clamped to the largest finite float32, so the codes stay
// finite (x * scale is then at most ~448) and the descale 1 / scale is a
// subnormal float32 (about 2.9e-39) instead of 0.
__device__ __forceinline__ float scale_of(float absmax) {
  return absmax > 0.f ? fminf(448.f / absmax, 3.40282347e38f) : 1.f;
}

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

// The column quantisers give one wave a tile of 128 columns: lane l takes the
// 8-column chunk l % 16 and, of every 32 rows, the 8 rows 8 * (l / 16) + i, so
// one load instruction reads four 256-byte row segments and a lane has 8 loads
// in flight.  The four row groups of a column meet in two lane shuffles.  The
// wave's task and its row pointers are uniform (scalar registers); a lane adds
// a 32-bit byte offset, at most 32 rows of 2N bytes (N <= 2^24 is checked by
// the callers).
constexpr int QW = 4;    // waves per column-quantisation block
constexpr int QG = 16;   // 8-column chunks per wave tile (128 columns)

struct ColTask {
  int64_t e, cg, hg;     // expert, column group, row group
};

__device__ __forceinline__ int64_t wave_task() {
  return (int64_t)blockIdx.x * QW + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// column group fastest: the waves in flight together read side by side along
// rows rather than at one column offset a chunk of rows apart
__device__ __forceinline__ ColTask col_task(int64_t task, int64_t cgs, int64_t hgs) {
  ColTask t;
  t.cg = task % cgs;
  const int64_t r = task / cgs;
  t.hg = r % hgs;
  t.e = r / hgs;
  return t;
}

struct ColLane {
  int c, rs;             // column chunk within the group, row group of 8
  uint32_t n8;           // the lane's 8-column chunk, clamped into the matrix for loads
  bool ok;               // n8 is a real chunk (stores are guarded by it)
};

__device__ __forceinline__ ColLane col_lane(int64_t cg, int64_t n8s) {
  ColLane l;
  const int lane = threadIdx.x & 63;
  l.c = lane & 15;
  l.rs = lane >> 4;
  const int64_t n8 = cg * QG + l.c;
  l.ok = n8 < n8s;
  l.n8 = (uint32_t)(l.ok ? n8 : n8s - 1);
  return l;
}

__device__ __forceinline__ u32x4 load16(const char* row, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(row + off);
}

// running max |v| over a lane's 8 rows of 8 columns
__device__ __forceinline__ void rows_absmax(const u32x4 (&raw)[8], float (&m)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[8];
    unpack8(raw[i], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(v[j]));
  }
}

// the maxima of the wave's four row groups of a column (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ void wave_colmax(float (&m)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    m[j] = fmaxf(m[j], __shfl_xor(m[j], 16));
    m[j] = fmaxf(m[j], __shfl_xor(m[j], 32));
  }
}

// Pass 1 of the weight quantisation: the column maxima of each QH-row chunk ->
// pmax[hc][e][n].  Rows past the chunk's end are clamped onto its last row (a
// repeated row leaves a maximum unchanged).
__global__ void __launch_bounds__(64 * QW) quant_cols_max(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                          int64_t N, float* __restrict__ pmax) {
  const int64_t n8s = N / 8, cgs = (n8s + QG - 1) / QG, HC = (H + QH - 1) / QH;
  const int64_t task = wave_task();
  if (task >= E * cgs * HC) return;
  const ColTask t = col_task(task, cgs, HC);
  const ColLane l = col_lane(t.cg, n8s);
  const int64_t h0 = t.hg * QH, h1 = min(H, h0 + QH);
  const uint32_t pitch = (uint32_t)N * 2;
  const char* wb = reinterpret_cast<const char*>(w + t.e * H * N);
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t hb = h0; hb < h1; hb += 32) {
    const char* row = wb + hb * (int64_t)pitch;
    const int last = (int)min((int64_t)31, h1 - 1 - hb);
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = load16(row, l.n8 * 16u + (uint32_t)min(l.rs * 8 + i, last) * pitch);
    rows_absmax(raw, m);
  }
  wave_colmax(m);
  if (l.rs == 0 && l.ok) {
    float4* out = reinterpret_cast<float4*>(pmax + (t.hg * E + t.e) * N + l.n8 * 8);
    out[0] = make_float4(m[0], m[1], m[2], m[3]);
    out[1] = make_float4(m[4], m[5], m[6], m[7]);
  }
}

// Pass 2: column scale from the chunk maxima, then the chunk's rows quantised.
__global__ void __launch_bounds__(64 * QW) quant_cols_apply(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                            int64_t N, const float* __restrict__ pmax,
                                                            uint8_t* __restrict__ wq, float* __restrict__ dsw) {
  const int64_t n8s = N / 8, cgs = (n8s + QG - 1) / QG, HC = (H + QH - 1) / QH;
  const int64_t task = wave_task();
  if (task >= E * cgs * HC) return;
  const ColTask t = col_task(task, cgs, HC);
  const ColLane l = col_lane(t.cg, n8s);
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t q = 0; q < HC; ++q) {
    const float4* pm = reinterpret_cast<const float4*>(pmax + (q * E + t.e) * N + l.n8 * 8);
    const float4 a = pm[0], b = pm[1];
    m[0] = fmaxf(m[0], a.x); m[1] = fmaxf(m[1], a.y); m[2] = fmaxf(m[2], a.z); m[3] = fmaxf(m[3], a.w);
    m[4] = fmaxf(m[4], b.x); m[5] = fmaxf(m[5], b.y); m[6] = fmaxf(m[6], b.z); m[7] = fmaxf(m[7], b.w);
  }
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = scale_of(m[j]);
  if (t.hg == 0 && l.rs == 0 && l.ok) {
    float4* out = reinterpret_cast<float4*>(dsw + t.e * N + l.n8 * 8);
    out[0] = make_float4(1.f / s[0], 1.f / s[1], 1.f / s[2], 1.f / s[3]);
    out[1] = make_float4(1.f / s[4], 1.f / s[5], 1.f / s[6], 1.f / s[7]);
  }
  const int64_t h0 = t.hg * QH, h1 = min(H, h0 + QH);
  const uint32_t pitch = (uint32_t)N * 2;
  const char* wb = reinterpret_cast<const char*>(w + t.e * H * N);
  uint8_t* qb = wq + t.e * H * N;
  for (int64_t hb = h0; hb < h1; hb += 32) {
    const char* row = wb + hb * (int64_t)pitch;
    uint8_t* qrow = qb + hb * N;
    const int last = (int)min((int64_t)31, h1 - 1 - hb);
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = load16(row, l.n8 * 16u + (uint32_t)min(l.rs * 8 + i, last) * pitch);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      unpack8(raw[i], v);
      const int r = l.rs * 8 + i;
      if (l.ok && r <= last)
        *reinterpret_cast<uint2*>(qrow + (l.n8 * 8u + (uint32_t)r * (uint32_t)N)) = to_e4m3x8(v, s);
    }
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

// 8 values of 8 columns, each times its column's 2^-e -> 8 saturated E4M3 bytes
__device__ __forceinline__ uint2 mx_codes8_cols(const float (&v)[8], const float (&s)[8]) {
  float c[8], one[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    c[j] = fminf(448.f, fmaxf(-448.f, v[j] * s[j]));
    one[j] = 1.f;
  }
  return to_e4m3x8(c, one);
}

// 8 values of one block times 2^-e -> 8 saturated E4M3 bytes
__device__ __forceinline__ uint2 mx_codes8(const float (&v)[8], int e) {
  const float s = __builtin_ldexpf(1.f, -e);  // e <= 119 for bf16 data: a normal float
  const float sv[8] = {s, s, s, s, s, s, s, s};
  return mx_codes8_cols(v, sv);
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

// w [E][H][N] -> wq [E][H][N], ws [E][N][H/32].  A wave's task is 128 columns
// by up to QB 32-row blocks; each block's 32 rows are read once (8 per lane in
// registers), their column maxima give the exponents, the codes follow from
// the registers.  The exponent bytes of the task gather in the wave's part of
// LDS and leave as one run per column (ws is column-major), so every line of
// ws is written by whole runs rather than byte by byte from many waves.
constexpr int QB = 32;   // 32-row blocks per wave task

__global__ void __launch_bounds__(64 * QW) quant_cols_mx(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                         int64_t N, uint8_t* __restrict__ wq, uint8_t* __restrict__ ws) {
  __shared__ __align__(16) uint8_t sx[QW][QB][QG * 8];   // [wave][block][column] exponent bytes
  const int64_t n8s = N / 8, cgs = (n8s + QG - 1) / QG, hbs = H / 32, hgs = (hbs + QB - 1) / QB;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * QW + wv;
  const bool live = task < E * cgs * hgs;
  const ColTask t = col_task(live ? task : 0, cgs, hgs);
  const ColLane l = col_lane(t.cg, n8s);
  const int64_t hb0 = t.hg * QB;
  const int nb = live ? (int)min(hbs - hb0, (int64_t)QB) : 0;
  const uint32_t pitch = (uint32_t)N * 2;
  const char* wb = reinterpret_cast<const char*>(w + (t.e * H + hb0 * 32) * N);
  uint8_t* qb = wq + (t.e * H + hb0 * 32) * N;
  const uint32_t loff = l.n8 * 16u + (uint32_t)(l.rs * 8) * pitch;
  const uint32_t qoff = l.n8 * 8u + (uint32_t)(l.rs * 8) * (uint32_t)N;
  for (int b = 0; b < nb; ++b) {
    const char* row = wb + (int64_t)b * 32 * pitch;
    uint8_t* qrow = qb + (int64_t)b * 32 * N;
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = load16(row, loff + (uint32_t)i * pitch);
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    rows_absmax(raw, m);
    wave_colmax(m);
    int ex[8];
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ex[j] = mx_exp(m[j]);
      sc[j] = __builtin_ldexpf(1.f, -ex[j]);   // e <= 119 for bf16 data: a normal float
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      unpack8(raw[i], v);
      if (l.ok) *reinterpret_cast<uint2*>(qrow + (qoff + (uint32_t)i * (uint32_t)N)) = mx_codes8_cols(v, sc);
    }
    if (l.rs == 0) {
      uint2 pk;
      pk.x = (uint32_t)(ex[0] + 127) | (uint32_t)(ex[1] + 127) << 8 | (uint32_t)(ex[2] + 127) << 16 |
             (uint32_t)(ex[3] + 127) << 24;
      pk.y = (uint32_t)(ex[4] + 127) | (uint32_t)(ex[5] + 127) << 8 | (uint32_t)(ex[6] + 127) << 16 |
             (uint32_t)(ex[7] + 127) << 24;
      *reinterpret_cast<uint2*>(&sx[wv][b][l.c * 8]) = pk;
    }
  }
  __syncthreads();   // every wave of the block reaches this once
  if (!live) return;
  // the task's exponents: column n = cg * 128 + col, bytes [hb0, hb0 + nb) of its run
  const int ncol = (int)min((int64_t)QG * 8, N - t.cg * QG * 8);
  uint8_t* sbase = ws + (t.e * N + t.cg * QG * 8) * hbs + hb0;
  const uint32_t sp = (uint32_t)hbs;
  if (hbs % 4 == 0 && ((uintptr_t)ws & 3) == 0) {   // then hb0 and nb are multiples of 4: whole dwords
    const int nq = nb / 4;
    for (int k = lane; k < ncol * nq; k += 64) {
      const int col = k / nq, q = k - col * nq;
      const uint32_t d = (uint32_t)sx[wv][4 * q][col] | (uint32_t)sx[wv][4 * q + 1][col] << 8 |
                         (uint32_t)sx[wv][4 * q + 2][col] << 16 | (uint32_t)sx[wv][4 * q + 3][col] << 24;
      *reinterpret_cast<uint32_t*>(sbase + ((uint32_t)col * sp + 4u * q)) = d;
    }
  } else {
    for (int k = lane; k < ncol * nb; k += 64) {
      const int col = k / nb, b = k - col * nb;
      sbase[(uint32_t)col * sp + (uint32_t)b] = sx[wv][b][col];
    }
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
  const int64_t tasks = E * ((N / 8 + QG - 1) / QG) * ((H / 32 + QB - 1) / QB);
  if (tasks <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_cols_mx, dim3((unsigned)((tasks + QW - 1) / QW)), dim3(64 * QW), 0, stream, w, E, H, N,
                     wq, ws);
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
  const int64_t tasks = quant_cols_chunks(H) * E * ((N / 8 + QG - 1) / QG);
  const unsigned blocks = (unsigned)((tasks + QW - 1) / QW);
  hipLaunchKernelGGL(quant_cols_max, dim3(blocks), dim3(64 * QW), 0, stream, w, E, H, N, pmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_cols_apply, dim3(blocks), dim3(64 * QW), 0, stream, w, E, H, N, pmax, wq, dsw);
  return hipGetLastError();
}

}  // namespace hmm

// ---------------------------------------------------------------- per group
// MoeDistributeDispatchV2 case 4 (per-group dynamic quantisation): case 3's
// rule over groups of QGROUP = 128 consecutive hidden elements of a token row,
// and, for the weight, over blocks of 128 rows of one column.

namespace hmm {

constexpr int QGROUP = 128;

// xq[t] = e4m3(x[t] * scale_g), dsx[t][g] = 1 / scale_g.  16 consecutive lanes
// hold one group (8 elements each); H is a multiple of 128, so H / 8 is a
// multiple of 16 and a group's lanes are active together.
__global__ void __launch_bounds__(QT) quant_rows_group(const uint16_t* __restrict__ x, int64_t chunks, int64_t H,
                                                       uint8_t* __restrict__ xq, float* __restrict__ dsx) {
  for (int64_t c = (int64_t)blockIdx.x * QT + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * QT) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4*>(x + c * 8), v);
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    const float sx = scale_of(m);
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = sx;
    *reinterpret_cast<uint2*>(xq + c * 8) = to_e4m3x8(v, s);
    if ((c & 15) == 0) dsx[c >> 4] = 1.f / sx;  // chunk c of the flat [T][H] array starts group c / 16
  }
}

// wq[e][k][n] = e4m3(w[e][k][n] * scale), dsw[e][k / 128][n] = 1 / scale, the
// scale from the column's 128-row block.  A wave takes a 128-column by 128-row
// tile (the column quantisers' wave tile, four 32-row slabs): the column maxima
// of the slabs, met in two lane shuffles, then the slabs again for the codes
// (the second read finds the tile in L2).
__global__ void __launch_bounds__(64 * QW) quant_cols_group(const uint16_t* __restrict__ w, int64_t E, int64_t H,
                                                            int64_t N, uint8_t* __restrict__ wq,
                                                            float* __restrict__ dsw) {
  const int64_t n8s = N / 8, cgs = (n8s + QG - 1) / QG, hb = H / QGROUP;
  const int64_t task = wave_task();
  if (task >= E * cgs * hb) return;
  const ColTask t = col_task(task, cgs, hb);
  const ColLane l = col_lane(t.cg, n8s);
  const uint32_t pitch = (uint32_t)N * 2;
  const char* wb = reinterpret_cast<const char*>(w + (t.e * H + t.hg * QGROUP) * N);
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sl = 0; sl < QGROUP / 32; ++sl) {
    const char* row = wb + (int64_t)sl * 32 * pitch;
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = load16(row, l.n8 * 16u + (uint32_t)(l.rs * 8 + i) * pitch);
    rows_absmax(raw, m);
  }
  wave_colmax(m);
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = scale_of(m[j]);
  if (l.rs == 0 && l.ok) {
    float4* out = reinterpret_cast<float4*>(dsw + (t.e * hb + t.hg) * N + l.n8 * 8);
    out[0] = make_float4(1.f / s[0], 1.f / s[1], 1.f / s[2], 1.f / s[3]);
    out[1] = make_float4(1.f / s[4], 1.f / s[5], 1.f / s[6], 1.f / s[7]);
  }
  uint8_t* qb = wq + (t.e * H + t.hg * QGROUP) * N;
#pragma unroll
  for (int sl = 0; sl < QGROUP / 32; ++sl) {
    const char* row = wb + (int64_t)sl * 32 * pitch;
    uint8_t* qrow = qb + (int64_t)sl * 32 * N;
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = load16(row, l.n8 * 16u + (uint32_t)(l.rs * 8 + i) * pitch);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      unpack8(raw[i], v);
      if (l.ok)
        *reinterpret_cast<uint2*>(qrow + (l.n8 * 8u + (uint32_t)(l.rs * 8 + i) * (uint32_t)N)) = to_e4m3x8(v, s);
    }
  }
}

hipError_t launch_quant_rows_group(const uint16_t* x, int64_t T, int64_t H, uint8_t* xq, float* dsx,
                                   hipStream_t stream) {
  const int64_t chunks = T * (H / 8);
  if (chunks <= 0) return hipSuccess;
  int64_t blocks = (chunks + QT - 1) / QT;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  hipLaunchKernelGGL(quant_rows_group, dim3((unsigned)blocks), dim3(QT), 0, stream, x, chunks, H, xq, dsx);
  return hipGetLastError();
}

hipError_t launch_quant_cols_group(const uint16_t* w, int64_t E, int64_t H, int64_t N, uint8_t* wq, float* dsw,
                                   hipStream_t stream) {
  const int64_t tasks = E * ((N / 8 + QG - 1) / QG) * (H / QGROUP);
  if (tasks <= 0) return hipSuccess;
  if ((tasks + QW - 1) / QW > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_cols_group, dim3((unsigned)((tasks + QW - 1) / QW)), dim3(64 * QW), 0, stream, w, E, H, N,
                     wq, dsw);
  return hipGetLastError();
}

}  // namespace hmm
