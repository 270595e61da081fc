// Helpers shared by the grouped-product kernels (bf16 and FP8): workgroup to
// XCD mapping, tile rasterisation, buffer resources.
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

}  // namespace hmm
