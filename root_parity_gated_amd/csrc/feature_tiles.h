// feature_tiles.h -- MFMA operand fragments read from rows of materialized feature or value tiles, shared by
// the materialized-feature prefill and the backward kernels.
#pragma once

#include "prefill_common.h"

namespace sanatan {

// 8 elements of one row, slots (h, i) <-> column base + 8 (i / 4) + 4 h + i % 4 (the accumulator row order):
// two 4-element vector loads
template <typename T>
__device__ __forceinline__ typename FragT<T>::type slot_frag(const T* row, int base, int h) {
  typename FragT<T>::type f;
  if constexpr (sizeof(T) == 2) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(row + base + 4 * h);
    const u32x2 b = *reinterpret_cast<const u32x2*>(row + base + 8 + 4 * h);
    const u32x4 w = {a[0], a[1], b[0], b[1]};
    f = __builtin_bit_cast(typename FragT<T>::type, w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(row + base + 4 * h);
    const float4 b = *reinterpret_cast<const float4*>(row + base + 8 + 4 * h);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  return f;
}

// The fp32 counterpart of lds_tokfrag read from a token-major array in global memory: lane (row = l % 32, h)
// gets column col0 + (l % 32) at tokens tok0 + 8 (i / 4) + 4 h + i % 4, each token clamped to tmax.
__device__ __forceinline__ f32x8 gtok_frag(const float* base, int pitch, int tok0, int col0, int l, int tmax) {
  const int col = col0 + (l & 31), tb = tok0 + 4 * (l >> 5);
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[i] = base[(size_t)min(tb + i, tmax) * pitch + col];
    f[4 + i] = base[(size_t)min(tb + 8 + i, tmax) * pitch + col];
  }
  return f;
}

// x - (float)rounded, packed: the part of 8 fp32 values that their bf16 rounding dropped
template <typename T>
__device__ __forceinline__ typename FragT<T>::type residual8(const float (&x)[8], const typename FragT<T>::type& rounded) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; i++) r[i] = x[i] - (float)rounded[i];
  return pack8f<T>(r);
}

}  // namespace sanatan
