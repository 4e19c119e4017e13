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
// gets its column col at tokens tok0 + 8 (i / 4) + 4 h + i % 4, each token clamped to tmax.
__device__ __forceinline__ f32x8 gtok_frag(const float* base, int pitch, int tok0, int col, int l, int tmax) {
  const int tb = tok0 + 4 * (l >> 5);
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

// The feature map's vector-Jacobian product for one component u (one token, one dim): from the gradients
// g1 .. g5 of its features cos y, sin y, r, r cos y, r sin y (y the rotated angle; the constant feature has none),
// du = dtheta pi / (1 + |u|)^2 with
//   dtheta = r' (g3 + g4 cos y + g5 sin y) - sin y (g1 + r g4) + cos y (g2 + r g5),   r' = dr/dtheta = dr/domega,
// and the omega gradient r' (g3 + g4 cos y + g5 sin y).  The angle, root and rotation are recomputed with the
// same hardware operations and reduced phase as the feature map.
__device__ __forceinline__ void feature_vjp(float u, float rho, float om4, float kr, float g1, float g2, float g3,
                                            float g4, float g5, float& du, float& dom) {
  const float xr = u * rcp_hw(fmaf(fabsf(u), 2.0f, 2.0f));  // theta / (2 pi)
  const float y = xr + rho;
  const float cy = cos_rev(y), sy = sin_rev(y);
  const float gg = cos_rev(xr + om4);
  const float e = exp2_hw(kr * gg);
  const float r = fmaf(-2.0f, rcp_hw(e + 1.0f), 1.0f);
  // r = tanh(gamma sqrt2 cos(theta + omega + pi/4)); kr = 2 sqrt2 gamma log2(e), so gamma sqrt2 = kr ln2 / 2
  const float rp = -(kr * 0.34657359027997264f) * (1.0f - r * r) * sin_rev(xr + om4);
  const float gr = g3 + g4 * cy + g5 * sy;
  const float dth = rp * gr - sy * (g1 + r * g4) + cy * (g2 + r * g5);
  const float den = 1.0f + fabsf(u);
  du = dth * 3.14159265358979f * rcp_hw(den * den);
  dom = rp * gr;
}

}  // namespace sanatan
