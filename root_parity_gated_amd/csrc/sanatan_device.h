// sanatan_device.h -- device helpers shared by the gfx950 kernels of libsanatan.
//
// Feature map of one content component u at position t, content dim a (SANATAN reading notes,
// §2.2 angle map / root label / rotation; §2.3 six-channel block), evaluated in revolutions so
// that the hardware sine/cosine (which take x and return sin(2 pi x)) need no range reduction:
//   x   = u / (2 (1 + |u|))            = theta / (2 pi),       theta in (-pi, pi)
//   rho = frac(t lambda_a / (2 pi))     (position phase, reduced in fp64)
//   cos theta_rot = cos_rev(x + rho),   sin theta_rot = sin_rev(x + rho)
//   cos(theta+omega) - sin(theta+omega) = sqrt2 cos(theta + omega + pi/4) = sqrt2 cos_rev(x + om4),
//       om4 = frac((omega + pi/4) / (2 pi))
//   r = tanh(gamma sqrt2 g) = 1 - 2 / (exp2(kr g) + 1),  kr = 2 sqrt2 gamma log2(e)
// The root label uses the UNROTATED angle, as the notes require.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sanatan {

constexpr int kD = 64;          // content dims per head (the only supported value)
constexpr int kDV = 64;         // value dims per head
constexpr int kF = 6 * kD;      // feature dims (6 channels)
constexpr int kStateFloats = kF * kDV + kF;  // S [6d][d_v] then z [6d]
constexpr int kCompactRows = 5 * kD + 1;     // compact state: the d equal channel-0 rows kept once
constexpr int kFourRows = 3 * kD + 1;        // four-channel kernel's state: shared channel 0, then r, r cos, r sin

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ hardware transcendentals
__device__ __forceinline__ float sin_rev(float x) { return __builtin_amdgcn_sinf(x); }
__device__ __forceinline__ float cos_rev(float x) { return __builtin_amdgcn_cosf(x); }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// Position phase in revolutions, frac(t * lambda_a / (2 pi)), lambda_a = base^(-a/d); fp64
// so that large positions keep full fp32 accuracy of the reduced phase.  phase_step gives
// lambda_a / (2 pi) (one fp64 exp2, worth hoisting out of loops over t).
__device__ __forceinline__ double phase_step(int a, double log2_base) {
  return exp2(-(double)a * (1.0 / kD) * log2_base) * 0.15915494309189533576888376;
}
// The product t * step is split into its rounded value p and its exact rounding error e (an fma two-product;
// t converts exactly for |t| < 2^53), and each part is reduced on its own, so the phase keeps about 2^-53
// revolutions of accuracy at any such position instead of losing the product's high bits.
__device__ __forceinline__ float phase_at(int64_t t, double step) {
#pragma clang fp contract(off)  // p must be the rounded product, or e would count the error twice
  const double tt = (double)t;
  const double p = tt * step;
  const double e = fma(tt, step, -p);
  const double x = (p - floor(p)) + e;
  return (float)(x - floor(x));
}
__device__ __forceinline__ float phase_rev(int64_t t, int a, double log2_base) {
  return phase_at(t, phase_step(a, log2_base));
}

// Root anchor in revolutions, frac((omega + pi/4) / (2 pi)), in fp64.
__device__ __forceinline__ float anchor_rev(float omega) {
  const double x = ((double)omega + 0.78539816339744830961566085) * 0.15915494309189533576888376;
  return (float)(x - floor(x));
}

// One component -> (cos theta_rot, sin theta_rot, r).
__device__ __forceinline__ void featurize1(float u, float rho, float om4, float kr, float& cr, float& sr,
                                           float& r) {
  const float x = u * rcp_hw(fmaf(fabsf(u), 2.0f, 2.0f));
  const float y = x + rho;
  cr = cos_rev(y);
  sr = sin_rev(y);
  const float g = cos_rev(x + om4);
  const float e = exp2_hw(kr * g);
  r = fmaf(-2.0f, rcp_hw(e + 1.0f), 1.0f);
}

// ------------------------------------------------------------------ element types
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// 4 consecutive elements -> float[4]
__device__ __forceinline__ void load4(const float* p, float (&o)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const __bf16* p, float (&o)[4]) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}

// ------------------------------------------------------------------ MFMA 16x16 tiles
// Lane l of a wave: row/col index l % 16, quarter l / 16.  Operand fragments hold 8 K-values per
// lane; the bf16 form feeds one v_mfma_f32_16x16x32_bf16 (K = 8 * quarter + slot), the fp32 form
// feeds eight v_mfma_f32_16x16x4_f32 (MFMA number = slot, K = quarter): the same (quarter, slot)
// -> K-index assignment either way.  Accumulator: lane holds D[4 * quarter + i][l % 16], i < 4.
template <typename T> struct FragT;
template <> struct FragT<__bf16> { typedef bf16x8 type; };
template <> struct FragT<float> { typedef f32x8 type; };

__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; i++) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
}

// Build a fragment from two 4-vectors (slots 0..3, 4..7).
template <typename T> __device__ __forceinline__ typename FragT<T>::type pack8(const float (&lo)[4], const float (&hi)[4]);
template <> __device__ __forceinline__ bf16x8 pack8<__bf16>(const float (&lo)[4], const float (&hi)[4]) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 4; i++) { f[i] = (__bf16)lo[i]; f[4 + i] = (__bf16)hi[i]; }
  return f;
}
template <> __device__ __forceinline__ f32x8 pack8<float>(const float (&lo)[4], const float (&hi)[4]) {
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; i++) { f[i] = lo[i]; f[4 + i] = hi[i]; }
  return f;
}
template <typename T> __device__ __forceinline__ typename FragT<T>::type pack8v(const f32x4& lo, const f32x4& hi) {
  float a[4] = {lo[0], lo[1], lo[2], lo[3]}, b[4] = {hi[0], hi[1], hi[2], hi[3]};
  return pack8<T>(a, b);
}
template <typename T> __device__ __forceinline__ typename FragT<T>::type zero_frag() {
  typename FragT<T>::type f;
#pragma unroll
  for (int i = 0; i < 8; i++) f[i] = (T)0.0f;
  return f;
}

}  // namespace sanatan
