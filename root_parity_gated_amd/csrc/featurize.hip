// featurize.hip -- position phase table and the standalone feature-map kernel.
//
// Feature map: SANATAN reading notes §2.2 (angle map, root label from the unrotated angle,
// temporal rotation) and §2.3 (six-channel block), written channel-major: row c*d + a.
// Both kernels are HBM-bound; one thread per (token, content dim) keeps every load and every
// channel store a contiguous 64-element run.
#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

// rho[t][a] = phase of position pos0 + t; a block covers 16 positions, each thread one dim and 4 of them.
__global__ __launch_bounds__(256) void phase_table_kernel(float* __restrict__ rho, int T, int64_t pos0,
                                                          double log2_base) {
  const int a = threadIdx.x & 63;
  const double step = phase_step(a, log2_base);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int64_t t = (int64_t)blockIdx.x * 16 + 4 * j + (threadIdx.x >> 6);
    if (t < T) rho[t * kD + a] = phase_at(pos0 + t, step);
  }
}

hipError_t launch_phase_table(float* rho, int T, int64_t pos0, double log2_base, hipStream_t stream) {
  const unsigned blocks = (unsigned)((T + 15) / 16);
  hipLaunchKernelGGL(phase_table_kernel, dim3(blocks), dim3(256), 0, stream, rho, T, pos0, log2_base);
  return hipGetLastError();
}

// 8 consecutive values of one token, in and out
__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const __bf16* p, float (&o)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; i++) o[i] = (float)v[i];
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(__bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = (__bf16)x[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}

// Phi of every token of one sequence tile: a thread owns dims 8 j .. 8 j + 7 (j = thread % 8) of
// kFeatRows tokens 32 apart, so its phase steps and anchors are computed once, and each channel of a
// token leaves as one 16- or 32-byte store per thread (8 threads cover a channel's 64 dims).
constexpr int kFeatRows = 4;
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void featurize_kernel(const TIn* __restrict__ u, TOut* __restrict__ phi, int H,
                                                        int T, int64_t pos0, const float* __restrict__ omega,
                                                        int nph, double log2_base, float kr, int ntiles) {
  const int bh = (int)(blockIdx.x / ntiles), tile = (int)(blockIdx.x % ntiles), j = threadIdx.x & 7, a0 = 8 * j;
  const int h = bh % H;
  double step[8];
  float om4[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    step[i] = phase_step(a0 + i, log2_base);
    om4[i] = anchor_rev(omega[(size_t)(h % nph) * kD + a0 + i]);
  }
  const TIn* ub = u + (size_t)bh * T * kD;
  TOut* pb = phi + (size_t)bh * T * kF;
#pragma unroll
  for (int r = 0; r < kFeatRows; r++) {
    const int t = tile * (32 * kFeatRows) + 32 * r + (threadIdx.x >> 3);
    if (t >= T) break;
    float x[8];
    load8(ub + (size_t)t * kD + a0, x);
    float ch[6][8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float cr, sr, rr;
      featurize1(x[i], phase_at(pos0 + t, step[i]), om4[i], kr, cr, sr, rr);
      ch[0][i] = 1.0f;
      ch[1][i] = cr;
      ch[2][i] = sr;
      ch[3][i] = rr;
      ch[4][i] = rr * cr;
      ch[5][i] = rr * sr;
    }
    TOut* o = pb + (size_t)t * kF + a0;
#pragma unroll
    for (int c = 0; c < 6; c++) store8(o + c * kD, ch[c]);
  }
}

template <typename TIn, typename TOut>
static void launch_feat_t(const void* u, int B, int H, int T, int64_t pos0, const MethodConsts& mc, void* phi,
                          hipStream_t stream) {
  const int ntiles = (T + 32 * kFeatRows - 1) / (32 * kFeatRows);
  const unsigned blocks = (unsigned)((long long)ntiles * B * H);
  hipLaunchKernelGGL((featurize_kernel<TIn, TOut>), dim3(blocks), dim3(256), 0, stream, static_cast<const TIn*>(u),
                     static_cast<TOut*>(phi), H, T, pos0, mc.omega, mc.nph, mc.log2_base, mc.kr, ntiles);
}

hipError_t launch_featurize(const void* u, sanatan_dtype in_t, int B, int H, int T, int64_t pos0,
                            const MethodConsts& mc, void* phi, sanatan_dtype out_t, hipStream_t stream) {
  if (in_t == SANATAN_F32 && out_t == SANATAN_F32) launch_feat_t<float, float>(u, B, H, T, pos0, mc, phi, stream);
  else if (in_t == SANATAN_F32) launch_feat_t<float, __bf16>(u, B, H, T, pos0, mc, phi, stream);
  else if (out_t == SANATAN_F32) launch_feat_t<__bf16, float>(u, B, H, T, pos0, mc, phi, stream);
  else launch_feat_t<__bf16, __bf16>(u, B, H, T, pos0, mc, phi, stream);
  return hipGetLastError();
}

}  // namespace sanatan
