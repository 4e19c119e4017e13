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

template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void featurize_kernel(const TIn* __restrict__ u, TOut* __restrict__ phi, int H,
                                                        int T, int64_t pos0, const float* __restrict__ omega,
                                                        int nph, double log2_base, float kr, int64_t n_tokens) {
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int a = threadIdx.x & 63;
  if (tok >= n_tokens) return;
  const int64_t i = tok % T;
  const int h = (int)((tok / T) % H);
  const float uv = to_f32(u[tok * kD + a]);
  const float om4 = anchor_rev(omega[(size_t)(h % nph) * kD + a]);
  const float rho = phase_rev(pos0 + i, a, log2_base);
  float cr, sr, r;
  featurize1(uv, rho, om4, kr, cr, sr, r);
  TOut* o = phi + tok * kF;
  o[0 * kD + a] = from_f32<TOut>(1.0f);
  o[1 * kD + a] = from_f32<TOut>(cr);
  o[2 * kD + a] = from_f32<TOut>(sr);
  o[3 * kD + a] = from_f32<TOut>(r);
  o[4 * kD + a] = from_f32<TOut>(r * cr);
  o[5 * kD + a] = from_f32<TOut>(r * sr);
}

template <typename TIn, typename TOut>
static void launch_feat_t(const void* u, int B, int H, int T, int64_t pos0, const MethodConsts& mc, void* phi,
                          hipStream_t stream) {
  const int64_t n_tokens = (int64_t)B * H * T;
  const unsigned blocks = (unsigned)((n_tokens + 3) / 4);
  hipLaunchKernelGGL((featurize_kernel<TIn, TOut>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const TIn*>(u), static_cast<TOut*>(phi), H, T, pos0, mc.omega, mc.nph,
                     mc.log2_base, mc.kr, n_tokens);
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
