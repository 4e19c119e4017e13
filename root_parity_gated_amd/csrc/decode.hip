// decode.hip -- one token of the p = 1 constant-state recurrence for N head-states.
//
// SANATAN reading notes §2.7: S_t = S_{t-1} + Phi(k_t) v_t^T, z_t = z_{t-1} + Phi(k_t),
// o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c eps) -- the state is written before it is read.
//
// HBM-bound: 2 x 99,840 B of state move per head-state and token, against 0.5 flop/byte.
// One 256-thread workgroup owns one head-state and streams its S once: each thread holds 24
// float4 row pieces (rows rg + 16m, columns 4cg..4cg+3), so a wave reads 4 KB-contiguous
// slabs; the rank-1 update and the readout share one pass, and the readout uses the updated S.
#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

__global__ __launch_bounds__(256) void decode_step_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, int64_t pos,
                                                          const float* __restrict__ omega, int nph,
                                                          double log2_base, float kr, float ceps,
                                                          float* __restrict__ S, float* __restrict__ z,
                                                          float* __restrict__ out) {
  __shared__ float fk[kF];
  __shared__ float fq[kF];
  __shared__ float vs[kDV];
  __shared__ float red[16][kDV + 4];
  __shared__ float dred[4];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  float* __restrict__ Si = S + (size_t)i * kF * kDV;
  float* __restrict__ zi = z + (size_t)i * kF;

  // Issue the state loads first so their latency overlaps the feature computation.
  const int cg = tid & 15;  // column group: columns 4cg .. 4cg+3
  const int rg = tid >> 4;  // row group: rows rg + 16m, m < 24
  float4 rows[kF / 16];
#pragma unroll
  for (int m = 0; m < kF / 16; m++) rows[m] = *reinterpret_cast<const float4*>(&Si[(rg + 16 * m) * kDV + 4 * cg]);
  float zr[2];
  zr[0] = zi[tid];
  zr[1] = (tid + 256 < kF) ? zi[tid + 256] : 0.0f;

  if (tid < 2 * kD) {
    const int a = tid & (kD - 1);
    const float u = (tid < kD) ? k[(size_t)i * kD + a] : q[(size_t)i * kD + a];
    const float om4 = anchor_rev(omega[(size_t)(i % nph) * kD + a]);
    const float rho = phase_rev(pos, a, log2_base);
    float cr, sr, r;
    featurize1(u, rho, om4, kr, cr, sr, r);
    float* dst = (tid < kD) ? fk : fq;
    dst[0 * kD + a] = 1.0f;
    dst[1 * kD + a] = cr;
    dst[2 * kD + a] = sr;
    dst[3 * kD + a] = r;
    dst[4 * kD + a] = r * cr;
    dst[5 * kD + a] = r * sr;
  } else if (tid < 2 * kD + kDV) {
    vs[tid - 2 * kD] = v[(size_t)i * kDV + (tid - 2 * kD)];
  }
  __syncthreads();

  const float4 vv = *reinterpret_cast<const float4*>(&vs[4 * cg]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < kF / 16; m++) {
    const int f = rg + 16 * m;
    const float a = fk[f], b = fq[f];
    float4 s = rows[m];
    s.x = fmaf(a, vv.x, s.x);
    s.y = fmaf(a, vv.y, s.y);
    s.z = fmaf(a, vv.z, s.z);
    s.w = fmaf(a, vv.w, s.w);
    *reinterpret_cast<float4*>(&Si[f * kDV + 4 * cg]) = s;
    acc.x = fmaf(b, s.x, acc.x);
    acc.y = fmaf(b, s.y, acc.y);
    acc.z = fmaf(b, s.z, acc.z);
    acc.w = fmaf(b, s.w, acc.w);
  }
  // z update and the denominator partial
  float dpart;
  {
    const float z0 = zr[0] + fk[tid];
    zi[tid] = z0;
    dpart = fq[tid] * z0;
    if (tid + 256 < kF) {
      const float z1 = zr[1] + fk[tid + 256];
      zi[tid + 256] = z1;
      dpart = fmaf(fq[tid + 256], z1, dpart);
    }
  }
  red[rg][4 * cg + 0] = acc.x;
  red[rg][4 * cg + 1] = acc.y;
  red[rg][4 * cg + 2] = acc.z;
  red[rg][4 * cg + 3] = acc.w;
  // wave-level reduction of the denominator partials (fixed order: deterministic)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off);
  if ((tid & 63) == 0) dred[tid >> 6] = dpart;
  __syncthreads();
  if (tid < kDV) {
    float num = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; g++) num += red[g][tid];
    const float den = ((dred[0] + dred[1]) + dred[2]) + dred[3];
    out[(size_t)i * kDV + tid] = num / (den + ceps);
  }
}

hipError_t launch_decode_step(const float* q, const float* k, const float* v, int N, int64_t pos,
                              const MethodConsts& mc, float* S, float* z, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(decode_step_kernel, dim3(N), dim3(256), 0, stream, q, k, v, pos, mc.omega, mc.nph,
                     mc.log2_base, mc.kr, mc.ceps, S, z, out);
  return hipGetLastError();
}

}  // namespace sanatan
