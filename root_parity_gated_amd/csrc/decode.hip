// decode.hip -- one token of the p = 1 constant-state recurrence for N head-states.
//
// SANATAN reading notes §2.7: S_t = S_{t-1} + Phi(k_t) v_t^T, z_t = z_{t-1} + Phi(k_t),
// o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c eps) -- the state is written before it is read.
// The token's absolute position t sets the rotation of both feature maps (§2.2); it is one position for
// all head-states, or one per head-state (sequences of a batch at different lengths).
//
// HBM-bound: 2 x 99,840 B of state move per head-state and token, against 0.5 flop/byte.
// One 512-thread workgroup owns one head-state and streams its S once: each thread holds 12
// float4 row pieces (rows rg + 32m, columns 4cg..4cg+3), so each wave touches 4 KB-contiguous
// slabs; the rank-1 update and the readout share one pass, and the readout uses the updated S.
// When the head-states together exceed what the last-level cache can keep between tokens, the
// state is streamed with non-temporal loads and stores (caching it would only evict other data);
// a smaller state (one sequence's 144 head-states: 14.4 MB) stays cache-resident between tokens.
#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

namespace {
constexpr int kDecThreads = 512;
constexpr int kDecRows = kDecThreads / 16;  // row groups: 16 threads cover the 64 columns of a row
typedef float f32x4v __attribute__((ext_vector_type(4)));
}  // namespace

template <bool NT>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, int64_t pos,
    const int64_t* __restrict__ posv, const float* __restrict__ omega, int nph, double log2_base, float kr, float ceps, float* __restrict__ S,
    float* __restrict__ z, float* __restrict__ out) {
  __shared__ float fk[kF];
  __shared__ float fq[kF];
  __shared__ float vs[kDV];
  __shared__ float red[kDecRows][kDV + 4];
  __shared__ float dred[kDecThreads / 64];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  float* __restrict__ Si = S + (size_t)i * kF * kDV;
  float* __restrict__ zi = z + (size_t)i * kF;

  // Issue the state loads first so their latency overlaps the feature computation.
  const int cg = tid & 15;  // column group: columns 4cg .. 4cg+3
  const int rg = tid >> 4;  // row group: rows rg + kDecRows m
  f32x4v rows[kF / kDecRows];
#pragma unroll
  for (int m = 0; m < kF / kDecRows; m++)
    rows[m] = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(&Si[(rg + kDecRows * m) * kDV + 4 * cg]))
                 : *reinterpret_cast<const f32x4v*>(&Si[(rg + kDecRows * m) * kDV + 4 * cg]);
  const float zr = tid < kF ? zi[tid] : 0.0f;

  if (tid < 2 * kD) {
    const int a = tid & (kD - 1);
    const float u = (tid < kD) ? k[(size_t)i * kD + a] : q[(size_t)i * kD + a];
    const float om4 = anchor_rev(omega[(size_t)(i % nph) * kD + a]);
    const float rho = phase_rev(posv ? posv[i] : pos, a, log2_base);
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

  const f32x4v vv = *reinterpret_cast<const f32x4v*>(&vs[4 * cg]);
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < kF / kDecRows; m++) {
    const int f = rg + kDecRows * m;
    const float a = fk[f], b = fq[f];
    f32x4v s = rows[m];
#pragma unroll
    for (int e = 0; e < 4; e++) s[e] = fmaf(a, vv[e], s[e]);
    if (NT)
      __builtin_nontemporal_store(s, reinterpret_cast<f32x4v*>(&Si[f * kDV + 4 * cg]));
    else
      *reinterpret_cast<f32x4v*>(&Si[f * kDV + 4 * cg]) = s;
#pragma unroll
    for (int e = 0; e < 4; e++) acc[e] = fmaf(b, s[e], acc[e]);
  }
  // z update and the denominator partial
  float dpart = 0.0f;
  if (tid < kF) {
    const float z0 = zr + fk[tid];
    zi[tid] = z0;
    dpart = fq[tid] * z0;
  }
#pragma unroll
  for (int e = 0; e < 4; e++) red[rg][4 * cg + e] = acc[e];
  // wave-level reduction of the denominator partials (fixed order: deterministic)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off);
  if ((tid & 63) == 0) dred[tid >> 6] = dpart;
  __syncthreads();
  if (tid < kDV) {
    float num = 0.0f;
#pragma unroll
    for (int g = 0; g < kDecRows; g++) num += red[g][tid];
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecThreads / 64; w++) den += dred[w];
    out[(size_t)i * kDV + tid] = num / (den + ceps);
  }
}

hipError_t launch_decode_step(const float* q, const float* k, const float* v, int N, int64_t pos,
                              const int64_t* posv, const MethodConsts& mc, float* S, float* z, float* out, hipStream_t stream) {
  // states above 128 MB (half of the 256 MB last-level cache) are streamed
  const bool stream_state = (size_t)N * kStateFloats * sizeof(float) > ((size_t)128 << 20);
  if (stream_state)
    hipLaunchKernelGGL(decode_step_kernel<true>, dim3(N), dim3(kDecThreads), 0, stream, q, k, v, pos, posv, mc.omega,
                       mc.nph, mc.log2_base, mc.kr, mc.ceps, S, z, out);
  else
    hipLaunchKernelGGL(decode_step_kernel<false>, dim3(N), dim3(kDecThreads), 0, stream, q, k, v, pos, posv, mc.omega,
                       mc.nph, mc.log2_base, mc.kr, mc.ceps, S, z, out);
  return hipGetLastError();
}

}  // namespace sanatan
