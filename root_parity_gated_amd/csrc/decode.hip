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
//
// Compact state.  Channel 0 of both feature maps is the constant 1 (§2.3), so the d rows of S that
// channel 0 owns all receive the same v_t and stay equal, and so do their d entries of z.  The compact
// layout keeps them once: row 0 is the shared channel-0 row, rows 1 .. 5d are channels 1..5 (full rows
// d .. 6d-1).  A token adds 1 x v to row 0, and the readout weighs row 0 by d (the d equal rows, each read
// with phi(q) = 1).  (5d+1) x (d_v+1) floats instead of 6d x (d_v+1): 17 % fewer bytes per token.
#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

namespace {
constexpr int kDecThreads = 512;
constexpr int kDecRows = kDecThreads / 16;  // row groups: 16 threads cover the 64 columns of a row
typedef float f32x4v __attribute__((ext_vector_type(4)));
}  // namespace

// Layout: 0 full six-channel state (6d rows), 1 compact six-channel (5d+1), 2 the unclipped four-channel kernel's
// state ([N] §2.5: features [1, r, r cos, r sin]; kept compact too, 3d+1 rows: the shared channel-0 row, then
// r, r cos, r sin).
// Layout 3: the spectral-harmonic map with NH harmonics, full state of (2 + 4 NH) d rows (channel 0 = 1; 2n-1, 2n =
// cos, sin of n theta_rot; 2 NH + 1 = r; 2 NH + 2n, 2 NH + 2n + 1 = r cos, r sin of n theta_rot).
template <bool NT, int Layout, int NH = 1>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, int64_t pos,
    const int64_t* __restrict__ posv, const float* __restrict__ omega, int nph, double log2_base, float kr,
    float ceps, float* __restrict__ S, float* __restrict__ z, float* __restrict__ out) {
  constexpr bool Compact = Layout == 1 || Layout == 2;
  constexpr int R = Layout == 0 ? kF : Layout == 1 ? kCompactRows : Layout == 2 ? kFourRows : (2 + 4 * NH) * kD;
  constexpr int MR = (R + kDecRows - 1) / kDecRows;   // row pieces per thread
  __shared__ float fk[R];
  __shared__ float fq[R];
  __shared__ float vs[kDV];
  __shared__ float red[kDecRows][kDV + 4];
  __shared__ float dred[kDecThreads / 64];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  float* __restrict__ Si = S + (size_t)i * R * kDV;
  float* __restrict__ zi = z + (size_t)i * R;

  // Issue the state loads first so their latency overlaps the feature computation.
  const int cg = tid & 15;  // column group: columns 4cg .. 4cg+3
  const int rg = tid >> 4;  // row group: rows rg + kDecRows m
  f32x4v rows[MR];
#pragma unroll
  for (int m = 0; m < MR; m++) {
    const int f = rg + kDecRows * m;
    const f32x4v* src = reinterpret_cast<const f32x4v*>(&Si[f * kDV + 4 * cg]);
    if (f < R) rows[m] = NT ? __builtin_nontemporal_load(src) : *src;
  }
  constexpr int ZR = (R + kDecThreads - 1) / kDecThreads;  // z rows per thread (two for the 640-row state)
  float zr[ZR];
#pragma unroll
  for (int m = 0; m < ZR; m++) zr[m] = tid + kDecThreads * m < R ? zi[tid + kDecThreads * m] : 0.0f;

  if (tid < 2 * kD) {
    const int a = tid & (kD - 1);
    const bool is_k = tid < kD;
    const float u = is_k ? k[(size_t)i * kD + a] : q[(size_t)i * kD + a];
    const float om4 = anchor_rev(omega[(size_t)(i % nph) * kD + a]);
    const float rho = phase_rev(posv ? posv[i] : pos, a, log2_base);
    float cr, sr, r;
    featurize1(u, rho, om4, kr, cr, sr, r);
    float* dst = is_k ? fk : fq;
    if constexpr (Layout == 3) {
      const float y = u * rcp_hw(fmaf(fabsf(u), 2.0f, 2.0f)) + rho;  // rotated angle in revolutions
      dst[a] = 1.0f;
      dst[(2 * NH + 1) * kD + a] = r;
#pragma unroll
      for (int n = 1; n <= NH; n++) {
        const float c = n == 1 ? cr : cos_rev((float)n * y), s = n == 1 ? sr : sin_rev((float)n * y);
        dst[(2 * n - 1) * kD + a] = c;
        dst[(2 * n) * kD + a] = s;
        dst[(2 * NH + 2 * n) * kD + a] = r * c;
        dst[(2 * NH + 2 * n + 1) * kD + a] = r * s;
      }
    }
    // channel c >= 1 of dim a: row c d + a, or 1 + (c - 1) d + a in the compact layout, or 1 + (c - 3) d + a
    // for the four-channel channels c = 3..5
    constexpr int sh = Layout == 0 ? 0 : Layout == 1 ? 1 - kD : 1 - 3 * kD;
    if constexpr (Layout != 3) {
      if constexpr (Compact) {
        // the shared channel-0 row: a key adds 1 x v to it, a query reads it once for each of its d rows
        if (a == 0) dst[0] = is_k ? 1.0f : (float)kD;
      } else {
        dst[a] = 1.0f;
      }
      if constexpr (Layout != 2) {
        dst[sh + 1 * kD + a] = cr;
        dst[sh + 2 * kD + a] = sr;
      }
      dst[sh + 3 * kD + a] = r;
      dst[sh + 4 * kD + a] = r * cr;
      dst[sh + 5 * kD + a] = r * sr;
    }
  } else if (tid < 2 * kD + kDV) {
    vs[tid - 2 * kD] = v[(size_t)i * kDV + (tid - 2 * kD)];
  }
  __syncthreads();

  const f32x4v vv = *reinterpret_cast<const f32x4v*>(&vs[4 * cg]);
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < MR; m++) {
    const int f = rg + kDecRows * m;
    if (f < R) {
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
  }
  // z update and the denominator partial
  float dpart = 0.0f;
#pragma unroll
  for (int m = 0; m < ZR; m++) {
    const int f = tid + kDecThreads * m;
    if (f < R) {
      const float z0 = zr[m] + fk[f];
      zi[f] = z0;
      dpart = fmaf(fq[f], z0, dpart);
    }
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

// Full <-> compact state, one workgroup per head-state: row copies in float4 pieces.
template <bool ToCompact>
__global__ __launch_bounds__(256) void state_convert_kernel(const float* __restrict__ src_S,
                                                            const float* __restrict__ src_z, float* __restrict__ dst_S,
                                                            float* __restrict__ dst_z) {
  const int i = blockIdx.x, tid = threadIdx.x;
  const size_t full = (size_t)i * kF, compact = (size_t)i * kCompactRows;
  constexpr int P = kDV / 4;  // float4 pieces per row
  // destination rows: compact 0 .. 5d (from full 0, d .. 6d-1), or full 0 .. 6d-1 (from compact 0 or f - d + 1)
  constexpr int rows = ToCompact ? kCompactRows : kF;
  for (int e = tid; e < rows * P; e += 256) {
    const int row = e / P, c = e % P;
    const int srow = ToCompact ? (row == 0 ? 0 : row + kD - 1) : (row < kD ? 0 : row - kD + 1);
    const size_t sbase = ToCompact ? full : compact, dbase = ToCompact ? compact : full;
    reinterpret_cast<f32x4v*>(dst_S + (dbase + row) * kDV)[c] =
        reinterpret_cast<const f32x4v*>(src_S + (sbase + srow) * kDV)[c];
  }
  for (int row = tid; row < rows; row += 256) {
    const int srow = ToCompact ? (row == 0 ? 0 : row + kD - 1) : (row < kD ? 0 : row - kD + 1);
    dst_z[(ToCompact ? compact : full) + row] = src_z[(ToCompact ? full : compact) + srow];
  }
}

hipError_t launch_decode_step(const float* q, const float* k, const float* v, int N, int64_t pos,
                              const int64_t* posv, int layout, const MethodConsts& mc, float* S, float* z,
                              float* out, hipStream_t stream) {
  // states above 128 MB (half of the 256 MB last-level cache) are streamed
  const int rows = layout == 0 ? kF : layout == 1 ? kCompactRows : kFourRows;
  const size_t floats = (size_t)rows * (kDV + 1);
  const bool stream_state = (size_t)N * floats * sizeof(float) > ((size_t)128 << 20);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(N), dim3(kDecThreads), 0, stream, q, k, v, pos, posv, mc.omega, mc.nph,
                       mc.log2_base, mc.kr, mc.ceps, S, z, out);
  };
  if (layout == 2) {
    if (stream_state) go(decode_step_kernel<true, 2>); else go(decode_step_kernel<false, 2>);
  } else if (layout == 1) {
    if (stream_state) go(decode_step_kernel<true, 1>); else go(decode_step_kernel<false, 1>);
  } else {
    if (stream_state) go(decode_step_kernel<true, 0>); else go(decode_step_kernel<false, 0>);
  }
  return hipGetLastError();
}

// the spectral-harmonic map with nh = 2 harmonics (nh = 1 is layout 0)
hipError_t launch_decode_step_harmonics(const float* q, const float* k, const float* v, int N, int64_t pos,
                                        const int64_t* posv, int nh, const MethodConsts& mc, float* S, float* z,
                                        float* out, hipStream_t stream) {
  const size_t floats = (size_t)(2 + 4 * nh) * kD * (kDV + 1);
  const bool stream_state = (size_t)N * floats * sizeof(float) > ((size_t)128 << 20);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(N), dim3(kDecThreads), 0, stream, q, k, v, pos, posv, mc.omega, mc.nph,
                       mc.log2_base, mc.kr, mc.ceps, S, z, out);
  };
  if (nh == 1) return launch_decode_step(q, k, v, N, pos, posv, 0, mc, S, z, out, stream);
  if (nh == 2) {
    if (stream_state) go(decode_step_kernel<true, 3, 2>); else go(decode_step_kernel<false, 3, 2>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_state_convert(const float* S, const float* z, int N, bool to_compact, float* dS, float* dz,
                                hipStream_t stream) {
  if (to_compact)
    hipLaunchKernelGGL(state_convert_kernel<true>, dim3(N), dim3(256), 0, stream, S, z, dS, dz);
  else
    hipLaunchKernelGGL(state_convert_kernel<false>, dim3(N), dim3(256), 0, stream, S, z, dS, dz);
  return hipGetLastError();
}

}  // namespace sanatan
