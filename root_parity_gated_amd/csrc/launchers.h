// launchers.h -- host-side interface between the C ABI (api.hip) and the kernel files.
// All sizes have been validated by the caller; launchers only compute grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sanatan.h"

namespace sanatan {

// Method constants prepared once per call on the host.
struct MethodConsts {
  const float* omega;   // device [nph][64]
  int nph;              // omega rows
  float kr;             // 2 sqrt2 gamma log2(e)
  double log2_base;     // log2(lambda_base)
  float ceps;           // c * eps (raw-unit epsilon)
  float inv_c;          // 1 / c
  float eps;            // normalised epsilon
};

// rho[t][a] = frac((pos0 + t) lambda_a / 2pi), t < T (fp32 table, fp64 reduction)
hipError_t launch_phase_table(float* rho, int T, int64_t pos0, double log2_base, hipStream_t stream);

hipError_t launch_featurize(const void* u, sanatan_dtype in_t, int B, int H, int T, int64_t pos0,
                            const MethodConsts& mc, void* phi, sanatan_dtype out_t, hipStream_t stream);

// posv: device [N] positions, one per head-state, or nullptr for the single position pos;
// layout 0: S [N][6d][d_v], z [N][6d]; 1: compact, [N][5d+1] rows (channel-0 rows kept once); 2: the unclipped
// four-channel kernel's state, [N][3d+1] rows (shared channel 0, then r, r cos, r sin)
hipError_t launch_decode_step(const float* q, const float* k, const float* v, int N, int64_t pos,
                              const int64_t* posv, int layout, const MethodConsts& mc, float* S, float* z,
                              float* out, hipStream_t stream);
// full state (S, z) -> compact (dS, dz), or compact -> full
hipError_t launch_state_convert(const float* S, const float* z, int N, bool to_compact, float* dS, float* dz,
                                hipStream_t stream);

// Prefill plan: the flattened (sequence, chunk) list split into G equal ranges (one workgroup
// each) and the workspace layout (phase table, then boundary-state slots).
struct PrefillPlan {
  int chunk;            // tokens per chunk
  int ncs;              // chunks per sequence
  int G;                // workgroups
  long long total;      // B*H*ncs chunks
  int multi;            // some sequence spans several ranges (pass 1 needed)
  int scanned;          // so many pieces per sequence that a separate scan kernel runs
  size_t rho_bytes;     // position-phase table [T][64] fp32 (256-byte aligned)
  size_t state_bytes;   // (B*H + G - 1) boundary states of kStateFloats fp32
  size_t total_bytes;
};
// workgroups: 0 = one per compute unit, else that many (capped at the chunk count); with_state: the call
// passes an initial state (S, z)
bool prefill_plan(int B, int H, int T, int chunk, int workgroups, bool with_state, PrefillPlan* plan);
int device_cus();  // compute units of the current device (256 if it cannot be queried)
bool prefill_chunk_supported(int chunk, sanatan_dtype t);
hipError_t launch_prefill(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                          int64_t pos0, const MethodConsts& mc, float* S, float* z, void* out, void* ws,
                          const PrefillPlan& plan, hipStream_t stream, const int* lens = nullptr);

// The no-allocation prefill's workspace: a fixed device array of the library (one per GPU)
size_t noalloc_scratch_bytes();
void* noalloc_scratch();  // this device's array (address looked up once per device); null on error

size_t quadratic_ws_bytes(int B, int H, int T, sanatan_dtype t);
// four_channel: the unclipped four-channel kernel ([1, r, r cos, r sin] per dim) instead of the six-channel one
// inv_out (nullable): the saved statistics of a training step, fp32: the output rows [B][H][T][d_v], then 1 / Dn
// per query row [B][H][T] (the normaliser in the kernel's scaled units)
hipError_t launch_quadratic(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                            int p, bool four_channel, int64_t pos0, const MethodConsts& mc, void* out, void* ws,
                            hipStream_t stream, float* inv_out = nullptr);

// Materialized-feature chunked prefill: nh_or_zero = 1 or 2 spectral harmonics (state rows (2 + 4 nh) d), or 0 for the
// unclipped four-channel compact map (3d + 1 rows).  Workspace: Phi(Q), Phi(K) padded to ext_features_padded.
int ext_features_padded(int nh_or_zero);
size_t ext_prefill_ws_bytes(int B, int H, int T, sanatan_dtype t, int nh_or_zero);
hipError_t launch_ext_prefill(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                              int nh_or_zero, int64_t pos0, const MethodConsts& mc, float* S, float* z, void* out,
                              void* ws, hipStream_t stream);
hipError_t launch_decode_step_harmonics(const float* q, const float* k, const float* v, int N, int64_t pos,
                                        const int64_t* posv, int nh, const MethodConsts& mc, float* S, float* z,
                                        float* out, hipStream_t stream);

// Gradient of normalised causal power attention (p = 1 or 2) with respect to q, k, v and omega.  Workspace:
// phase table, Phi(Q), Phi(K) (element type t), per-row statistics, fp32 feature gradients, omega partials.
size_t backward_ws_bytes(int B, int H, int T, sanatan_dtype t);
// saved (nullable): the statistics saved by the forward (fp32 output rows, then 1 / Dn per row); at p = 2 they
// replace the statistics pass
hipError_t launch_backward(const void* q, const void* k, const void* v, const void* dout, sanatan_dtype t, int B,
                           int H, int T, int p, int64_t pos0, const MethodConsts& mc, void* dq, void* dk, void* dv,
                           float* domega, void* ws, hipStream_t stream, const float* saved = nullptr);

}  // namespace sanatan
