// api.hip -- the C ABI of libsanatan.so: argument validation on the host, then launches.
// Every check happens before the first launch, so a non-OK status (other than
// SANATAN_ERR_HIP) means nothing was enqueued.
#include <math.h>

#include "launchers.h"
#include "sanatan.h"
#include "sanatan_device.h"

using namespace sanatan;

namespace {

sanatan_status check_params(const sanatan_params* p) {
  if (!p || !p->omega) return SANATAN_ERR_INVALID_ARG;
  if (p->n_param_heads < 1) return SANATAN_ERR_INVALID_ARG;
  if (!(p->gamma >= 0.0f) || !isfinite(p->gamma)) return SANATAN_ERR_INVALID_ARG;
  if (!(p->c > 0.0f) || !isfinite(p->c)) return SANATAN_ERR_INVALID_ARG;
  if (!(p->eps >= 0.0f) || !isfinite(p->eps)) return SANATAN_ERR_INVALID_ARG;
  if (!(p->lambda_base > 0.0) || !isfinite(p->lambda_base)) return SANATAN_ERR_INVALID_ARG;
  if (p->d <= 0 || p->d_v <= 0) return SANATAN_ERR_INVALID_ARG;
  if (p->d != kD || p->d_v != kDV) return SANATAN_ERR_UNSUPPORTED;
  return SANATAN_OK;
}

bool dtype_ok(sanatan_dtype t) { return t == SANATAN_F32 || t == SANATAN_BF16; }

MethodConsts consts(const sanatan_params* p) {
  MethodConsts mc;
  mc.omega = p->omega;
  mc.nph = p->n_param_heads;
  mc.kr = (float)(2.0 * 1.4142135623730950488 * (double)p->gamma * 1.4426950408889634074);
  mc.log2_base = log2(p->lambda_base);
  mc.ceps = (float)((double)p->c * (double)p->eps);
  mc.inv_c = (float)(1.0 / (double)p->c);
  mc.eps = p->eps;
  return mc;
}

// Sizes whose element counts must stay addressable with the kernels' index arithmetic.
bool sizes_ok(int B, int H, int T) {
  if (B <= 0 || H <= 0 || T <= 0) return false;
  const long long tokens = (long long)B * H * T;
  return tokens * kF < (1LL << 40);
}

sanatan_status hip_status(hipError_t e) { return e == hipSuccess ? SANATAN_OK : SANATAN_ERR_HIP; }

// Positions are converted to fp64 exactly and reduced with an exact two-product, so any |pos| < 2^53 keeps the
// phase accurate to about 2^-53 revolutions.
bool pos_ok(int64_t p) { return p > -(int64_t(1) << 53) && p < (int64_t(1) << 53); }

// Longest sequence a prefill call accepts: the per-sequence byte ranges of the buffer loads (position table
// [T][d] fp32, key and value rows) must fit the 31-bit range of a buffer descriptor.
constexpr int kMaxPrefillT = 1 << 22;
// Longest sequence of the quadratic form: its key-feature rows [T][6d] fp32 must fit the same range.
constexpr int kMaxQuadraticT = 1 << 20;

}  // namespace

extern "C" {

size_t sanatan_state_bytes(int d, int d_v) {
  if (d <= 0 || d_v <= 0) return 0;
  return ((size_t)6 * d * d_v + (size_t)6 * d) * sizeof(float);
}

const char* sanatan_status_string(sanatan_status status) {
  switch (status) {
    case SANATAN_OK: return "ok";
    case SANATAN_ERR_INVALID_ARG: return "invalid argument";
    case SANATAN_ERR_UNSUPPORTED: return "unsupported configuration";
    case SANATAN_ERR_WORKSPACE: return "workspace missing or too small";
    case SANATAN_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

sanatan_status sanatan_featurize(const void* u, sanatan_dtype in_t, int B, int H, int T, int64_t pos0,
                                 const sanatan_params* params, void* phi, sanatan_dtype out_t, hipStream_t stream) {
  if (!u || !phi || !dtype_ok(in_t) || !dtype_ok(out_t) || !sizes_ok(B, H, T)) return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  return hip_status(launch_featurize(u, in_t, B, H, T, pos0, consts(params), phi, out_t, stream));
}

size_t sanatan_prefill_workspace_bytes_partitioned(int B, int H, int T, int chunk, int workgroups,
                                                  const sanatan_params* params) {
  (void)params;
  PrefillPlan plan;
  if (!sizes_ok(B, H, T) || T > kMaxPrefillT || chunk <= 0 || !prefill_plan(B, H, T, chunk, workgroups, false, &plan))
    return 0;
  return plan.total_bytes;
}

size_t sanatan_prefill_workspace_bytes(int B, int H, int T, int chunk, const sanatan_params* params) {
  return sanatan_prefill_workspace_bytes_partitioned(B, H, T, chunk, 0, params);
}

sanatan_status sanatan_prefill_chunked_partitioned(const void* q, const void* k, const void* v, sanatan_dtype t,
                                                   int B, int H, int T, int chunk, int workgroups, int64_t pos0,
                                                   const sanatan_params* params, float* S, float* z, void* out,
                                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !dtype_ok(t) || !sizes_ok(B, H, T) || chunk <= 0 || workgroups < 0)
    return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxPrefillT) return SANATAN_ERR_UNSUPPORTED;
  if ((S == nullptr) != (z == nullptr)) return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (chunk % 16 != 0 || !prefill_chunk_supported(chunk, t)) return SANATAN_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (!prefill_plan(B, H, T, chunk, workgroups, S != nullptr, &plan)) return SANATAN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < plan.total_bytes) return SANATAN_ERR_WORKSPACE;
  return hip_status(launch_prefill(q, k, v, t, B, H, T, pos0, consts(params), S, z, out, ws, plan, stream));
}

sanatan_status sanatan_prefill_chunked(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H,
                                       int T, int chunk, int64_t pos0, const sanatan_params* params, float* S,
                                       float* z, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return sanatan_prefill_chunked_partitioned(q, k, v, t, B, H, T, chunk, 0, pos0, params, S, z, out, ws, ws_bytes,
                                             stream);
}

sanatan_status sanatan_prefill_chunked_ragged(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                              int H, int T, int chunk, const int32_t* lengths, int64_t pos0,
                                              const sanatan_params* params, float* S, float* z, void* out, void* ws,
                                              size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !lengths || !dtype_ok(t) || !sizes_ok(B, H, T) || chunk <= 0)
    return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxPrefillT) return SANATAN_ERR_UNSUPPORTED;
  if ((S == nullptr) != (z == nullptr)) return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (chunk % 16 != 0 || !prefill_chunk_supported(chunk, t)) return SANATAN_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (!prefill_plan(B, H, T, chunk, 0, S != nullptr, &plan)) return SANATAN_ERR_INVALID_ARG;
  if (!ws || ws_bytes < plan.total_bytes) return SANATAN_ERR_WORKSPACE;
  return hip_status(launch_prefill(q, k, v, t, B, H, T, pos0, consts(params), S, z, out, ws, plan, stream,
                                   reinterpret_cast<const int*>(lengths)));
}

sanatan_status sanatan_prefill_chunked_noalloc(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                               int H, int T, int chunk, int64_t pos0, const sanatan_params* params,
                                               float* S, float* z, void* out, hipStream_t stream) {
  if (!q || !k || !v || !out || !dtype_ok(t) || !sizes_ok(B, H, T) || chunk <= 0) return SANATAN_ERR_INVALID_ARG;
  if ((S == nullptr) != (z == nullptr)) return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxPrefillT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (chunk % 16 != 0 || !prefill_chunk_supported(chunk, t)) return SANATAN_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (!prefill_plan(B, H, T, chunk, 0, S != nullptr, &plan)) return SANATAN_ERR_INVALID_ARG;
  if (plan.total_bytes > noalloc_scratch_bytes()) return SANATAN_ERR_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return SANATAN_ERR_HIP;
  return hip_status(launch_prefill(q, k, v, t, B, H, T, pos0, consts(params), S, z, out, ws, plan, stream));
}

sanatan_status sanatan_decode_step(const float* q, const float* k, const float* v, int N, int64_t pos,
                                   const sanatan_params* params, float* S, float* z, float* out, hipStream_t stream) {
  if (!q || !k || !v || !S || !z || !out || N <= 0 || !pos_ok(pos)) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  return hip_status(launch_decode_step(q, k, v, N, pos, nullptr, 0, consts(params), S, z, out, stream));
}

sanatan_status sanatan_decode_step_positions(const float* q, const float* k, const float* v, int N,
                                             const int64_t* pos, const sanatan_params* params, float* S, float* z,
                                             float* out, hipStream_t stream) {
  if (!q || !k || !v || !pos || !S || !z || !out || N <= 0) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  return hip_status(launch_decode_step(q, k, v, N, 0, pos, 0, consts(params), S, z, out, stream));
}

size_t sanatan_compact_state_bytes(int d, int d_v) {
  if (d <= 0 || d_v <= 0) return 0;
  return ((size_t)5 * d + 1) * ((size_t)d_v + 1) * sizeof(float);
}

sanatan_status sanatan_state_compact(const float* S, const float* z, int N, float* Sc, float* zc,
                                     hipStream_t stream) {
  if (!S || !z || !Sc || !zc || N <= 0) return SANATAN_ERR_INVALID_ARG;
  return hip_status(launch_state_convert(S, z, N, true, Sc, zc, stream));
}

sanatan_status sanatan_state_expand(const float* Sc, const float* zc, int N, float* S, float* z,
                                    hipStream_t stream) {
  if (!Sc || !zc || !S || !z || N <= 0) return SANATAN_ERR_INVALID_ARG;
  return hip_status(launch_state_convert(Sc, zc, N, false, S, z, stream));
}

sanatan_status sanatan_decode_step_compact(const float* q, const float* k, const float* v, int N, int64_t pos,
                                           const int64_t* posv, const sanatan_params* params, float* Sc,
                                           float* zc, float* out, hipStream_t stream) {
  if (!q || !k || !v || !Sc || !zc || !out || N <= 0 || (!posv && !pos_ok(pos))) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  return hip_status(launch_decode_step(q, k, v, N, pos, posv, 1, consts(params), Sc, zc, out, stream));
}

size_t sanatan_four_channel_state_bytes(int d, int d_v) {
  if (d <= 0 || d_v <= 0) return 0;
  return ((size_t)3 * d + 1) * ((size_t)d_v + 1) * sizeof(float);
}

sanatan_status sanatan_decode_step_four_channel(const float* q, const float* k, const float* v, int N,
                                                int64_t pos, const int64_t* posv, const sanatan_params* params,
                                                float* S4, float* z4, float* out, hipStream_t stream) {
  if (!q || !k || !v || !S4 || !z4 || !out || N <= 0 || (!posv && !pos_ok(pos))) return SANATAN_ERR_INVALID_ARG;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  return hip_status(launch_decode_step(q, k, v, N, pos, posv, 2, consts(params), S4, z4, out, stream));
}

size_t sanatan_quadratic_workspace_bytes(int B, int H, int T, sanatan_dtype t, const sanatan_params* params) {
  (void)params;
  if (!sizes_ok(B, H, T) || T > kMaxQuadraticT || !dtype_ok(t)) return 0;
  return quadratic_ws_bytes(B, H, T, t);
}

sanatan_status sanatan_quadratic_ref_p2(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H,
                                        int T, int p, int64_t pos0, const sanatan_params* params, void* out, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !dtype_ok(t) || !sizes_ok(B, H, T) || (p != 1 && p != 2))
    return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxQuadraticT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (!ws || ws_bytes < quadratic_ws_bytes(B, H, T, t)) return SANATAN_ERR_WORKSPACE;
  return hip_status(launch_quadratic(q, k, v, t, B, H, T, p, false, pos0, consts(params), out, ws, stream));
}

size_t sanatan_quadratic_saved_bytes(int B, int H, int T, const sanatan_params* params) {
  (void)params;
  if (!sizes_ok(B, H, T) || T > kMaxQuadraticT) return 0;
  return (size_t)B * H * T * (kDV + 1) * sizeof(float);
}

sanatan_status sanatan_quadratic_train(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H,
                                       int T, int p, int64_t pos0, const sanatan_params* params, void* out,
                                       float* saved, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !saved || !dtype_ok(t) || !sizes_ok(B, H, T) || (p != 1 && p != 2))
    return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxQuadraticT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (!ws || ws_bytes < quadratic_ws_bytes(B, H, T, t)) return SANATAN_ERR_WORKSPACE;
  return hip_status(launch_quadratic(q, k, v, t, B, H, T, p, false, pos0, consts(params), out, ws, stream, saved));
}

sanatan_status sanatan_quadratic_four_channel(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                              int H, int T, int p, int64_t pos0, const sanatan_params* params,
                                              void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !dtype_ok(t) || !sizes_ok(B, H, T) || (p != 1 && p != 2))
    return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxQuadraticT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (!ws || ws_bytes < quadratic_ws_bytes(B, H, T, t)) return SANATAN_ERR_WORKSPACE;
  return hip_status(launch_quadratic(q, k, v, t, B, H, T, p, true, pos0, consts(params), out, ws, stream));
}

size_t sanatan_harmonics_state_bytes(int d, int d_v, int nh) {
  if (d <= 0 || d_v <= 0 || nh <= 0) return 0;
  return (size_t)(2 + 4 * nh) * d * ((size_t)d_v + 1) * sizeof(float);
}

size_t sanatan_prefill_harmonics_workspace_bytes(int B, int H, int T, sanatan_dtype t, int nh,
                                                 const sanatan_params* params) {
  (void)params;
  if (!sizes_ok(B, H, T) || T > kMaxPrefillT || !dtype_ok(t) || nh < 1 || nh > 2) return 0;
  return ext_prefill_ws_bytes(B, H, T, t, nh);
}

size_t sanatan_prefill_four_channel_workspace_bytes(int B, int H, int T, sanatan_dtype t,
                                                    const sanatan_params* params) {
  (void)params;
  if (!sizes_ok(B, H, T) || T > kMaxPrefillT || !dtype_ok(t)) return 0;
  return ext_prefill_ws_bytes(B, H, T, t, 0);
}

static sanatan_status ext_prefill(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                                  int nh_or_zero, int64_t pos0, const sanatan_params* params, float* S, float* z,
                                  void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !dtype_ok(t) || !sizes_ok(B, H, T)) return SANATAN_ERR_INVALID_ARG;
  if ((S == nullptr) != (z == nullptr)) return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxPrefillT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (!ws || ws_bytes < ext_prefill_ws_bytes(B, H, T, t, nh_or_zero)) return SANATAN_ERR_WORKSPACE;
  return hip_status(launch_ext_prefill(q, k, v, t, B, H, T, nh_or_zero, pos0, consts(params), S, z, out, ws, stream));
}

sanatan_status sanatan_prefill_harmonics(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H,
                                         int T, int nh, int64_t pos0, const sanatan_params* params, float* S, float* z,
                                         void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (nh < 1) return SANATAN_ERR_INVALID_ARG;
  if (nh > 2) return SANATAN_ERR_UNSUPPORTED;
  return ext_prefill(q, k, v, t, B, H, T, nh, pos0, params, S, z, out, ws, ws_bytes, stream);
}

sanatan_status sanatan_prefill_four_channel(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                            int H, int T, int64_t pos0, const sanatan_params* params, float* S4,
                                            float* z4, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return ext_prefill(q, k, v, t, B, H, T, 0, pos0, params, S4, z4, out, ws, ws_bytes, stream);
}

sanatan_status sanatan_decode_step_harmonics(const float* q, const float* k, const float* v, int N, int64_t pos,
                                             const int64_t* posv, int nh, const sanatan_params* params, float* S,
                                             float* z, float* out, hipStream_t stream) {
  if (!q || !k || !v || !S || !z || !out || N <= 0 || nh < 1 || (!posv && !pos_ok(pos)))
    return SANATAN_ERR_INVALID_ARG;
  if (nh > 2) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  return hip_status(launch_decode_step_harmonics(q, k, v, N, pos, posv, nh, consts(params), S, z, out, stream));
}

size_t sanatan_attention_backward_workspace_bytes(int B, int H, int T, sanatan_dtype t, const sanatan_params* params) {
  (void)params;
  if (!sizes_ok(B, H, T) || T > kMaxQuadraticT || !dtype_ok(t)) return 0;
  return backward_ws_bytes(B, H, T, t);
}

sanatan_status sanatan_attention_backward(const void* q, const void* k, const void* v, const void* dout,
                                          sanatan_dtype t, int B, int H, int T, int p, int64_t pos0,
                                          const sanatan_params* params, void* dq, void* dk, void* dv, float* domega,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv || !domega || !dtype_ok(t) || !sizes_ok(B, H, T) ||
      (p != 1 && p != 2))
    return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxQuadraticT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (!ws || ws_bytes < backward_ws_bytes(B, H, T, t)) return SANATAN_ERR_WORKSPACE;
  return hip_status(
      launch_backward(q, k, v, dout, t, B, H, T, p, pos0, consts(params), dq, dk, dv, domega, ws, stream));
}

sanatan_status sanatan_attention_backward_saved(const void* q, const void* k, const void* v, const void* dout,
                                                const float* saved, sanatan_dtype t, int B, int H, int T, int p,
                                                int64_t pos0, const sanatan_params* params, void* dq, void* dk,
                                                void* dv, float* domega, void* ws, size_t ws_bytes,
                                                hipStream_t stream) {
  if (!q || !k || !v || !dout || !saved || !dq || !dk || !dv || !domega || !dtype_ok(t) || !sizes_ok(B, H, T) ||
      (p != 1 && p != 2))
    return SANATAN_ERR_INVALID_ARG;
  if (!pos_ok(pos0) || !pos_ok(pos0 + (int64_t)T - 1)) return SANATAN_ERR_INVALID_ARG;
  if (T > kMaxQuadraticT) return SANATAN_ERR_UNSUPPORTED;
  const sanatan_status ps = check_params(params);
  if (ps != SANATAN_OK) return ps;
  if (!ws || ws_bytes < backward_ws_bytes(B, H, T, t)) return SANATAN_ERR_WORKSPACE;
  return hip_status(
      launch_backward(q, k, v, dout, t, B, H, T, p, pos0, consts(params), dq, dk, dv, domega, ws, stream, saved));
}

}  // extern "C"
