/*
 * sanatan.h -- C ABI of libsanatan.so: SANATAN root-parity gated angular attention on gfx950.
 *
 * Method (cited by page title and section):
 *   [N] "SANATAN: root-label gated angular kernel, exact recurrence and revised evidence"
 *       (reading notes on the SANATAN v2 paper), §2.2 angle map / root label / rotation,
 *       §2.3 six-channel feature map, §2.6 normalised power attention, §2.7 exact recurrence.
 *   [F] The author's forum post restating the feature map and the p=1 recurrence.
 *
 * Per head, with content dim d, value dim d_v, positions t = pos0 + i:
 *   theta = pi u / (1 + |u|)                                    [N] §2.2
 *   r     = tanh(gamma (cos(theta + omega_a) - sin(theta + omega_a)))   (unrotated angle)
 *   theta_rot = theta + t lambda_a,  lambda_a = lambda_base^(-a/d), a = 0..d-1
 *   Phi   = [1, cos theta_rot, sin theta_rot, r, r cos theta_rot, r sin theta_rot]  [N] §2.3
 *   kappa(t,s) = <Phi(q_t), Phi(k_s)> = sum_a (1 + r_q r_k)(1 + cos dtheta_rot)
 *   p-th power attention: w = (kappa/c)^p, o_t = sum_{s<=t} w v_s / (sum_{s<=t} w + eps)  [N] §2.6
 *   p = 1 recurrence: S_t = S_{t-1} + Phi(k_t) v_t^T, z_t = z_{t-1} + Phi(k_t),
 *                     o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c eps)                     [N] §2.7
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller; contiguous row-major, last dim fastest.
 *   - Feature vectors and state rows use channel-major order: feature row c*d + a, channel
 *     c = 0..5 for (1, cos, sin, r, r cos, r sin).  (The notes concatenate per-dim blocks;
 *     kappa is invariant to the permutation.)
 *   - The library never allocates device memory inside a call and keeps no state between calls
 *     beyond cached device properties.  Calls are asynchronous on `stream`; errors are returned as
 *     status codes, never thrown.  Arguments are validated on the host BEFORE any launch; on a
 *     non-OK status nothing has been launched, except SANATAN_ERR_HIP, which reports a launch
 *     failure (hipGetLastError) after the fact.
 *   - Only d = d_v = 64 is implemented; other values return SANATAN_ERR_UNSUPPORTED.
 *   - Calls that share output or state buffers on overlapping streams race; order them on one stream.
 *   - NaN/Inf inputs propagate; they are not checked.
 */
#ifndef SANATAN_H
#define SANATAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SANATAN_OK = 0,
  SANATAN_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, unknown enum, bad parameter value */
  SANATAN_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (d or d_v != 64, chunk not supported) */
  SANATAN_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the matching *_workspace_bytes() */
  SANATAN_ERR_HIP = 4          /* a kernel launch failed */
} sanatan_status;

typedef enum { SANATAN_F32 = 0, SANATAN_BF16 = 1 } sanatan_dtype;

/* Method parameters. The struct itself is host memory, read during the call only. */
typedef struct {
  int d;               /* content dims per head; must be 64 */
  int d_v;             /* value dims per head; must be 64 */
  float gamma;         /* root sharpness gamma (>= 0) */
  float c;             /* score normaliser c (> 0); the notes use 4d */
  float eps;           /* normalised epsilon (>= 0); denominators are sum(kappa) + c*eps */
  double lambda_base;  /* rotation ladder base (> 0): lambda_a = lambda_base^(-a/d) */
  const float* omega;  /* DEVICE [n_param_heads][d] fp32 root anchors omega (learned per head in [N]) */
  int n_param_heads;   /* head h (or head-state i) uses omega row h % n_param_heads; >= 1 */
} sanatan_params;

/* Bytes of one head's fp32 recurrent state: S [6d][d_v] plus z [6d].  [N] §4.5 memory equation. */
size_t sanatan_state_bytes(int d, int d_v);

/*
 * sanatan_featurize -- the feature map Phi of every vector of u.  [N] §2.2-§2.3.
 *   u    : [B][H][T][d], element type in_t (F32 or BF16).
 *   pos0 : position of u[..][..][0]; token i sits at pos0 + i.  Every position must satisfy |pos| < 2^53
 *          (else INVALID_ARG); the phase t lambda_a / (2 pi) is reduced in fp64 with an exact two-product,
 *          so it stays accurate to about 2^-53 revolutions over that whole range.
 *   phi  : [B][H][T][6d], element type out_t; row c*d + a as above.
 * Head h uses omega row h % n_param_heads.  Returns INVALID_ARG for NULL pointers or
 * B, H, T <= 0; UNSUPPORTED for d != 64.
 */
sanatan_status sanatan_featurize(const void* u, sanatan_dtype in_t, int B, int H, int T, int64_t pos0,
                                 const sanatan_params* params, void* phi, sanatan_dtype out_t,
                                 hipStream_t stream);

/* Workspace bytes sanatan_prefill_chunked needs for these sizes (0 on invalid sizes).  The prefill splits the
 * B*H*ceil(T/chunk) chunks over one workgroup per compute unit of the current device. */
size_t sanatan_prefill_workspace_bytes(int B, int H, int T, int chunk, const sanatan_params* params);

/*
 * sanatan_prefill_chunked -- normalised causal p=1 attention over whole sequences, computed as
 * the exact chunked regrouping of the recurrence of [N] §2.7: within a chunk the masked product
 * mask(Phi(Q) Phi(K)^T) V, across chunks the readout Phi(Q) S; S += Phi(K)^T V after each chunk.
 *   q, k  : [B][H][T][d],  v : [B][H][T][d_v], element type t (F32 or BF16).
 *   chunk : chunk length in tokens; one of 16, 32, 64, 128 (128 with BF16 only).
 *   pos0  : position of token 0; pos0 and pos0 + T - 1 must satisfy |pos| < 2^53 (else INVALID_ARG).
 *   T     : at most 2^22 (else UNSUPPORTED): the per-sequence byte ranges of the kernels' buffer loads must
 *           fit a buffer descriptor's 31-bit range.
 *   S, z  : both NULL -> start from the zero state and do not return a final state;
 *           both non-NULL -> fp32 S [B][H][6d][d_v], z [B][H][6d] hold the initial state on entry
 *           and the state after the last token on exit (in place).  One NULL -> INVALID_ARG.
 *   out   : [B][H][T][d_v], element type t; o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c eps).
 *   ws    : device workspace of at least sanatan_prefill_workspace_bytes() bytes, else WORKSPACE.
 * Accumulation is fp32; with BF16 inputs the products run on bf16 MFMA with fp32 accumulation.
 */
sanatan_status sanatan_prefill_chunked(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                       int H, int T, int chunk, int64_t pos0, const sanatan_params* params,
                                       float* S, float* z, void* out, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/*
 * Test hook: sanatan_prefill_chunked with the chunk list split over `workgroups` workgroups instead of one
 * per compute unit (0 = one per compute unit; larger counts are capped at the number of chunks), so that
 * tests can force a sequence into many pieces or one workgroup through many sequences.  The results equal
 * those of the default split up to the rounding order of the pieces' state sums.  The workspace must hold
 * sanatan_prefill_workspace_bytes_partitioned() bytes for the same count; a negative count is INVALID_ARG.
 */
size_t sanatan_prefill_workspace_bytes_partitioned(int B, int H, int T, int chunk, int workgroups,
                                                  const sanatan_params* params);
sanatan_status sanatan_prefill_chunked_partitioned(const void* q, const void* k, const void* v, sanatan_dtype t,
                                                   int B, int H, int T, int chunk, int workgroups, int64_t pos0,
                                                   const sanatan_params* params, float* S, float* z, void* out,
                                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sanatan_prefill_chunked_ragged -- sanatan_prefill_chunked over a batch of sequences of different lengths in
 * one call: the prompts of a serving batch, whose states then continue at their own positions in
 * sanatan_decode_step_positions.  The recurrence of [N] §2.7 runs per sequence, so batch element b is the
 * prefill of its first lengths[b] tokens alone.
 *   q, k, v, out : [B][H][T][.] as for sanatan_prefill_chunked, right-padded: batch element b uses rows
 *                  0 .. lengths[b] - 1 of each head; rows from lengths[b] on are neither read nor written.
 *   lengths      : DEVICE int32 [B]; each value is clamped to [0, T] (the host cannot see them).  A length of
 *                  0 leaves that element's output rows and state untouched.
 *   pos0         : position of token 0 of every sequence; checked as for sanatan_prefill_chunked over T.
 *   S, z         : as for sanatan_prefill_chunked; on exit element b's state is the one after its last token.
 *   ws           : at least sanatan_prefill_workspace_bytes(B, H, T, chunk) bytes.
 * The chunks of all sequences are split over one workgroup per compute unit as one flattened list, so one
 * launch balances the whole batch.  Every call runs the state pass and the boundary scan (the pieces depend
 * on the lengths), a few microseconds more than a uniform call with the same chunk count.
 * Errors: those of sanatan_prefill_chunked, and INVALID_ARG for a NULL lengths pointer.
 */
sanatan_status sanatan_prefill_chunked_ragged(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                              int H, int T, int chunk, const int32_t* lengths, int64_t pos0,
                                              const sanatan_params* params, float* S, float* z, void* out,
                                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sanatan_prefill_chunked_noalloc -- sanatan_prefill_chunked without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The workspace is a fixed 48 MiB device array inside the library (one per GPU, held until
 * the process ends); the call allocates nothing.  Arguments, results and errors are those of
 * sanatan_prefill_chunked without ws/ws_bytes, plus SANATAN_ERR_WORKSPACE when the sizes need more than
 * 48 MiB of workspace (sanatan_prefill_workspace_bytes() > 48 MiB: e.g. B*H above about 240 sequences at
 * T = 2048 on a 256-CU device), and SANATAN_ERR_HIP if the array's address cannot be found.
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU race; order them on
 * one stream.  The results are bitwise those of sanatan_prefill_chunked with the same arguments.
 */
sanatan_status sanatan_prefill_chunked_noalloc(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                               int H, int T, int chunk, int64_t pos0, const sanatan_params* params,
                                               float* S, float* z, void* out, hipStream_t stream);

/*
 * sanatan_decode_step -- one token of the p=1 constant-state recurrence for N independent
 * head-states (e.g. batch x layers x heads).  [N] §2.7: write the token into the state, then read.
 *   q, k : [N][d] fp32;  v : [N][d_v] fp32;  pos : position of this token (shared by all N), |pos| < 2^53
 *          (else INVALID_ARG).
 *   S    : [N][6d][d_v] fp32, z : [N][6d] fp32, updated in place.
 *   out  : [N][d_v] fp32.
 * Head-state i uses omega row i % n_param_heads.  Streams each state once (read + write).
 */
sanatan_status sanatan_decode_step(const float* q, const float* k, const float* v, int N, int64_t pos,
                                   const sanatan_params* params, float* S, float* z, float* out,
                                   hipStream_t stream);

/*
 * sanatan_decode_step_positions -- sanatan_decode_step with one position per head-state, for a batch
 * whose sequences have reached different lengths.  The position of a token sets the rotation
 * theta + t lambda_a of both its feature maps ([N] §2.2), so each head-state's phase comes from its
 * own entry.
 *   pos  : device [N] int64, the position of head-state i's token, read only.  The library cannot check
 *          device values: an entry with |pos| >= 2^53 gives a phase of reduced accuracy (never a fault).
 *   Everything else as sanatan_decode_step.  With every entry equal to one position the results are
 *   bitwise those of sanatan_decode_step at that position.  A null pos is INVALID_ARG.
 */
sanatan_status sanatan_decode_step_positions(const float* q, const float* k, const float* v, int N,
                                             const int64_t* pos, const sanatan_params* params, float* S,
                                             float* z, float* out, hipStream_t stream);

/*
 * Compact recurrent state.  Channel 0 of both feature maps is the constant 1 ([N] §2.3), so the d rows of
 * S that channel 0 owns all receive the same v_t in every update ([N] §2.7) and stay equal, as do their d
 * entries of z.  The compact layout keeps them once:
 *   Sc : [N][5d+1][d_v] fp32, row 0 = the shared channel-0 row, row 1 + (c-1) d + a = full row c d + a
 *        (channels c = 1..5);
 *   zc : [N][5d+1] fp32, the same rows.
 * It holds the same information as a full state whose channel-0 rows are equal (every state the
 * recurrence builds from a zero or compact start), in 17 % fewer bytes.
 */
/* Bytes of one head's compact state: (5d+1) x (d_v+1) floats. */
size_t sanatan_compact_state_bytes(int d, int d_v);

/*
 * sanatan_state_compact -- full state (S [N][6d][d_v], z [N][6d]) -> compact (Sc, zc), taking row 0 of the
 * channel-0 block.  sanatan_state_expand -- compact -> full, writing the shared row into all d channel-0
 * rows.  Pure copies (bitwise); d = d_v = 64 layouts; source and destination must not overlap.
 * INVALID_ARG for NULL pointers or N <= 0.
 */
sanatan_status sanatan_state_compact(const float* S, const float* z, int N, float* Sc, float* zc,
                                     hipStream_t stream);
sanatan_status sanatan_state_expand(const float* Sc, const float* zc, int N, float* S, float* z,
                                    hipStream_t stream);

/*
 * sanatan_decode_step_compact -- sanatan_decode_step on the compact state.  A token adds 1 x v to the
 * shared channel-0 row and 1 to its z entry; the readout weighs that row (and entry) by d, once for each
 * of the d equal rows it stands for.  The results equal those of the full-state call up to the rounding
 * of that sum.
 *   pos, posv : posv NULL -> every head-state at position pos; else device [N] int64, one position per
 *               head-state (as sanatan_decode_step_positions), and pos is ignored.
 *   Sc, zc    : the compact state, updated in place.  Everything else as sanatan_decode_step.
 */
sanatan_status sanatan_decode_step_compact(const float* q, const float* k, const float* v, int N, int64_t pos,
                                           const int64_t* posv, const sanatan_params* params, float* Sc,
                                           float* zc, float* out, hipStream_t stream);

/*
 * The unclipped four-channel kernel of [N] §2.5 ([1, r, r cos theta_rot, r sin theta_rot] per dim) has the
 * same exact p = 1 recurrence over its own features.  Its state is kept compact like the six-channel one:
 *   S4 : [N][3d+1][d_v] fp32, row 0 = the shared channel-0 row, row 1 + (c-3) d + a = channel c of dim a
 *        (c = 3, 4, 5: r, r cos, r sin);
 *   z4 : [N][3d+1] fp32, the same rows.
 * sanatan_four_channel_state_bytes: (3d+1) x (d_v+1) floats.
 * sanatan_decode_step_four_channel: one token for N head-states on that state,
 *   o = Phi4(q)^T S4 / (Phi4(q)^T z4 + c eps), with the updated state as in sanatan_decode_step; the weight
 *   kappa4 is not clipped, so the denominator can be near zero or negative.  pos / posv as in
 *   sanatan_decode_step_compact; everything else as sanatan_decode_step.
 */
size_t sanatan_four_channel_state_bytes(int d, int d_v);
sanatan_status sanatan_decode_step_four_channel(const float* q, const float* k, const float* v, int N,
                                                int64_t pos, const int64_t* posv, const sanatan_params* params,
                                                float* S4, float* z4, float* out, hipStream_t stream);

/* Workspace bytes sanatan_quadratic_ref_p2 needs (0 on invalid sizes). */
size_t sanatan_quadratic_workspace_bytes(int B, int H, int T, sanatan_dtype t, const sanatan_params* params);

/*
 * sanatan_quadratic_ref_p2 -- normalised causal power attention in its masked quadratic
 * (training) form, no recurrence: w = (kappa/c)^p, o_t = sum_{s<=t} w v_s / (sum w + eps).
 * [N] §2.6; p = 2 is the sharpened kernel trained first in [N] §4.1, p = 1 the deployed one.
 *   q, k : [B][H][T][d], v, out : [B][H][T][d_v], element type t; p : 1 or 2 (else INVALID_ARG).
 *   T    : at most 2^20 (else UNSUPPORTED): one sequence's key features [T][6d] must fit a buffer
 *          descriptor's 31-bit byte range.  pos0 as in sanatan_featurize.
 *   ws   : at least sanatan_quadratic_workspace_bytes() bytes: the position phase table [T][d] fp32
 *          (padded to 256 bytes), then Phi(K) [B][H][T][6d] in element type t.
 */
sanatan_status sanatan_quadratic_ref_p2(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                        int H, int T, int p, int64_t pos0, const sanatan_params* params,
                                        void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sanatan_quadratic_train -- sanatan_quadratic_ref_p2 that also saves what its backward pass needs, so that a
 * training step's backward (sanatan_attention_backward_saved) skips its statistics pass.  saved: DEVICE fp32,
 * 16-byte aligned, sanatan_quadratic_saved_bytes() bytes, written: the output rows in fp32 [B][H][T][d_v], then per
 * query row the reciprocal of its normaliser in the kernels' scaled units, 1 / (sum_{s<=t} kappa_ts^p + eps c^p),
 * [B][H][T].  saved NULL is INVALID_ARG; everything else as sanatan_quadratic_ref_p2 (out is bitwise the same).
 */
size_t sanatan_quadratic_saved_bytes(int B, int H, int T, const sanatan_params* params);
sanatan_status sanatan_quadratic_train(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H,
                                       int T, int p, int64_t pos0, const sanatan_params* params, void* out,
                                       float* saved, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sanatan_quadratic_four_channel -- the same masked quadratic form on the unclipped four-channel kernel
 * of [N] §2.5: per dim the features are [1, r, r cos theta_rot, r sin theta_rot] (the independent cos and
 * sin channels dropped), so
 *   kappa4(t,s) = sum_a 1 + r_q r_k (1 + cos(theta_q - theta_k + (t - s) lambda_a)),
 *   w = (kappa4/c)^p for s <= t, o_t = sum_{s<=t} w v_s / (sum w + eps).
 * No max(kappa4, 0) is applied: a mismatched pair of hard roots contributes -cos(dtheta) to a dim, so with
 * p = 1 a weight, and the denominator, can be negative or near zero.  With p = 2 strongly mismatched pairs
 * get large positive weights: this is not the clipped four-channel attention max(kappa4, 0)^p of the pages'
 * own implementation, which this library does not provide.  c is the caller's (params->c).
 * Arguments, workspace and errors exactly as sanatan_quadratic_ref_p2.
 */
sanatan_status sanatan_quadratic_four_channel(const void* q, const void* k, const void* v, sanatan_dtype t,
                                              int B, int H, int T, int p, int64_t pos0,
                                              const sanatan_params* params, void* out, void* ws,
                                              size_t ws_bytes, hipStream_t stream);

/*
 * sanatan_prefill_four_channel -- the chunked p = 1 prefill on the unclipped four-channel kernel of [N] §2.5
 * (features [1, r, r cos theta_rot, r sin theta_rot] per dim), whose recurrence ([N] §2.7 applied to these
 * features) is exact: o_t = Phi4(q_t)^T S4_t / (Phi4(q_t)^T z4_t + c eps).  The weights are not clipped, so a
 * denominator can be near zero or negative.
 *   S4, z4 : NULL (zero start, no final state) or the compact four-channel state of
 *            sanatan_decode_step_four_channel, [B][H][3d+1][d_v] and [B][H][3d+1], in/out.
 *   Everything else as sanatan_prefill_chunked without `chunk` (this path walks 32-token chunks, one workgroup
 *   per sequence); ws: at least sanatan_prefill_four_channel_workspace_bytes() bytes: for bf16 the position
 *   phase table (the features are formed while each chunk is staged), for fp32 Phi4(Q) and Phi4(K); then, when
 *   sequences are split across compute units, the pieces' state increments.  The final state continues exactly
 *   in sanatan_decode_step_four_channel.
 */
size_t sanatan_prefill_four_channel_workspace_bytes(int B, int H, int T, sanatan_dtype t,
                                                    const sanatan_params* params);
sanatan_status sanatan_prefill_four_channel(const void* q, const void* k, const void* v, sanatan_dtype t, int B,
                                            int H, int T, int64_t pos0, const sanatan_params* params, float* S4,
                                            float* z4, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Spectral harmonics (the notes' reading of the paper's Appendix B outlook: cos(n theta), sin(n theta) harmonics
 * added per dim keep the p = 1 map explicit, at the cost of more features and a larger state).  Reading taken:
 * harmonics n = 1..nh of the rotated angle theta_rot = theta + t lambda_a, each gated by the same root label,
 *   Phi_h per dim = [1, cos n theta_rot, sin n theta_rot (n = 1..nh), r, r cos n theta_rot, r sin n theta_rot],
 *   kappa_h(t,s)  = sum_a (1 + r_q r_k)(1 + sum_{n=1..nh} cos(n dtheta_a)),
 * stored channel-major: channel 0 = 1, 2n-1 / 2n = cos / sin of n theta_rot, 2nh+1 = r, 2nh+2n / 2nh+2n+1 =
 * r cos / r sin of n theta_rot; feature row c d + a.  nh = 1 is the six-channel map.  For nh >= 2 the factor
 * 1 + sum cos(n x) takes negative values, so kappa_h and a denominator can be negative (no clipping).
 * The state of one head is S [(2+4nh)d][d_v], z [(2+4nh)d] (sanatan_harmonics_state_bytes).  nh: 1 or 2
 * (nh < 1 INVALID_ARG, nh > 2 UNSUPPORTED).
 * sanatan_prefill_harmonics: the chunked p = 1 prefill on Phi_h; arguments as sanatan_prefill_four_channel, with
 *   S, z of this layout; ws at least sanatan_prefill_harmonics_workspace_bytes().
 * sanatan_decode_step_harmonics: one token of the recurrence on Phi_h for N head-states; pos / posv as in
 *   sanatan_decode_step_compact; everything else as sanatan_decode_step.
 */
size_t sanatan_harmonics_state_bytes(int d, int d_v, int nh);
size_t sanatan_prefill_harmonics_workspace_bytes(int B, int H, int T, sanatan_dtype t, int nh,
                                                 const sanatan_params* params);
sanatan_status sanatan_prefill_harmonics(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H,
                                         int T, int nh, int64_t pos0, const sanatan_params* params, float* S, float* z,
                                         void* out, void* ws, size_t ws_bytes, hipStream_t stream);
sanatan_status sanatan_decode_step_harmonics(const float* q, const float* k, const float* v, int N, int64_t pos,
                                             const int64_t* posv, int nh, const sanatan_params* params, float* S,
                                             float* z, float* out, hipStream_t stream);

/*
 * Backward pass of normalised causal power attention: the gradients of L = sum_t <dout_t, o_t> with respect
 * to q, k, v and the root anchors omega, where o is the output of sanatan_quadratic_ref_p2 with the same p
 * (for p = 1 also of sanatan_prefill_chunked, which computes the same function).  omega is learned and the
 * method is trained, p = 2 first and then p = 1 ([N] §2.2 root equation, §4.1), so both exponents are served.
 *   q, k, dq, dk : [B][H][T][d];  v, dout, dv : [B][H][T][d_v]; element type t for all of them.
 *   domega : DEVICE fp32 [n_param_heads][d]; row r receives the sum over every head h with h % n_param_heads
 *            == r (overwritten, not accumulated).
 *   p : 1 or 2 (else INVALID_ARG);  pos0 as in sanatan_featurize;  T at most 2^20 (else UNSUPPORTED).
 *   ws : at least sanatan_attention_backward_workspace_bytes() bytes (else WORKSPACE): the position phase
 *        table, Phi(Q) and Phi(K) in element type t, per-row statistics, fp32 feature gradients
 *        [B][H][T][6d] for q and k (used at p = 2), per-block omega partials, and (p = 1, sequences split into
 *        pieces) the pieces' recurrence states.  The size depends on the device's compute-unit count.
 * The forward statistics (denominators and <dout_t, o_t>) are recomputed from q, k, v in fp32.  At p = 1 they
 * and the gradients follow the recurrence form (reading notes §2.7: each is a prefix or suffix sum of feature
 * outer products), in time linear in T; at p = 2 they sum over score tiles.  Products run on bf16 MFMA (fp32
 * MFMA for fp32 inputs) with fp32 accumulation.  Bitwise deterministic.
 */
size_t sanatan_attention_backward_workspace_bytes(int B, int H, int T, sanatan_dtype t,
                                                  const sanatan_params* params);
sanatan_status sanatan_attention_backward(const void* q, const void* k, const void* v, const void* dout,
                                          sanatan_dtype t, int B, int H, int T, int p, int64_t pos0,
                                          const sanatan_params* params, void* dq, void* dk, void* dv, float* domega,
                                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sanatan_attention_backward_saved -- sanatan_attention_backward given the statistics that sanatan_quadratic_train
 * saved for the same q, k, v, p, pos0 and params.  At p = 2 they replace the statistics pass (a second
 * forward-sized pass over the score tiles): delta_t = <dout_t, o_t> is summed in fp32 from the saved fp32 output
 * rows (the bf16 output would leave delta too coarse for G's cancelling rows).  At p = 1 the chunked recurrences
 * form the statistics on the way and the saved values are not read.  saved NULL is INVALID_ARG; workspace,
 * outputs and everything else as sanatan_attention_backward.
 */
sanatan_status sanatan_attention_backward_saved(const void* q, const void* k, const void* v, const void* dout,
                                                const float* saved, sanatan_dtype t, int B, int H, int T, int p,
                                                int64_t pos0, const sanatan_params* params, void* dq, void* dk,
                                                void* dv, float* domega, void* ws, size_t ws_bytes,
                                                hipStream_t stream);

/* Static human-readable name of a status code. */
const char* sanatan_status_string(sanatan_status status);

#ifdef __cplusplus
}
#endif

#endif /* SANATAN_H */
