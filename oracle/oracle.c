/*
 * oracle.c -- plain, slow, fp64 CPU reference for SANATAN p=1/p=2 attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Every quantity is IEEE binary64 with the C library's cos/sin/tanh/pow; built without
 * fast-math and with FMA contraction off, so what is written is what is computed.
 *
 * Sources (the pages are cited by title and section):
 *   [N]  "SANATAN: root-label gated angular kernel, exact recurrence and revised
 *        evidence" -- reading notes on the SANATAN v2 paper (page 1).
 *   [F]  The author's forum post restating the method (page 2).
 *
 * Definitions used (one head, d content dims, d_v value dims, positions t = pos0 + i):
 *   theta(u)   = pi * u / (1 + |u|)                         [N] §2.2, angle map phi(u)
 *   r(u)       = tanh(gamma * (cos(theta+omega_a) - sin(theta+omega_a)))
 *                 -- from the UNROTATED angle                [N] §2.2, root equation; [F]
 *   lambda_a   = base^(-a/d), a = 0..d-1                     (fixed geometric ladder; the
 *                 notes' §2.2 rotation equation uses a learned per-dim frequency -- this
 *                 ladder is the reading taken, first frequency 1 rad/token)
 *   theta_rot  = theta + t * lambda_a                        [N] §2.2, rotation equation
 *   kappa(t,s) = sum_a (1 + r_q r_k)(1 + cos(theta_q - theta_k + (t-s) lambda_a))
 *                                                            [N] overview kappa equation
 *   w(t,s)     = (kappa / c)^p, s <= t                       [N] §2.6 power normalisation
 *   o_t        = sum_s w v_s / (sum_s w + eps)               [N] §2.6
 *   Phi_a      = [1, cos th_rot, sin th_rot, r, r cos th_rot, r sin th_rot]
 *                                                            [N] §2.3 six-channel block; [F]
 *                stored channel-major: feature row c*d + a.
 *   S_t = S_{t-1} + Phi(k_t) v_t^T, z_t = z_{t-1} + Phi(k_t),
 *   o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c*eps)          [N] §2.7 recurrence and the
 *                                                            normalising-constant paragraph
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PI 3.14159265358979323846

/* Angle map: [N] §2.2, phi(u) = pi u / (1 + |u|). */
static double sanatan_angle(double u) { return ORACLE_PI * u / (1.0 + fabs(u)); }

/* Soft root label from the unrotated angle: [N] §2.2 root equation. */
static double sanatan_root(double theta, double omega, double gamma) {
  return tanh(gamma * (cos(theta + omega) - sin(theta + omega)));
}

/* Rotation frequency of content dim a: base^(-a/d). */
static double sanatan_freq(int a, int d, double base) { return pow(base, -(double)a / (double)d); }

/* Exported so that tests can check angle/root/frequency at special points. */
double oracle_angle(double u) { return sanatan_angle(u); }
double oracle_root(double u, double omega, double gamma) { return sanatan_root(sanatan_angle(u), omega, gamma); }
double oracle_freq(int a, int d, double base) { return sanatan_freq(a, d, base); }

/*
 * Feature map of T vectors u[T][d] at positions pos0..pos0+T-1 -> phi[T][6d], channel-major
 * (row c*d + a; c = 0..5 for 1, cos, sin, r, r cos, r sin).  [N] §2.3, six-channel block.
 */
void oracle_features(const double* u, int T, int d, int64_t pos0, const double* omega, double gamma,
                     double lambda_base, double* phi) {
  for (int i = 0; i < T; i++) {
    const double t = (double)(pos0 + i);
    double* row = phi + (size_t)i * 6 * d;
    for (int a = 0; a < d; a++) {
      const double th = sanatan_angle(u[(size_t)i * d + a]);
      const double r = sanatan_root(th, omega[a], gamma);
      const double th_rot = th + t * sanatan_freq(a, d, lambda_base);
      const double c = cos(th_rot), s = sin(th_rot);
      row[0 * d + a] = 1.0;
      row[1 * d + a] = c;
      row[2 * d + a] = s;
      row[3 * d + a] = r;
      row[4 * d + a] = r * c;
      row[5 * d + a] = r * s;
    }
  }
}

/*
 * kappa between query q[d] at position t and key k[d] at position s, written as the
 * sum of gate times angular similarity with the cosine of the rotated-angle
 * difference -- NOT through the feature map.  [N] overview equation; §2.2 notes that
 * the rotation enters only as (t - s) lambda.
 */
double oracle_kappa(const double* q, const double* k, int d, int64_t t, int64_t s, const double* omega,
                    double gamma, double lambda_base) {
  double acc = 0.0;
  for (int a = 0; a < d; a++) {
    const double thq = sanatan_angle(q[a]), thk = sanatan_angle(k[a]);
    const double rq = sanatan_root(thq, omega[a], gamma), rk = sanatan_root(thk, omega[a], gamma);
    const double dth = thq - thk + (double)(t - s) * sanatan_freq(a, d, lambda_base);
    acc += (1.0 + rq * rk) * (1.0 + cos(dth));
  }
  return acc;
}

/*
 * The four-channel kernel, unclipped: Phi_4 = [1, r, r cos, r sin] per dim drops the independent
 * cos and sin channels, so one dim contributes 1 + r_q r_k (1 + cos(dtheta)) -- [N] §2.5.  It can be
 * negative (mismatched hard roots give -cos(dtheta)); no max(., 0) is applied here.
 */
double oracle_kappa4(const double* q, const double* k, int d, int64_t t, int64_t s, const double* omega,
                     double gamma, double lambda_base) {
  double acc = 0.0;
  for (int a = 0; a < d; a++) {
    const double thq = sanatan_angle(q[a]), thk = sanatan_angle(k[a]);
    const double rq = sanatan_root(thq, omega[a], gamma), rk = sanatan_root(thk, omega[a], gamma);
    const double dth = thq - thk + (double)(t - s) * sanatan_freq(a, d, lambda_base);
    acc += 1.0 + rq * rk * (1.0 + cos(dth));
  }
  return acc;
}

/*
 * Normalised causal power attention, direct quadratic form, one head.
 *   q,k [T][d], v [T][dv], positions pos0+i.  Output rows: all T rows when rows == NULL
 *   (out [T][dv]), else only rows[0..n_rows) (out [n_rows][dv]).
 * Weight w(t,s) = (kappa(t,s)/c)^p for s <= t, o_t = sum w v / (sum w + eps).
 * [N] §2.6 normalised power attention; mask inclusive s <= t as in §2.7.
 * The per-token angles and roots are tabulated first (they are per-token quantities of
 * the definition); kappa itself is summed with the cosine of a difference per pair.
 */
static void attention_direct_impl(const double* q, const double* k, const double* v, int T, int d, int dv,
                                  const double* omega, double gamma, double lambda_base, double c, double eps,
                                  int p, const int* rows, int n_rows, int four, double* out) {
  double* thq = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* thk = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* rq = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* rk = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* lam = (double*)malloc(sizeof(double) * (size_t)d);
  for (int a = 0; a < d; a++) lam[a] = sanatan_freq(a, d, lambda_base);
  for (size_t i = 0; i < (size_t)T * d; i++) {
    const int a = (int)(i % (size_t)d);
    thq[i] = sanatan_angle(q[i]);
    thk[i] = sanatan_angle(k[i]);
    rq[i] = sanatan_root(thq[i], omega[a], gamma);
    rk[i] = sanatan_root(thk[i], omega[a], gamma);
  }
  const int n_out = rows ? n_rows : T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < n_out; j++) {
    const int t = rows ? rows[j] : j;
    double* o = out + (size_t)j * dv;
    double* num = (double*)calloc((size_t)dv, sizeof(double));
    double den = 0.0;
    for (int s = 0; s <= t; s++) {
      double kap = 0.0;
      for (int a = 0; a < d; a++) {
        const double dth = thq[(size_t)t * d + a] - thk[(size_t)s * d + a] + (double)(t - s) * lam[a];
        const double gate = rq[(size_t)t * d + a] * rk[(size_t)s * d + a];
        kap += four ? 1.0 + gate * (1.0 + cos(dth)) : (1.0 + gate) * (1.0 + cos(dth));
      }
      double w = kap / c;
      double wp = 1.0;
      for (int e = 0; e < p; e++) wp *= w;
      den += wp;
      for (int n = 0; n < dv; n++) num[n] += wp * v[(size_t)s * dv + n];
    }
    for (int n = 0; n < dv; n++) o[n] = num[n] / (den + eps);
    free(num);
  }
  free(thq);
  free(thk);
  free(rq);
  free(rk);
  free(lam);
}

void oracle_attention_direct(const double* q, const double* k, const double* v, int T, int d, int dv,
                             int64_t pos0, const double* omega, double gamma, double lambda_base, double c,
                             double eps, int p, const int* rows, int n_rows, double* out) {
  (void)pos0; /* only t - s enters */
  attention_direct_impl(q, k, v, T, d, dv, omega, gamma, lambda_base, c, eps, p, rows, n_rows, 0, out);
}

/* The same normalised power attention on the unclipped four-channel kernel (oracle_kappa4), [N] §2.5-§2.6. */
void oracle_attention_direct4(const double* q, const double* k, const double* v, int T, int d, int dv,
                              int64_t pos0, const double* omega, double gamma, double lambda_base, double c,
                              double eps, int p, const int* rows, int n_rows, double* out) {
  (void)pos0;
  attention_direct_impl(q, k, v, T, d, dv, omega, gamma, lambda_base, c, eps, p, rows, n_rows, 1, out);
}

/*
 * p = 1 constant-state recurrence, one head, token by token.  [N] §2.7:
 *   S_t = S_{t-1} + Phi(k_t) v_t^T ; z_t = z_{t-1} + Phi(k_t)   (write, then read)
 *   o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c*eps)
 * S [6d][dv] and z [6d] hold the initial state on entry and the final state on exit.
 * out [T][dv] may be NULL (state only).
 */
void oracle_recurrent(const double* q, const double* k, const double* v, int T, int d, int dv, int64_t pos0,
                      const double* omega, double gamma, double lambda_base, double c, double eps, double* S,
                      double* z, double* out) {
  const int D = 6 * d;
  double* fq = (double*)malloc(sizeof(double) * (size_t)D);
  double* fk = (double*)malloc(sizeof(double) * (size_t)D);
  for (int i = 0; i < T; i++) {
    oracle_features(k + (size_t)i * d, 1, d, pos0 + i, omega, gamma, lambda_base, fk);
    for (int f = 0; f < D; f++) {
      z[f] += fk[f];
      for (int n = 0; n < dv; n++) S[(size_t)f * dv + n] += fk[f] * v[(size_t)i * dv + n];
    }
    if (!out) continue;
    oracle_features(q + (size_t)i * d, 1, d, pos0 + i, omega, gamma, lambda_base, fq);
    double den = 0.0;
    for (int f = 0; f < D; f++) den += fq[f] * z[f];
    for (int n = 0; n < dv; n++) {
      double num = 0.0;
      for (int f = 0; f < D; f++) num += fq[f] * S[(size_t)f * dv + n];
      out[(size_t)i * dv + n] = num / (den + c * eps);
    }
  }
  free(fq);
  free(fk);
}

/*
 * Many independent heads of the recurrence, one OpenMP task per head.
 *   q,k [NH][T][d], v [NH][T][dv]; omega rows: head j uses omega[(j % n_param_heads)*d ..].
 *   S [NH][6d][dv], z [NH][6d] in/out; out [NH][T][dv] or NULL.
 */
void oracle_recurrent_heads(const double* q, const double* k, const double* v, int NH, int T, int d, int dv,
                            int64_t pos0, const double* omega, int n_param_heads, double gamma,
                            double lambda_base, double c, double eps, double* S, double* z, double* out) {
  const size_t D = (size_t)6 * d;
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < NH; j++) {
    oracle_recurrent(q + (size_t)j * T * d, k + (size_t)j * T * d, v + (size_t)j * T * dv, T, d, dv, pos0,
                     omega + (size_t)(j % n_param_heads) * d, gamma, lambda_base, c, eps, S + (size_t)j * D * dv,
                     z + (size_t)j * D, out ? out + (size_t)j * T * dv : NULL);
  }
}

/*
 * Spectral harmonics (the outlook of Appendix B as the notes present it): cos(n theta), sin(n theta) harmonics
 * are added to each dim's angular part; at p = 1 the map stays explicit, but the features per dim, and so the
 * recurrent state, grow with the number of harmonics.  The notes fix no feature set; the reading taken here:
 * harmonics n = 1..nh of the ROTATED angle (so only t - s enters, as for the six-channel kernel), each gated
 * by the same root label:
 *   Phi_h per dim = [1, cos th_rot, sin th_rot, ..., cos nh th_rot, sin nh th_rot,
 *                    r, r cos th_rot, r sin th_rot, ..., r cos nh th_rot, r sin nh th_rot]   (2 + 4 nh channels)
 *   kappa_h(t,s) = sum_a (1 + r_q r_k)(1 + sum_{n=1..nh} cos(n x_a)),  x_a = theta_q - theta_k + (t - s) lambda_a
 * nh = 1 is the six-channel kernel.  For nh >= 2 the angular factor 1 + sum cos(n x) takes negative values,
 * so kappa_h can be negative: no clipping is applied (as for the unclipped four-channel kernel).
 * Channel-major layout: channel 0 = 1; channel 2n-1 = cos n th_rot, 2n = sin n th_rot (n = 1..nh);
 * channel 2nh+1 = r; channel 2nh+2n = r cos n th_rot, 2nh+2n+1 = r sin n th_rot.  Feature row c*d + a.
 */
void oracle_features_h(const double* u, int T, int d, int nh, int64_t pos0, const double* omega, double gamma,
                       double lambda_base, double* phi) {
  const int C = 2 + 4 * nh;
  for (int i = 0; i < T; i++) {
    const double t = (double)(pos0 + i);
    double* row = phi + (size_t)i * C * d;
    for (int a = 0; a < d; a++) {
      const double th = sanatan_angle(u[(size_t)i * d + a]);
      const double r = sanatan_root(th, omega[a], gamma);
      const double th_rot = th + t * sanatan_freq(a, d, lambda_base);
      row[0 * d + a] = 1.0;
      row[(size_t)(2 * nh + 1) * d + a] = r;
      for (int n = 1; n <= nh; n++) {
        const double c = cos((double)n * th_rot), s = sin((double)n * th_rot);
        row[(size_t)(2 * n - 1) * d + a] = c;
        row[(size_t)(2 * n) * d + a] = s;
        row[(size_t)(2 * nh + 2 * n) * d + a] = r * c;
        row[(size_t)(2 * nh + 2 * n + 1) * d + a] = r * s;
      }
    }
  }
}

/* kappa_h of one pair, as a sum over dims of gate times (1 + sum of cosines of multiples of the difference). */
double oracle_kappa_h(const double* q, const double* k, int d, int nh, int64_t t, int64_t s, const double* omega,
                      double gamma, double lambda_base) {
  double acc = 0.0;
  for (int a = 0; a < d; a++) {
    const double thq = sanatan_angle(q[a]), thk = sanatan_angle(k[a]);
    const double rq = sanatan_root(thq, omega[a], gamma), rk = sanatan_root(thk, omega[a], gamma);
    const double x = thq - thk + (double)(t - s) * sanatan_freq(a, d, lambda_base);
    double ang = 1.0;
    for (int n = 1; n <= nh; n++) ang += cos((double)n * x);
    acc += (1.0 + rq * rk) * ang;
  }
  return acc;
}

/* Normalised causal p = 1 attention on kappa_h, direct form, one head: o_t = sum_{s<=t} kappa_h v_s /
 * (sum_{s<=t} kappa_h + c eps) -- the p = 1 weights of [N] §2.6 with kappa/c, written in raw units.  Rows as in
 * oracle_attention_direct. */
void oracle_attention_direct_h(const double* q, const double* k, const double* v, int T, int d, int dv, int nh,
                               const double* omega, double gamma, double lambda_base, double c, double eps,
                               const int* rows, int n_rows, double* out) {
  const int n_out = rows ? n_rows : T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < n_out; j++) {
    const int t = rows ? rows[j] : j;
    double* o = out + (size_t)j * dv;
    double* num = (double*)calloc((size_t)dv, sizeof(double));
    double den = 0.0;
    for (int s = 0; s <= t; s++) {
      const double w = oracle_kappa_h(q + (size_t)t * d, k + (size_t)s * d, d, nh, t, s, omega, gamma, lambda_base) / c;
      den += w;
      for (int n = 0; n < dv; n++) num[n] += w * v[(size_t)s * dv + n];
    }
    for (int n = 0; n < dv; n++) o[n] = num[n] / (den + eps);
    free(num);
  }
}

/* The p = 1 recurrence on Phi_h, one head (state S [(2+4nh)d][dv], z [(2+4nh)d] in/out), as oracle_recurrent. */
void oracle_recurrent_h(const double* q, const double* k, const double* v, int T, int d, int dv, int nh,
                        int64_t pos0, const double* omega, double gamma, double lambda_base, double c, double eps,
                        double* S, double* z, double* out) {
  const int D = (2 + 4 * nh) * d;
  double* fq = (double*)malloc(sizeof(double) * (size_t)D);
  double* fk = (double*)malloc(sizeof(double) * (size_t)D);
  for (int i = 0; i < T; i++) {
    oracle_features_h(k + (size_t)i * d, 1, d, nh, pos0 + i, omega, gamma, lambda_base, fk);
    for (int f = 0; f < D; f++) {
      z[f] += fk[f];
      for (int n = 0; n < dv; n++) S[(size_t)f * dv + n] += fk[f] * v[(size_t)i * dv + n];
    }
    if (!out) continue;
    oracle_features_h(q + (size_t)i * d, 1, d, nh, pos0 + i, omega, gamma, lambda_base, fq);
    double den = 0.0;
    for (int f = 0; f < D; f++) den += fq[f] * z[f];
    for (int n = 0; n < dv; n++) {
      double num = 0.0;
      for (int f = 0; f < D; f++) num += fq[f] * S[(size_t)f * dv + n];
      out[(size_t)i * dv + n] = num / (den + c * eps);
    }
  }
  free(fq);
  free(fk);
}

/*
 * Gradient of the direct form, one head: the derivatives of L = sum_t <g_t, o_t> (g = dout [T][dv], the
 * gradient arriving at the outputs) with respect to q, k [T][d], v [T][dv] and omega [d], for the weights
 * w(t,s) = (kappa(t,s)/c)^p of oracle_attention_direct.  Needed because omega is learned ([N] §2.2) and the
 * method is trained, p = 2 first, then adapted to p = 1 ([N] §4.1).  Plain chain rule through the definition:
 *   D_t = sum_{s<=t} w_ts + eps,  o_t = sum_{s<=t} w_ts v_s / D_t
 *   dL/dw_ts   = <g_t, v_s - o_t> / D_t                  dL/dv_s = sum_{t>=s} w_ts g_t / D_t
 *   dw/dkappa  = p kappa^(p-1) / c^p
 *   kappa_ts   = sum_a (1 + r_qa r_ka)(1 + cos x_a),  x_a = theta_qa - theta_ka + (t - s) lambda_a
 *   dkappa/dtheta_qa = -(1 + r_qa r_ka) sin x_a + r_ka (1 + cos x_a) r'(theta_qa)
 *   dkappa/dtheta_ka = +(1 + r_qa r_ka) sin x_a + r_qa (1 + cos x_a) r'(theta_ka)
 *   dkappa/domega_a  = r_ka (1 + cos x_a) r'(theta_qa) + r_qa (1 + cos x_a) r'(theta_ka)
 *   r'(theta)  = dr/dtheta = dr/domega = gamma (1 - r^2)(-sin(theta + omega) - cos(theta + omega))
 *   dtheta/du  = pi / (1 + |u|)^2    (theta is C^1 at u = 0, with this value there)
 * The query-side terms are summed over s <= t for each t, the key-side terms over t >= s for each s, in two
 * separate loops (each recomputes kappa), so that every output is summed by one thread in a fixed order.
 */
static double sanatan_root_slope(double theta, double omega, double gamma, double r) {
  return gamma * (1.0 - r * r) * (-sin(theta + omega) - cos(theta + omega));
}

void oracle_attention_direct_grad(const double* q, const double* k, const double* v, const double* g, int T, int d,
                                  int dv, const double* omega, double gamma, double lambda_base, double c,
                                  double eps, int p, double* dq, double* dk, double* dvv, double* domega) {
  const size_t Td = (size_t)T * d;
  double* thq = (double*)malloc(sizeof(double) * Td);
  double* thk = (double*)malloc(sizeof(double) * Td);
  double* rq = (double*)malloc(sizeof(double) * Td);
  double* rk = (double*)malloc(sizeof(double) * Td);
  double* sq = (double*)malloc(sizeof(double) * Td); /* r'(theta) of each query component */
  double* sk = (double*)malloc(sizeof(double) * Td);
  double* lam = (double*)malloc(sizeof(double) * (size_t)d);
  double* o = (double*)malloc(sizeof(double) * (size_t)T * dv);
  double* D = (double*)malloc(sizeof(double) * (size_t)T);
  double* dom_q = (double*)calloc(Td, sizeof(double)); /* per-query-row omega terms, summed at the end */
  double* dom_k = (double*)calloc(Td, sizeof(double));
  for (int a = 0; a < d; a++) lam[a] = sanatan_freq(a, d, lambda_base);
  for (size_t i = 0; i < Td; i++) {
    const int a = (int)(i % (size_t)d);
    thq[i] = sanatan_angle(q[i]);
    thk[i] = sanatan_angle(k[i]);
    rq[i] = sanatan_root(thq[i], omega[a], gamma);
    rk[i] = sanatan_root(thk[i], omega[a], gamma);
    sq[i] = sanatan_root_slope(thq[i], omega[a], gamma, rq[i]);
    sk[i] = sanatan_root_slope(thk[i], omega[a], gamma, rk[i]);
  }
  const double cp = pow(c, (double)p);
  /* kappa of one pair, from the tabulated angles and roots (the cosine of a difference, as in the forward) */
#define KAPPA_OF(t, s, out_kap)                                                                          \
  do {                                                                                                   \
    double acc_ = 0.0;                                                                                   \
    for (int a_ = 0; a_ < d; a_++) {                                                                     \
      const double x_ = thq[(size_t)(t) * d + a_] - thk[(size_t)(s) * d + a_] + (double)((t) - (s)) * lam[a_]; \
      acc_ += (1.0 + rq[(size_t)(t) * d + a_] * rk[(size_t)(s) * d + a_]) * (1.0 + cos(x_));            \
    }                                                                                                    \
    (out_kap) = acc_;                                                                                    \
  } while (0)

  /* forward rows: o_t and D_t */
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; t++) {
    double den = 0.0;
    double* ot = o + (size_t)t * dv;
    for (int n = 0; n < dv; n++) ot[n] = 0.0;
    for (int s = 0; s <= t; s++) {
      double kap;
      KAPPA_OF(t, s, kap);
      const double w = pow(kap, (double)p) / cp;
      den += w;
      for (int n = 0; n < dv; n++) ot[n] += w * v[(size_t)s * dv + n];
    }
    D[t] = den + eps;
    for (int n = 0; n < dv; n++) ot[n] /= D[t];
  }
  /* query side: dq and the query-side omega terms, one row t per iteration */
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; t++) {
    double* dth = (double*)calloc((size_t)d, sizeof(double));
    for (int s = 0; s <= t; s++) {
      double kap;
      KAPPA_OF(t, s, kap);
      double gv = 0.0;
      for (int n = 0; n < dv; n++) gv += g[(size_t)t * dv + n] * (v[(size_t)s * dv + n] - o[(size_t)t * dv + n]);
      const double G = gv / D[t] * (double)p * pow(kap, (double)(p - 1)) / cp;
      for (int a = 0; a < d; a++) {
        const size_t ti = (size_t)t * d + a, si = (size_t)s * d + a;
        const double x = thq[ti] - thk[si] + (double)(t - s) * lam[a];
        dth[a] += G * (-(1.0 + rq[ti] * rk[si]) * sin(x) + rk[si] * (1.0 + cos(x)) * sq[ti]);
        dom_q[ti] += G * rk[si] * (1.0 + cos(x)) * sq[ti];
      }
    }
    for (int a = 0; a < d; a++) {
      const double u = q[(size_t)t * d + a];
      dq[(size_t)t * d + a] = dth[a] * ORACLE_PI / ((1.0 + fabs(u)) * (1.0 + fabs(u)));
    }
    free(dth);
  }
  /* key side: dk, dv and the key-side omega terms, one row s per iteration */
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < T; s++) {
    double* dth = (double*)calloc((size_t)d, sizeof(double));
    double* dvs = dvv + (size_t)s * dv;
    for (int n = 0; n < dv; n++) dvs[n] = 0.0;
    for (int t = s; t < T; t++) {
      double kap;
      KAPPA_OF(t, s, kap);
      const double w = pow(kap, (double)p) / cp;
      double gv = 0.0;
      for (int n = 0; n < dv; n++) {
        gv += g[(size_t)t * dv + n] * (v[(size_t)s * dv + n] - o[(size_t)t * dv + n]);
        dvs[n] += w * g[(size_t)t * dv + n] / D[t];
      }
      const double G = gv / D[t] * (double)p * pow(kap, (double)(p - 1)) / cp;
      for (int a = 0; a < d; a++) {
        const size_t ti = (size_t)t * d + a, si = (size_t)s * d + a;
        const double x = thq[ti] - thk[si] + (double)(t - s) * lam[a];
        dth[a] += G * ((1.0 + rq[ti] * rk[si]) * sin(x) + rq[ti] * (1.0 + cos(x)) * sk[si]);
        dom_k[si] += G * rq[ti] * (1.0 + cos(x)) * sk[si];
      }
    }
    for (int a = 0; a < d; a++) {
      const double u = k[(size_t)s * d + a];
      dk[(size_t)s * d + a] = dth[a] * ORACLE_PI / ((1.0 + fabs(u)) * (1.0 + fabs(u)));
    }
    free(dth);
  }
#undef KAPPA_OF
  for (int a = 0; a < d; a++) {
    double acc = 0.0;
    for (int t = 0; t < T; t++) acc += dom_q[(size_t)t * d + a] + dom_k[(size_t)t * d + a];
    domega[a] = acc;
  }
  free(thq); free(thk); free(rq); free(rk); free(sq); free(sk); free(lam); free(o); free(D); free(dom_q);
  free(dom_k);
}

/* Number of threads OpenMP will use (reported next to oracle timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
