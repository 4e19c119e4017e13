// quadratic.hip -- normalised causal power attention in masked quadratic form (p = 1 or 2).
//
// SANATAN reading notes §2.6: w_ts = (kappa_ts / c)^p for s <= t, o_t = sum w v_s / (sum w + eps);
// kappa_ts = <Phi(q_t), Phi(k_s)> (§2.3).  p = 2 has no small-state recurrence (§2.6, §4.1), so
// this is the training/parallel form.  Because 0 <= kappa <= 4d = c, every weight lies in [0, 1]
// and no running maximum is needed (unlike softmax): partial sums over key blocks just add.
//
// Phi(K) is featurized once into the workspace (element type of the call); each workgroup
// featurizes its own query rows straight into MFMA operand registers.  Per key block of 64
// keys: Phi(K) and V^T are staged in LDS, every wave forms the score tile transposed
// (rows = keys, cols = its query rows) so that the masked, powered tile is directly the A
// operand of w.V' (V' = [V | 1]: the fifth 16-column tile accumulates the denominator).
#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

template <typename T>
struct QuadGeom {
  static constexpr int MT = sizeof(T) == 2 ? 2 : 1;   // 16-row query tiles per wave
  static constexpr int QROWS = 4 * 16 * MT;           // query rows per workgroup
  static constexpr int KB = 64;                        // keys per block
  static constexpr int KPITCH = kF + 16 / (int)sizeof(T);
  static constexpr int VPITCH = KB + 16 / (int)sizeof(T);
  static constexpr size_t k_bytes = (size_t)KB * KPITCH * sizeof(T);
  static constexpr size_t v_bytes = (size_t)kDV * VPITCH * sizeof(T);
  static constexpr size_t lds = k_bytes + v_bytes;
};

template <typename T, int P>
__global__ __launch_bounds__(256, 1) void quadratic_kernel(const T* __restrict__ q, const T* __restrict__ phik,
                                                           const T* __restrict__ v, T* __restrict__ out,
                                                           const float* __restrict__ omega, int nph, int H, int Tn,
                                                           int BH, int nqb, int64_t pos0, double log2_base, float kr,
                                                           float inv_c, float eps) {
  using Gm = QuadGeom<T>;
  using Frag = typename FragT<T>::type;
  constexpr int MT = Gm::MT, KB = Gm::KB, KPITCH = Gm::KPITCH, VPITCH = Gm::VPITCH;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* Ks = reinterpret_cast<T*>(smem);                  // [KB][KPITCH]  Phi(K) block, token-major
  T* Vt = reinterpret_cast<T*>(smem + Gm::k_bytes);    // [64][VPITCH]  V^T block

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, qd = l >> 4;
  // heaviest (latest) query blocks first across all sequences
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int h = bh % H;
  const int row0 = qb * Gm::QROWS + w * 16 * MT;  // this wave's first query row
  const T* qp = q + (size_t)bh * Tn * kD;
  const T* kp = phik + (size_t)bh * Tn * kF;
  const T* vp = v + (size_t)bh * Tn * kDV;
  T* op = out + (size_t)bh * Tn * kDV;

  // Phi(Q) fragments, natural feature order: K-step j covers features 32j .. 32j+31 = channel j/2,
  // dims 32(j%2) + 8qd + i; this lane featurizes dims {8qd .. 8qd+7, 32+8qd .. 32+8qd+7}.
  Frag QF[MT][12];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const int t = row0 + 16 * mt + r;
    const bool valid = t < Tn;
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      float ch[6][8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int a = 32 * hh + 8 * qd + i;
        const float u = valid ? to_f32(qp[(size_t)t * kD + a]) : 0.0f;
        const float om4 = anchor_rev(omega[(size_t)(h % nph) * kD + a]);
        const float rho = phase_rev(pos0 + t, a, log2_base);
        float cr, sr, rr;
        featurize1(u, rho, om4, kr, cr, sr, rr);
        ch[0][i] = 1.0f;
        ch[1][i] = cr;
        ch[2][i] = sr;
        ch[3][i] = rr;
        ch[4][i] = rr * cr;
        ch[5][i] = rr * sr;
      }
#pragma unroll
      for (int c = 0; c < 6; c++) {
        float lo[4] = {ch[c][0], ch[c][1], ch[c][2], ch[c][3]}, hi[4] = {ch[c][4], ch[c][5], ch[c][6], ch[c][7]};
        QF[mt][2 * c + hh] = pack8<T>(lo, hi);
      }
    }
  }

  Frag ONES;
#pragma unroll
  for (int i = 0; i < 8; i++) ONES[i] = (T)(r == 0 ? 1.0f : 0.0f);
  f32x4 num[MT][5];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int nt = 0; nt < 5; nt++) num[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int last_row = min(Tn - 1, qb * Gm::QROWS + Gm::QROWS - 1);
  const int nkb = last_row / KB + 1;
  const int my_last = min(Tn - 1, row0 + 16 * MT - 1);
  for (int kb = 0; kb < nkb; kb++) {
    const int s0 = kb * KB;
    // stage Phi(K) rows s0 .. s0+63 (token-major) and V^T
    {
      constexpr int E = 16 / (int)sizeof(T);
      constexpr int PER_ROW = kF / E;
      for (int idx = tid; idx < KB * PER_ROW; idx += 256) {
        const int s = idx / PER_ROW, cpos = (idx % PER_ROW) * E;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (s0 + s < Tn) raw = *reinterpret_cast<const uint4*>(kp + (size_t)(s0 + s) * kF + cpos);
        *reinterpret_cast<uint4*>(Ks + s * KPITCH + cpos) = raw;
      }
      constexpr int TPT = kDV / E;
      const int n0 = (tid % TPT) * E;
      for (int s = tid / TPT; s < KB; s += 256 / TPT) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (s0 + s < Tn) raw = *reinterpret_cast<const uint4*>(vp + (size_t)(s0 + s) * kDV + n0);
        const T* rv = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < E; j++) Vt[(n0 + j) * VPITCH + s] = rv[j];
      }
    }
    __syncthreads();
    if (s0 <= my_last) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const int tq = row0 + 16 * mt;  // first row of this query tile
        if (s0 > tq + 15) continue;
        // score tiles transposed: D[sb] rows s = s0 + 16 sb + 4qd + i, cols t = tq + r
        f32x4 d[4];
#pragma unroll
        for (int sb = 0; sb < 4; sb++) {
          d[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (s0 + 16 * sb > tq + 15) continue;
#pragma unroll
          for (int j = 0; j < 12; j++) {
            Frag A;
            const T* pk = Ks + (16 * sb + r) * KPITCH + 32 * j + 8 * qd;
#pragma unroll
            for (int i = 0; i < 8; i++) A[i] = pk[i];
            mma(d[sb], A, QF[mt][j]);
          }
          // weight: (kappa / c)^p, masked s <= t
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int s = s0 + 16 * sb + 4 * qd + i;
            float wv = d[sb][i] * inv_c;
            if (P == 2) wv = wv * wv;
            d[sb][i] = (s > tq + r) ? 0.0f : wv;
          }
        }
#pragma unroll
        for (int m = 0; m < 2; m++) {
          if (s0 + 32 * m > tq + 15) continue;
          const Frag Pf = pack8v<T>(d[2 * m], d[2 * m + 1]);
#pragma unroll
          for (int nt = 0; nt < 4; nt++) {
            Frag B;
            const T* pv = Vt + (16 * nt + r) * VPITCH + 32 * m + 4 * qd;
#pragma unroll
            for (int i = 0; i < 4; i++) {
              B[i] = pv[i];
              B[4 + i] = pv[16 + i];
            }
            mma(num[mt][nt], Pf, B);
          }
          mma(num[mt][4], Pf, ONES);
        }
      }
    }
    __syncthreads();
  }

  // o = num / (den + eps); the denominator sits in column 0 of tile 4 (lanes r == 0).
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float den = __shfl(num[mt][4][i], l & 48);
      const int t = row0 + 16 * mt + 4 * qd + i;
      if (t < Tn) {
        const float inv = 1.0f / (den + eps);
#pragma unroll
        for (int nt = 0; nt < 4; nt++) op[(size_t)t * kDV + 16 * nt + r] = from_f32<T>(num[mt][nt][i] * inv);
      }
    }
  }
}

size_t quadratic_ws_bytes(int B, int H, int T, sanatan_dtype t) {
  const size_t el = (t == SANATAN_BF16) ? 2 : 4;
  return (size_t)B * H * T * kF * el;
}

template <typename T, int P>
static hipError_t launch_quad_t(const void* q, const void* k, const void* v, int B, int H, int Tn, int64_t pos0,
                                const MethodConsts& mc, void* out, void* ws, sanatan_dtype t, hipStream_t stream) {
  hipError_t e = launch_featurize(k, t, B, H, Tn, pos0, mc, ws, t, stream);
  if (e != hipSuccess) return e;
  using Gm = QuadGeom<T>;
  const int nqb = (Tn + Gm::QROWS - 1) / Gm::QROWS;
  const int BH = B * H;
  e = hipFuncSetAttribute((const void*)quadratic_kernel<T, P>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)Gm::lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quadratic_kernel<T, P>), dim3(BH * nqb), dim3(256), Gm::lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(ws), static_cast<const T*>(v),
                     static_cast<T*>(out), mc.omega, mc.nph, H, Tn, BH, nqb, pos0, mc.log2_base, mc.kr, mc.inv_c,
                     mc.eps);
  return hipGetLastError();
}

hipError_t launch_quadratic(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                            int p, int64_t pos0, const MethodConsts& mc, void* out, void* ws, hipStream_t stream) {
  if (t == SANATAN_BF16)
    return p == 1 ? launch_quad_t<__bf16, 1>(q, k, v, B, H, T, pos0, mc, out, ws, t, stream)
                  : launch_quad_t<__bf16, 2>(q, k, v, B, H, T, pos0, mc, out, ws, t, stream);
  return p == 1 ? launch_quad_t<float, 1>(q, k, v, B, H, T, pos0, mc, out, ws, t, stream)
                : launch_quad_t<float, 2>(q, k, v, B, H, T, pos0, mc, out, ws, t, stream);
}

}  // namespace sanatan
