// backward_chunked.hip -- the p = 1 backward pass as chunked linear recurrences: the forward statistics, the
// feature gradients and dv, all in time linear in T.
//
// SANATAN reading notes, §2.7: at p = 1 the attention is the recurrence of an explicit feature map, and so is
// each of its gradients.  With the forward statistics Dn_t (denominator, epsilon included) and
// delta_t = <g_t, o_t> (g = dout), the gradient of kappa_ts is (<g_t, v_s> - delta_t) / Dn_t for s <= t, so
//   dPhi(q_t) = (S_t g_t - delta_t z_t) / Dn_t,   S_t = sum_{s<=t} Phi(k_s) v_s^T,  z_t = sum_{s<=t} Phi(k_s),
//   dPhi(k_s) = R_s v_s - r_s,  dv_s = R_s^T Phi(k_s),
//   R_s = sum_{t>=s} Phi(q_t) g_t^T / Dn_t,  r_s = sum_{t>=s} Phi(q_t) delta_t / Dn_t.
// Per 32-token chunk, with A[t][s] = <g_t, v_s> - delta_t and the masked scores P[t][s] = <Phi(q_t), Phi(k_s)>:
//   dPhi(q_t) = (S g_t - delta_t z + sum_{s<=t} A[t][s] Phi(k_s)) / Dn_t        (S, z: the keys before the chunk)
//   dPhi(k_s) = R v_s - r + sum_{t>=s} Phi(q_t) A[t][s] / Dn_t                  (R, r: the queries after it)
//   dv_s      = R^T Phi(k_s) + sum_{t>=s} P[t][s] g_t / Dn_t.
// The statistics come from the forward pass over the same chunks: Dn_t = Phi(q_t) . z + sum_{s<=t} P[t][s] + c eps
// and delta_t Dn_t = Phi(q_t) . (S g_t) + sum_{s<=t} P[t][s] <g_t, v_s>, where S g_t is the product dPhi(q_t)
// needs anyway.  Phi(Q) and Phi(K) are materialized (6d = 384 features, the call's element type).  The feature
// map's Jacobian is applied in the chunk kernels themselves: each wave owns 16 dims of every channel, so after a
// chunk a lane holds all channels' gradients of its token's 8 dims and writes du (and accumulates the omega
// gradient) without a dPhi array.
//
// Work split.  The chunks of all sequences form one list (sequence-major), cut into G ranges of equal length, one
// workgroup per range and direction; with fewer sequences than compute units G = min(CUs, chunks), so a range
// covers the tail of one sequence and the head of the next at most (two segments), otherwise G is the number of
// sequences and each range is one whole sequence.  For each of its segments the forward direction walks the
// chunks in order carrying S^T (as 32 x 32 accumulator tiles [value][feature]) and z, and writes the statistics;
// the reverse direction, launched after it, walks them backwards carrying R^T and r.  Four waves share a workgroup, wave w owning dims 16 w .. 16 w + 15 of every channel (three 32-feature
// tiles).  The dPhi products need no exchange between waves; the statistics and dv sum over all features, so
// their four partials meet in LDS in a fixed order.  R^T Phi(k) contracts over features, the other way round
// from R v, so each R^T tile also passes through a wave-private LDS tile read back transposed.  When ranges split
// sequences, an increments pass writes the own S and z of each range's last segment that does not end its
// sequence to the range's slot before the forward direction, and another the own R and r (which need the
// statistics) of each range's first segment that does not start its sequence before the reverse one; a segment
// starts from the sum of the slots of the ranges before it (forward) or after it (reverse) in its sequence, in a
// fixed order.
// Operands: bf16 32x32x16 MFMA (fp32 32x32x2 for fp32 inputs), fp32 accumulation.  With bf16 operands, A, the
// states S and R, and g / Dn in the update of R enter the products as their rounding plus the rounding of their
// residual: S g and delta z (R v and r) nearly cancel, so a single rounding would leave an error near the
// result's own size.  dv takes R once rounded (its terms do not cancel).
#include <atomic>

#include "feature_tiles.h"

namespace sanatan {
namespace {

constexpr int kBC = 32;  // chunk tokens
// bf16 operands that also enter as the rounding of their residual: the state R in dPhi(k) = R v - r, and the
// masked A tiles
constexpr bool kResidR = true, kResidA = true;

template <typename T>
struct CGeom {
  static constexpr int Fp = kF;                      // 384 features
  static constexpr int NFT = Fp / 32, NW = NFT / 4;  // feature tiles, per wave
  static constexpr int EL = 16 / (int)sizeof(T);      // elements per 16-byte piece
  static constexpr int KP = Fp + EL, VP = kDV + EL, RLP = kDV + EL, RP = 68;
  // bf16: Phi(Q) rows staged in LDS like Phi(K); fp32 reads them from global memory (the rows would not fit)
  static constexpr bool QLDS = sizeof(T) == 2;
  static constexpr int kt_b = kBC * KP * (int)sizeof(T);
  static constexpr int qt_b = QLDS ? kt_b : 0;
  static constexpr int v_b = kBC * VP * (int)sizeof(T);
  static constexpr int o_kt = 0, o_qt = o_kt + kt_b, o_vt = o_qt + qt_b, o_gt = o_vt + v_b, o_ht = o_gt + v_b;
  // bf16: g / Dn is staged as its rounding (o_ht) and the rounding of its residual (o_hl)
  static constexpr int hl_b = sizeof(T) == 2 ? v_b : 0;
  static constexpr int o_hl = o_ht + v_b;
  static constexpr int o_st = o_hl + hl_b;         // 1 / Dn, delta, delta / Dn of the chunk's tokens
  static constexpr int o_zs = o_st + 3 * kBC * 4;  // z (forward) or r (reverse) [Fp]
  static constexpr int o_rl = o_zs + Fp * 4;       // per wave: one packed R^T tile as [32 features][RLP]
  static constexpr int rl_b = 4 * 32 * RLP * (int)sizeof(T);
  static constexpr int o_red = o_rl + rl_b;        // dv partials [4 waves][32 keys][RP]
  static constexpr int lds = o_red + 4 * kBC * RP * 4;
  static constexpr size_t SLOT = (size_t)Fp * kDV + Fp;  // one state: the tiles, then the vector
  static_assert(kBC * (Fp / EL) % 256 == 0 && kBC * (kDV / EL) % 256 == 0, "whole pieces per thread");
  static_assert(o_st % 16 == 0 && o_rl % 16 == 0 && o_red % 16 == 0, "aligned LDS regions");
};

// Ranges (workgroups per launch): with at least as many sequences as compute units one per sequence, otherwise
// one per compute unit (at most one per chunk).  G >= BH, so a range never spans more than two sequences.
int bwd_ranges(int B, int H, int Tn) {
  const long long BH = (long long)B * H, total = BH * ((Tn + kBC - 1) / kBC);
  long long G = device_cus();
  if (G <= BH) return (int)BH;
  return (int)(G < total ? G : total);
}

// The range a workgroup runs: workgroups are dealt round-robin to the 8 XCDs, so consecutive ranges (the segments
// of one sequence, which read each other's slots) go to workgroups on one XCD.  A bijection on [0, NR).
__device__ __forceinline__ int bwd_range_of_block(int NR) {
  const int b = (int)blockIdx.x, per = NR / 8;
  return b < 8 * per ? (b % 8) * per + b / 8 : b;
}

// 16 bytes of T scaled by s (hi), and for bf16 the rounding of what that rounding dropped (lo)
template <typename T>
__device__ __forceinline__ void scale16(const u32x4& x, float s, u32x4& hi, u32x4& lo) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, x);
    bf16x8 b, c;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float y = (float)a[i] * s;
      b[i] = (__bf16)y;
      c[i] = (__bf16)(y - (float)b[i]);
    }
    hi = __builtin_bit_cast(u32x4, b);
    lo = __builtin_bit_cast(u32x4, c);
  } else {
    const f32x4 a = __builtin_bit_cast(f32x4, x);
    const f32x4 b = {a[0] * s, a[1] * s, a[2] * s, a[3] * s};
    hi = __builtin_bit_cast(u32x4, b);
    lo = hi;
  }
}

// Internal feature order (LDS tiles, states, slots): dims in blocks of 16, each block's 6 channels together, so
// that wave w owns dims 16 w .. 16 w + 15 of every channel as its tiles 3 w, 3 w + 1, 3 w + 2 (tile j: channels
// 2 j and 2 j + 1).  Internal feature 96 m + 32 j + 16 c' + a' is channel 2 j + c', dim 16 m + a'; the
// materialized features are channel-major (64 c + a).
__device__ __forceinline__ int fint(int fg) {
  const int c = fg >> 6, a = fg & 63;
  return 96 * (a >> 4) + 32 * (c >> 1) + 16 * (c & 1) + (a & 15);
}
__device__ __forceinline__ int fglob(int fi) {
  const int m = fi / 96, rem = fi % 96;
  return 64 * (2 * (rem >> 5) + ((rem >> 4) & 1)) + 16 * m + (fi & 15);
}

// One chunk's staged operands (tokens t0 .. t0 + nv - 1 of a sequence) held in registers between their global
// loads and their LDS stores, so that the next chunk's loads are in flight while the current one computes.
// Flags: Phi(K), Phi(Q) (staged for bf16 only), V, g, g / Dn, and the statistics of the chunk's tokens (1 / Dn,
// delta and delta / Dn).  Rows past nv are stored as zeros (statistics too); rows are clamped into the
// sequence before they are read.  A workgroup-uniform mask can skip the feature rows (kq: Phi(K) and V; qq:
// Phi(Q) and g / Dn).
template <typename T, bool SK, bool SQ, bool SV, bool SG, bool SH, bool SS = true>
struct ChunkRegs {
  using G = CGeom<T>;
  static constexpr int EL = G::EL, FPC = G::Fp / EL, VPC = kDV / EL;
  static constexpr int NF = kBC * FPC / 256, NV = kBC * VPC / 256;
  static constexpr bool LQ = SQ && G::QLDS, LG = SG || SH;
  u32x4 k[SK ? NF : 1], q[LQ ? NF : 1], vv[SV ? NV : 1], gg[LG ? NV : 1];
  float dn_row[SH ? NV : 1];
  float2 st;
  int t0, nv;

  __device__ __forceinline__ void load(const T* kp, const T* qp, const T* vp, const T* gp, const float2* sp, int t0_,
                                       int nv_, int tid, bool kq = true, bool qq = true) {
    t0 = t0_;
    nv = nv_;
    if (SS && tid < kBC) st = sp[t0 + min(tid, nv - 1)];
#pragma unroll
    for (int i = 0; i < NF; i++) {
      const int e = tid + 256 * i, s = e / FPC, c = (e % FPC) * EL;
      const size_t off = (size_t)(t0 + min(s, nv - 1)) * G::Fp + c;
      if (SK && kq) k[i] = *reinterpret_cast<const u32x4*>(kp + off);
      if (LQ && qq) q[i] = *reinterpret_cast<const u32x4*>(qp + off);
    }
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int e = tid + 256 * i, s = e / VPC, c = (e % VPC) * EL;
      const int row = t0 + min(s, nv - 1);
      const size_t off = (size_t)row * kDV + c;
      if (SV && kq) vv[i] = *reinterpret_cast<const u32x4*>(vp + off);
      if (LG && (SG || qq)) gg[i] = *reinterpret_cast<const u32x4*>(gp + off);
      if (SH && qq) dn_row[i] = sp[row].x;
    }
  }

  __device__ __forceinline__ void store(char* smem, int tid, bool kq = true, bool qq = true) const {
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    if (SS && tid < kBC) {
      float* sl = reinterpret_cast<float*>(smem + G::o_st);
      const bool ok = tid < nv;
      const float inv = ok ? rcp_hw(st.x) : 0.0f, dl = ok ? st.y : 0.0f;
      sl[tid] = inv;
      sl[kBC + tid] = dl;
      sl[2 * kBC + tid] = dl * inv;
    }
    T* KT = reinterpret_cast<T*>(smem + G::o_kt);
    T* QT = reinterpret_cast<T*>(smem + G::o_qt);
#pragma unroll
    for (int i = 0; i < NF; i++) {
      const int e = tid + 256 * i, s = e / FPC, c = (e % FPC) * EL;
      const int ci = fint(c);
      if (SK && kq) *reinterpret_cast<u32x4*>(KT + s * G::KP + ci) = s < nv ? k[i] : zero4;
      if (LQ && qq) *reinterpret_cast<u32x4*>(QT + s * G::KP + ci) = s < nv ? q[i] : zero4;
    }
    T* VT = reinterpret_cast<T*>(smem + G::o_vt);
    T* GT = reinterpret_cast<T*>(smem + G::o_gt);
    T* HT = reinterpret_cast<T*>(smem + G::o_ht);
    T* HL = reinterpret_cast<T*>(smem + G::o_hl);
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int e = tid + 256 * i, s = e / VPC, c = (e % VPC) * EL;
      const bool ok = s < nv;
      if (SV && kq) *reinterpret_cast<u32x4*>(VT + s * G::VP + c) = ok ? vv[i] : zero4;
      if (SG) *reinterpret_cast<u32x4*>(GT + s * G::VP + c) = ok ? gg[i] : zero4;
      if (SH && qq) {
        u32x4 hi, lo;
        scale16<T>(gg[i], rcp_hw(dn_row[i]), hi, lo);
        *reinterpret_cast<u32x4*>(HT + s * G::VP + c) = ok ? hi : zero4;
        if constexpr (sizeof(T) == 2) *reinterpret_cast<u32x4*>(HL + s * G::VP + c) = ok ? lo : zero4;
      }
    }
  }
};

// A state slot in the accumulator's own order: tile (w, i, vt), register r, lane l at
// (((w NW + i) 2 + vt) 16 + r) 64 + l, then the feature vector [Fp].
template <typename T>
__device__ __forceinline__ void slot_add(const float* sl, f32x16 (&A)[CGeom<T>::NW][2], float* vec, int w, int l,
                                         int tid) {
  constexpr int NW = CGeom<T>::NW;
#pragma unroll
  for (int i = 0; i < NW; i++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int r = 0; r < 16; r++) A[i][vt][r] += sl[((size_t)((w * NW + i) * 2 + vt) * 16 + r) * 64 + l];
  for (int f = tid; f < kF; f += 256) vec[f] += sl[(size_t)kF * kDV + f];
}
template <typename T>
__device__ __forceinline__ void slot_put(float* sl, const f32x16 (&A)[CGeom<T>::NW][2], const float* vec, int w,
                                         int l, int tid) {
  constexpr int NW = CGeom<T>::NW;
#pragma unroll
  for (int i = 0; i < NW; i++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int r = 0; r < 16; r++) sl[((size_t)((w * NW + i) * 2 + vt) * 16 + r) * 64 + l] = A[i][vt][r];
  for (int f = tid; f < kF; f += 256) sl[(size_t)kF * kDV + f] = vec[f];
}

// Feature fragment of Phi(Q) with tokens along K (lane row = internal feature col0 + l % 32): from the LDS tile
// (bf16) or from global memory (fp32)
template <typename T>
__device__ __forceinline__ typename FragT<T>::type q_tokfrag(const char* smem, const T* qp, int t0, int tok0,
                                                             int col0, int l, int tmax) {
  using G = CGeom<T>;
  if constexpr (G::QLDS) {
    return lds_tokfrag(reinterpret_cast<const T*>(smem + G::o_qt), G::KP, tok0, col0, l);
  } else {
    return gtok_frag(qp, G::Fp, t0 + tok0, fglob(col0 + (l & 31)), l, tmax);
  }
}

// The feature map's Jacobian for this lane's token and its 8 dims 16 w + 8 hb + 4 h + e: gch[k - 1][hb][e] holds
// the gradient of feature channel k (1 .. 5).  Writes du (element type T) and adds the omega gradients to dom.
template <typename T>
__device__ __forceinline__ void lane_vjp(const float (&gch)[5][2][4], const float (&u)[2][4], const float (&rh)[2][4],
                                         const float (&om4)[2][4], float kr, T* du_row, float (&dom)[2][4]) {
#pragma unroll
  for (int hb = 0; hb < 2; hb++) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float dm;
      feature_vjp(u[hb][e], rh[hb][e], om4[hb][e], kr, gch[0][hb][e], gch[1][hb][e], gch[2][hb][e], gch[3][hb][e],
                  gch[4][hb][e], o[e], dm);
      dom[hb][e] += dm;
    }
    if constexpr (sizeof(T) == 2) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; e++) ov[e] = (__bf16)o[e];
      *reinterpret_cast<bf16x4*>(du_row + 8 * hb) = ov;
    } else {
      *reinterpret_cast<float4*>(du_row + 8 * hb) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

// This lane's raw components (8 dims, as lane_vjp) and their phases, for token row t of the sequence
template <typename T>
__device__ __forceinline__ void lane_inputs(const T* up, const float* rho, int t, int a0, float (&u)[2][4],
                                            float (&rh)[2][4]) {
#pragma unroll
  for (int hb = 0; hb < 2; hb++) {
    float x[4];
    load4(up + (size_t)t * kD + a0 + 8 * hb, x);
    const float4 r4 = *reinterpret_cast<const float4*>(rho + (size_t)t * kD + a0 + 8 * hb);
#pragma unroll
    for (int e = 0; e < 4; e++) u[hb][e] = x[e];
    rh[hb][0] = r4.x; rh[hb][1] = r4.y; rh[hb][2] = r4.z; rh[hb][3] = r4.w;
  }
}

// This lane's 8 omega partials summed over the 32 lanes of its half (fixed order), stored by lane 0 of the half
__device__ __forceinline__ void store_dom(float (&dom)[2][4], float* part, int a0, int n32) {
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float x = dom[hb][e];
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) x += __shfl_xor(x, off);
      if (n32 == 0) part[a0 + 8 * hb + e] = x;
    }
}

// The increments pass: the own S^T and z of the range's last segment if it does not end its sequence (MODE 1,
// before the forward direction), or the own R^T and r of its first segment if it does not start its sequence
// (MODE 2, after it: they need the statistics the forward direction writes), to the range's slot.
// Two register sets alternate, so each chunk's rows are loaded two chunks ahead of their use: the per-chunk work
// here is short, and one chunk of lead does not cover the loads' latency.
template <typename T, int MODE>
__global__ __launch_bounds__(256, 1) void bwd_incr_kernel(const T* __restrict__ phiq, const T* __restrict__ phik,
                                                          const T* __restrict__ v, const T* __restrict__ g,
                                                          const float2* __restrict__ stats, int Tn, int nch,
                                                          int BH, int NR, float* __restrict__ slots) {
  using G = CGeom<T>;
  typedef typename FragT<T>::type Frag;
  constexpr int NW = G::NW, Fp = G::Fp;
  constexpr bool DS = MODE == 1, DR = MODE == 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  const int rg = bwd_range_of_block(NR);
  const long long total = (long long)BH * nch, lo = range_lo(rg, total, NR), hi = range_lo(rg + 1, total, NR);
  int bh, t_lo, t_hi;
  if constexpr (DS) {  // the last segment, unless it ends its sequence
    bh = (int)((hi - 1) / nch);
    const long long seq0 = (long long)bh * nch;
    if (hi == seq0 + nch) return;
    t_lo = (int)((lo > seq0 ? lo : seq0) - seq0) * kBC;
    t_hi = (int)(hi - seq0) * kBC;
  } else {  // the first segment, unless it starts its sequence
    bh = (int)(lo / nch);
    const long long seq0 = (long long)bh * nch;
    if (lo == seq0) return;
    t_lo = (int)(lo - seq0) * kBC;
    t_hi = min(Tn, (int)((hi < seq0 + nch ? hi : seq0 + nch) - seq0) * kBC);
  }
  const size_t so = (size_t)bh * Tn;
  const T* qp = phiq + so * Fp;
  const T* kp = phik + so * Fp;
  const T* vp = v + so * kDV;
  const T* gp = g + so * kDV;
  const float2* sp = stats + so;
  const T* KT = reinterpret_cast<const T*>(smem + G::o_kt);
  const T* VT = reinterpret_cast<const T*>(smem + G::o_vt);
  const T* HT = reinterpret_cast<const T*>(smem + G::o_ht);
  const T* HL = reinterpret_cast<const T*>(smem + G::o_hl);
  const float* dh = reinterpret_cast<const float*>(smem + G::o_st) + 2 * kBC;
  float* vs = reinterpret_cast<float*>(smem + G::o_zs);  // z (MODE 1) or r (MODE 2)
  f32x16 A[NW][2];  // S^T or R^T tiles
#pragma unroll
  for (int i = 0; i < NW; i++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++) zero16(A[i][vt]);
  for (int f = tid; f < Fp; f += 256) vs[f] = 0.0f;
  auto compute = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int ft = 3 * w + i;
      float sum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        if constexpr (DS) {
          const Frag KF = lds_tokfrag(KT, G::KP, 16 * ks, 32 * ft, l);
          sum = frag_sum(KF, sum);
#pragma unroll
          for (int vt = 0; vt < 2; vt++) mma32(A[i][vt], lds_tokfrag(VT, G::VP, 16 * ks, 32 * vt, l), KF);
        } else {
          const Frag QF = q_tokfrag<T>(smem, qp, t0, 16 * ks, 32 * ft, l, Tn - 1);
#pragma unroll
          for (int e = 0; e < 8; e++) sum = fmaf((float)QF[e], dh[16 * ks + 8 * (e >> 2) + 4 * h + (e & 3)], sum);
#pragma unroll
          for (int vt = 0; vt < 2; vt++) {
            mma32(A[i][vt], lds_tokfrag(HT, G::VP, 16 * ks, 32 * vt, l), QF);
            if constexpr (sizeof(T) == 2) mma32(A[i][vt], lds_tokfrag(HL, G::VP, 16 * ks, 32 * vt, l), QF);
          }
        }
      }
      sum = xor32_sum(sum);
      if (h == 0) vs[32 * ft + n32] += sum;
    }
  };
  // MODE 1 stages Phi(K) and V; MODE 2 Phi(Q) (bf16), g / Dn and the statistics
  ChunkRegs<T, DS, DR, DS, false, DR, DR> R0, R1;
  const int sc = (t_hi - t_lo + kBC - 1) / kBC;
  auto nvof = [&](int c) { return min(kBC, t_hi - t_lo - c * kBC); };
  R0.load(kp, qp, vp, gp, sp, t_lo, nvof(0), tid);
  if (sc > 1) R1.load(kp, qp, vp, gp, sp, t_lo + kBC, nvof(1), tid);
  for (int c = 0; c < sc; c += 2) {
    R0.store(smem, tid);
    __syncthreads();
    if (c + 2 < sc) R0.load(kp, qp, vp, gp, sp, t_lo + (c + 2) * kBC, nvof(c + 2), tid);
    compute(t_lo + c * kBC);
    __syncthreads();
    if (c + 1 < sc) {
      R1.store(smem, tid);
      __syncthreads();
      if (c + 3 < sc) R1.load(kp, qp, vp, gp, sp, t_lo + (c + 3) * kBC, nvof(c + 3), tid);
      compute(t_lo + (c + 1) * kBC);
      __syncthreads();
    }
  }
  slot_put<T>(slots + (size_t)rg * G::SLOT, A, vs, w, l, tid);
}

// Method inputs of the fused Jacobian: the raw q and k, the phase table, the root anchors and kr.
struct JacArgs {
  const void* uq;
  const void* uk;
  const float* rho;
  const float* omega;
  int nph, H;
  float kr;
};

// Forward direction: the statistics and dq of one segment (tokens [t_lo, t_hi) of sequence bh, starting from the
// sum of the S slots of ranges [g0, g1)), and its omega partials (dom_row).  The
// statistics come out of the same pass: with W_t = S g_t (S before the chunk, the product that dPhi(q) needs
// anyway) and the chunk's scores P,
//   Dn_t = Phi(q_t) . z + sum_{s<=t} P[t][s] + c eps,   delta_t Dn_t = Phi(q_t) . W_t + sum_{s<=t} P[t][s] <g_t, v_s>,
// each wave summing over its features and the four partials meeting in LDS in a fixed order.  They are written
// to stats for the reverse direction.
template <typename T>
__device__ __forceinline__ void dq_piece(int bh, int t_lo, int t_hi, int g0, int g1, const T* __restrict__ phiq,
                                         const T* __restrict__ phik, const T* __restrict__ v,
                                         const T* __restrict__ g, float2* __restrict__ stats, int Tn, float ceps,
                                         const float* __restrict__ sslots, const JacArgs& ja, T* __restrict__ dq,
                                         float* __restrict__ dom_row, char* smem) {
  using G = CGeom<T>;
  typedef typename FragT<T>::type Frag;
  constexpr int NW = G::NW, Fp = G::Fp;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  const size_t so = (size_t)bh * Tn;
  const T* qp = phiq + so * Fp;
  const T* kp = phik + so * Fp;
  const T* vp = v + so * kDV;
  const T* gp = g + so * kDV;
  float2* sp = stats + so;
  const T* uq = static_cast<const T*>(ja.uq) + so * kD;
  T* dqp = dq + so * kD;
  const int da = 16 * w + 4 * h;  // this lane's dims da + 8 hb + e
  float om4[2][4], dom[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      om4[hb][e] = anchor_rev(ja.omega[(size_t)((bh % ja.H) % ja.nph) * kD + da + 8 * hb + e]);
      dom[hb][e] = 0.0f;
    }
  const T* KT = reinterpret_cast<const T*>(smem + G::o_kt);
  const T* QT = reinterpret_cast<const T*>(smem + G::o_qt);
  const T* VT = reinterpret_cast<const T*>(smem + G::o_vt);
  const T* GT = reinterpret_cast<const T*>(smem + G::o_gt);
  float* zs = reinterpret_cast<float*>(smem + G::o_zs);
  float4* part = reinterpret_cast<float4*>(smem + G::o_red);  // [4 waves][32 queries] statistics partials
  // S^T tiles: tile (i, vt) holds S[32 ft + n32][32 vt + 8 j + 4 h + i4] in register 4 j + i4, ft = 3 w + i
  f32x16 ST[NW][2];
#pragma unroll
  for (int i = 0; i < NW; i++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++) zero16(ST[i][vt]);
  for (int f = tid; f < Fp; f += 256) zs[f] = 0.0f;
  for (int q = g0; q < g1; q++) slot_add<T>(sslots + (size_t)q * G::SLOT, ST, zs, w, l, tid);
  ChunkRegs<T, true, true, true, true, false, false> R;
  R.load(kp, qp, vp, gp, nullptr, t_lo, min(kBC, t_hi - t_lo), tid);
  for (int t0 = t_lo; t0 < t_hi; t0 += kBC) {
    const int nv = R.nv;
    R.store(smem, tid);
    __syncthreads();
    if (t0 + kBC < t_hi) R.load(kp, qp, vp, gp, nullptr, t0 + kBC, min(kBC, t_hi - t0 - kBC), tid);
    // this lane's query t = n32
    float u[2][4], rh[2][4], gch[5][2][4];
    lane_inputs<T>(uq, ja.rho, t0 + min(n32, nv - 1), da, u, rh);
    const T* qrow = G::QLDS ? QT + n32 * G::KP : qp + (size_t)min(t0 + n32, Tn - 1) * Fp;
    // <g_t, v_s> and this wave's part of the scores, as accumulators [s][t]
    f32x16 acc, sc;
    zero16(acc);
    zero16(sc);
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
      mma32(acc, slot_frag<T>(VT + n32 * G::VP, 16 * kk, h), slot_frag<T>(GT + n32 * G::VP, 16 * kk, h));
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        const int base = 32 * (3 * w + i) + 16 * kk;
        mma32(sc, slot_frag<T>(KT + n32 * G::KP, base, h), slot_frag<T>(qrow, G::QLDS ? base : fglob(base), h));
      }
    // W = S g over this wave's tiles, as [feature][query]
    f32x16 d[NW];
#pragma unroll
    for (int i = 0; i < NW; i++) {
      zero16(d[i]);
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
          float x[8];
#pragma unroll
          for (int s = 0; s < 8; s++) x[s] = ST[i][vt][8 * kk + s];
          const Frag SF = pack8f<T>(x), GF = slot_frag<T>(GT + n32 * G::VP, 32 * vt + 16 * kk, h);
          mma32(d[i], SF, GF);
          if constexpr (sizeof(T) == 2) mma32(d[i], residual8<T>(x, SF), GF);
        }
    }
    // this wave's parts of Phi(q) . W, Phi(q) . z, sum_s P and sum_s P <g, v>
    float pw = 0.0f, pz = 0.0f, ps = 0.0f, pg = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int f0 = 32 * (3 * w + i) + 8 * j + 4 * h;
        float qv[4];
        load4(qrow + (G::QLDS ? f0 : fglob(f0)), qv);
        const float4 z4 = *reinterpret_cast<const float4*>(zs + f0);
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          pw = fmaf(qv[e], d[i][4 * j + e], pw);
          pz = fmaf(qv[e], zz[e], pz);
        }
      }
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int s = 8 * (r >> 2) + 4 * h + (r & 3);
      if (s <= n32) {
        ps += sc[r];
        pg = fmaf(sc[r], acc[r], pg);
      }
    }
    pw = xor32_sum(pw);
    pz = xor32_sum(pz);
    ps = xor32_sum(ps);
    pg = xor32_sum(pg);
    if (h == 0) part[w * kBC + n32] = make_float4(pw, pz, ps, pg);
    __syncthreads();
    float4 tot = part[n32];
#pragma unroll
    for (int ww = 1; ww < 4; ww++) {
      const float4 x = part[ww * kBC + n32];
      tot = make_float4(tot.x + x.x, tot.y + x.y, tot.z + x.z, tot.w + x.w);
    }
    const float dn = (tot.y + tot.z) + ceps, inv = rcp_hw(dn), dlt = (tot.x + tot.w) * inv;
    if (w == 0 && h == 0 && n32 < nv) sp[t0 + n32] = make_float2(dn, dlt);
    // A[t][s] = <g_t, v_s> - delta_t over s <= t, as accumulator [s][t]
    float a0[8], a1[8];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int s = 8 * (r >> 2) + 4 * h + (r & 3);
      const float x = s <= n32 ? acc[r] - dlt : 0.0f;
      if (r < 8) a0[r] = x;
      else a1[r - 8] = x;
    }
    const Frag A0 = pack8f<T>(a0), A1 = pack8f<T>(a1);
    Frag R0 = A0, R1 = A1;
    if constexpr (sizeof(T) == 2 && kResidA) R0 = residual8<T>(a0, A0), R1 = residual8<T>(a1, A1);
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int ft = 3 * w + i;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const Frag KF = lds_tokfrag(KT, G::KP, 16 * ks, 32 * ft, l);
        mma32(d[i], KF, ks ? A1 : A0);
        if constexpr (sizeof(T) == 2 && kResidA) mma32(d[i], KF, ks ? R1 : R0);
      }
      // dPhi(q): internal row 8 j + 4 h + e of tile i is channel 2 i + (j >> 1), dim da + 8 (j & 1) + e
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int c = 2 * i + (j >> 1);
        if (c == 0) continue;  // the constant feature has no Jacobian
        const float4 z4 = *reinterpret_cast<const float4*>(zs + 32 * ft + 8 * j + 4 * h);
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) gch[c - 1][j & 1][e] = (d[i][4 * j + e] - dlt * zz[e]) * inv;
      }
    }
    if (n32 < nv) lane_vjp<T>(gch, u, rh, om4, ja.kr, dqp + (size_t)(t0 + n32) * kD + da, dom);
    // S += Phi(K)^T V and z += Phi(K)^T 1 over this wave's tiles (each wave reads and updates its own z entries)
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int ft = 3 * w + i;
      float zsum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const Frag KF = lds_tokfrag(KT, G::KP, 16 * ks, 32 * ft, l);
        zsum = frag_sum(KF, zsum);
#pragma unroll
        for (int vt = 0; vt < 2; vt++) mma32(ST[i][vt], lds_tokfrag(VT, G::VP, 16 * ks, 32 * vt, l), KF);
      }
      zsum = xor32_sum(zsum);
      if (h == 0) zs[32 * ft + n32] += zsum;
    }
    __syncthreads();  // the next chunk's staging overwrites the tiles and the statistics partials
  }
  store_dom(dom, dom_row, da, n32);
}

// Reverse direction: dk and dv of one segment (tokens [t_lo, t_hi) of sequence bh, starting from the sum of the R
// slots of ranges [g0, g1), the farthest first), and its omega partials (dom_row).
template <typename T>
__device__ __forceinline__ void dkv_piece(int bh, int t_lo, int t_hi, int g0, int g1, const T* __restrict__ phiq,
                                          const T* __restrict__ phik, const T* __restrict__ v,
                                          const T* __restrict__ g, const float2* __restrict__ stats, int Tn,
                                          const float* __restrict__ rslots, const JacArgs& ja, T* __restrict__ dk,
                                          T* __restrict__ dv, float* __restrict__ dom_row, char* smem) {
  using G = CGeom<T>;
  typedef typename FragT<T>::type Frag;
  constexpr int NW = G::NW, Fp = G::Fp;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  const size_t so = (size_t)bh * Tn;
  const T* qp = phiq + so * Fp;
  const T* kp = phik + so * Fp;
  const T* vp = v + so * kDV;
  const T* gp = g + so * kDV;
  const float2* sp = stats + so;
  const T* uk = static_cast<const T*>(ja.uk) + so * kD;
  T* dkp = dk + so * kD;
  T* dvp = dv + so * kDV;
  const int da = 16 * w + 4 * h;  // this lane's dims da + 8 hb + e
  float om4[2][4], dom[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; hb++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      om4[hb][e] = anchor_rev(ja.omega[(size_t)((bh % ja.H) % ja.nph) * kD + da + 8 * hb + e]);
      dom[hb][e] = 0.0f;
    }
  const T* KT = reinterpret_cast<const T*>(smem + G::o_kt);
  const T* QT = reinterpret_cast<const T*>(smem + G::o_qt);
  const T* VT = reinterpret_cast<const T*>(smem + G::o_vt);
  const T* GT = reinterpret_cast<const T*>(smem + G::o_gt);
  const T* HT = reinterpret_cast<const T*>(smem + G::o_ht);
  const T* HL = reinterpret_cast<const T*>(smem + G::o_hl);
  const float* st = reinterpret_cast<const float*>(smem + G::o_st);
  float* rs = reinterpret_cast<float*>(smem + G::o_zs);
  T* RL = reinterpret_cast<T*>(smem + G::o_rl) + w * 32 * G::RLP;
  float* red = reinterpret_cast<float*>(smem + G::o_red);
  // R^T tiles: tile (i, vt) holds R[32 ft + n32][32 vt + 8 j + 4 h + i4] in register 4 j + i4, ft = w + 4 i
  f32x16 RT[NW][2];
#pragma unroll
  for (int i = 0; i < NW; i++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++) zero16(RT[i][vt]);
  for (int f = tid; f < Fp; f += 256) rs[f] = 0.0f;
  for (int q = g1 - 1; q >= g0; q--) slot_add<T>(rslots + (size_t)q * G::SLOT, RT, rs, w, l, tid);
  const int c_lo = t_lo / kBC, c_hi = (t_hi + kBC - 1) / kBC;
  ChunkRegs<T, true, true, true, true, true> R;
  R.load(kp, qp, vp, gp, sp, (c_hi - 1) * kBC, min(kBC, t_hi - (c_hi - 1) * kBC), tid);
  for (int c = c_hi - 1; c >= c_lo; c--) {
    const int t0 = c * kBC, nv = R.nv;
    R.store(smem, tid);
    __syncthreads();
    if (c > c_lo) R.load(kp, qp, vp, gp, sp, t0 - kBC, kBC, tid);
    // this lane's key s = n32.  <g_t, v_s> and this wave's part of the scores, as accumulators [t][s]
    float u[2][4], rh[2][4], gch[5][2][4];
    lane_inputs<T>(uk, ja.rho, t0 + min(n32, nv - 1), da, u, rh);
    f32x16 gv, sc;
    zero16(gv);
    zero16(sc);
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
      mma32(gv, slot_frag<T>(GT + n32 * G::VP, 16 * kk, h), slot_frag<T>(VT + n32 * G::VP, 16 * kk, h));
    const T* qrow = G::QLDS ? QT + n32 * G::KP : qp + (size_t)min(t0 + n32, Tn - 1) * Fp;
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        const int base = 32 * (3 * w + i) + 16 * kk;
        mma32(sc, slot_frag<T>(qrow, G::QLDS ? base : fglob(base), h), slot_frag<T>(KT + n32 * G::KP, base, h));
      }
    // A[t][s] / Dn_t and P[t][s] / Dn_t over t >= s (1 / Dn is zero past the chunk's end)
    float a0[8], a1[8], p0[8], p1[8];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int tb = 8 * j + 4 * h;
      const float4 inv4 = *reinterpret_cast<const float4*>(st + tb);
      const float4 dl4 = *reinterpret_cast<const float4*>(st + kBC + tb);
      const float inv[4] = {inv4.x, inv4.y, inv4.z, inv4.w}, dl[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int r = 4 * j + e;
        const bool keep = tb + e >= n32;
        const float x = keep ? (gv[r] - dl[e]) * inv[e] : 0.0f;
        const float y = keep ? sc[r] * inv[e] : 0.0f;
        if (r < 8) a0[r] = x, p0[r] = y;
        else a1[r - 8] = x, p1[r - 8] = y;
      }
    }
    const Frag A0 = pack8f<T>(a0), A1 = pack8f<T>(a1), P0 = pack8f<T>(p0), P1 = pack8f<T>(p1);
    Frag R0 = A0, R1 = A1;
    if constexpr (sizeof(T) == 2 && kResidA) R0 = residual8<T>(a0, A0), R1 = residual8<T>(a1, A1);
    // dv^T [value][key]: the chunk's queries, then R^T Phi(k) tile by tile below
    f32x16 dvt[2];
#pragma unroll
    for (int vt = 0; vt < 2; vt++) {
      zero16(dvt[vt]);
      mma32(dvt[vt], lds_tokfrag(GT, G::VP, 0, 32 * vt, l), P0);
      mma32(dvt[vt], lds_tokfrag(GT, G::VP, 16, 32 * vt, l), P1);
    }
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int ft = 3 * w + i;
      Frag RF[2][2];
      f32x16 d;  // dPhi(k) + r, as [feature][key]
      zero16(d);
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
          float x[8];
#pragma unroll
          for (int s = 0; s < 8; s++) x[s] = RT[i][vt][8 * kk + s];
          RF[vt][kk] = pack8f<T>(x);
          const Frag VF = slot_frag<T>(VT + n32 * G::VP, 32 * vt + 16 * kk, h);
          mma32(d, RF[vt][kk], VF);
          if constexpr (sizeof(T) == 2 && kResidR) mma32(d, residual8<T>(x, RF[vt][kk]), VF);
        }
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        const Frag QF = q_tokfrag<T>(smem, qp, t0, 16 * kt, 32 * ft, l, Tn - 1);
        mma32(d, QF, kt ? A1 : A0);
        if constexpr (sizeof(T) == 2 && kResidA) mma32(d, QF, kt ? R1 : R0);
      }
      // dPhi(k): internal row 8 j + 4 h + e of tile i is channel 2 i + (j >> 1), dim da + 8 (j & 1) + e
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int c = 2 * i + (j >> 1);
        if (c == 0) continue;  // the constant feature has no Jacobian
        const float4 r4 = *reinterpret_cast<const float4*>(rs + 32 * ft + 8 * j + 4 * h);
        const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) gch[c - 1][j & 1][e] = d[4 * j + e] - rr[e];
      }
      // the packed tile as R[feature][value] in this wave's LDS tile, read back with values along the rows
      // (the wave's LDS accesses complete in order, so no barrier is needed between the stores and the reads)
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
          T* dst = RL + n32 * G::RLP + 32 * vt + 16 * kk + 4 * h;
          if constexpr (sizeof(T) == 2) {
            const u32x4 wd = __builtin_bit_cast(u32x4, RF[vt][kk]);
            *reinterpret_cast<u32x2*>(dst) = (u32x2){wd[0], wd[1]};
            *reinterpret_cast<u32x2*>(dst + 8) = (u32x2){wd[2], wd[3]};
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(RF[vt][kk][0], RF[vt][kk][1], RF[vt][kk][2], RF[vt][kk][3]);
            *reinterpret_cast<float4*>(dst + 8) =
                make_float4(RF[vt][kk][4], RF[vt][kk][5], RF[vt][kk][6], RF[vt][kk][7]);
          }
        }
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
          mma32(dvt[vt], lds_tokfrag(RL, G::RLP, 16 * kk, 32 * vt, l),
                slot_frag<T>(KT + n32 * G::KP, 32 * ft + 16 * kk, h));
    }
    if (n32 < nv) lane_vjp<T>(gch, u, rh, om4, ja.kr, dkp + (size_t)(t0 + n32) * kD + da, dom);
    // the four waves' dv partials meet in LDS; summed in a fixed order
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        *reinterpret_cast<float4*>(red + (w * kBC + n32) * G::RP + 32 * vt + 8 * j + 4 * h) =
            make_float4(dvt[vt][4 * j], dvt[vt][4 * j + 1], dvt[vt][4 * j + 2], dvt[vt][4 * j + 3]);
    __syncthreads();
    {
      const int row = tid >> 3, c0 = 8 * (tid & 7);
      if (row < nv) {
        constexpr int WS = kBC * G::RP;
        const float* b0 = red + row * G::RP + c0;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] = ((b0[e] + b0[WS + e]) + b0[2 * WS + e]) + b0[3 * WS + e];
        T* dst = dvp + (size_t)(t0 + row) * kDV + c0;
        if constexpr (sizeof(T) == 2) {
          bf16x8 ov;
#pragma unroll
          for (int e = 0; e < 8; e++) ov[e] = (__bf16)o[e];
          *reinterpret_cast<bf16x8*>(dst) = ov;
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    }
    // R += Phi(Q)^T (G / Dn) and r += Phi(Q)^T (delta / Dn) with the chunk's queries (each wave reads and updates
    // its own r entries)
    const float* dh = st + 2 * kBC;
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int ft = 3 * w + i;
      float rsum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        const Frag QF = q_tokfrag<T>(smem, qp, t0, 16 * kt, 32 * ft, l, Tn - 1);
#pragma unroll
        for (int e = 0; e < 8; e++) rsum = fmaf((float)QF[e], dh[16 * kt + 8 * (e >> 2) + 4 * h + (e & 3)], rsum);
#pragma unroll
        for (int vt = 0; vt < 2; vt++) {
          mma32(RT[i][vt], lds_tokfrag(HT, G::VP, 16 * kt, 32 * vt, l), QF);
          if constexpr (sizeof(T) == 2) mma32(RT[i][vt], lds_tokfrag(HL, G::VP, 16 * kt, 32 * vt, l), QF);
        }
      }
      rsum = xor32_sum(rsum);
      if (h == 0) rs[32 * ft + n32] += rsum;
    }
    __syncthreads();  // the next chunk's staging overwrites the tiles and the reduction buffer
  }
  store_dom(dom, dom_row, da, n32);
}

// DIR 0: the forward direction (statistics, dq); DIR 1: the reverse one (dk, dv).  One workgroup per range, which
// runs its one or two segments in order; segment j of range r writes its omega partials to row (DIR NR + r) 2 + j
// of dom_part.
template <typename T, int DIR>
__global__ __launch_bounds__(256, 1) void bwd_chunk_kernel(const T* __restrict__ phiq, const T* __restrict__ phik,
                                                           const T* __restrict__ v, const T* __restrict__ g,
                                                           float2* __restrict__ stats, int Tn, int nch, int BH,
                                                           int NR, float ceps, const float* __restrict__ sslots,
                                                           const float* __restrict__ rslots, const JacArgs ja,
                                                           T* __restrict__ dq, T* __restrict__ dk,
                                                           T* __restrict__ dv, float* __restrict__ dom_part) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the range's one or two segments, as workgroup-uniform 32-bit values (kept in scalar registers, out of the way
  // of the chunk loop's vector registers): sequence bh0 chunks [a0, a1), then, if nseg = 2, sequence bh0 + 1
  // chunks [0, b1)
  const int rg = bwd_range_of_block(NR);
  const long long total = (long long)BH * nch, lo = range_lo(rg, total, NR), hi = range_lo(rg + 1, total, NR);
  const long long s0 = lo / nch * nch;
  const int bh0 = __builtin_amdgcn_readfirstlane((int)(lo / nch));
  const int a0 = __builtin_amdgcn_readfirstlane((int)(lo - s0));
  const int a1 = __builtin_amdgcn_readfirstlane((int)((hi < s0 + nch ? hi : s0 + nch) - s0));
  const int nseg = hi > s0 + nch ? 2 : 1;
  const int b1 = __builtin_amdgcn_readfirstlane((int)(hi - s0 - nch));
  // forward: the ranges before the first segment in its sequence (the second starts its sequence); reverse: the
  // ranges after the last segment in its sequence (the first ends its sequence when there is a second)
  const int pre = __builtin_amdgcn_readfirstlane(a0 > 0 ? range_of_chunk(s0, total, NR) : rg);
  const long long sl = nseg == 2 ? s0 + nch : s0;  // the last segment's sequence start
  const int c_last = nseg == 2 ? b1 : a1;
  const int post = __builtin_amdgcn_readfirstlane(c_last < nch ? range_of_chunk(sl + nch - 1, total, NR) + 1 : rg + 1);
  // (two inlined calls rather than a loop: each copy then keeps the registers of a single segment)
  float* drow = dom_part + (size_t)(DIR * NR + rg) * 2 * kD;
  if constexpr (DIR == 0)
    dq_piece<T>(bh0, a0 * kBC, min(Tn, a1 * kBC), pre, rg, phiq, phik, v, g, stats, Tn, ceps, sslots, ja, dq, drow,
                smem);
  else
    dkv_piece<T>(bh0, a0 * kBC, min(Tn, a1 * kBC), rg + 1, nseg == 2 ? rg + 1 : post, phiq, phik, v, g, stats, Tn,
                 rslots, ja, dk, dv, drow, smem);
  if (nseg == 2) {
    __syncthreads();  // the first segment's LDS tiles and vectors are dead
    if constexpr (DIR == 0)
      dq_piece<T>(bh0 + 1, 0, min(Tn, b1 * kBC), rg, rg, phiq, phik, v, g, stats, Tn, ceps, sslots, ja, dq,
                  drow + kD, smem);
    else
      dkv_piece<T>(bh0 + 1, 0, min(Tn, b1 * kBC), rg + 1, post, phiq, phik, v, g, stats, Tn, rslots, ja, dk, dv,
                   drow + kD, smem);
  }
}

// Per (side, sequence): the omega partials of the sequence's segments summed in range order (side 0: the dq
// rows, side 1: the dk rows), to seq_sum[side BH + bh].
__global__ __launch_bounds__(64) void bwd_domega_seg_kernel(const float* __restrict__ part, int nch, int BH, int NR,
                                                            float* __restrict__ seq_sum) {
  const int sb = blockIdx.x, side = sb / BH, bh = sb % BH, a = threadIdx.x;
  const long long total = (long long)BH * nch, seq0 = (long long)bh * nch;
  const int gf = range_of_chunk(seq0, total, NR), gl = range_of_chunk(seq0 + nch - 1, total, NR);
  float acc = 0.0f;
  for (int r = gf; r <= gl; r++) {
    const int j = (r == gf && range_lo(r, total, NR) < seq0) ? 1 : 0;  // the sequence is the range's second segment
    acc += part[((size_t)(side * NR + r) * 2 + j) * kD + a];
  }
  seq_sum[(size_t)sb * kD + a] = acc;
}

template <typename Kern>
hipError_t set_lds_attr(Kern k, int bytes, std::atomic<bool>& flag) {
  if (flag.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) flag.store(true, std::memory_order_release);
  return e;
}

template <typename T>
hipError_t launch_t(const void* phiq, const void* phik, const void* v, const void* g, float2* stats, int B, int H,
                    int Tn, float ceps, const JacArgs& ja, void* dq, void* dk, void* dv, float* seq_sum,
                    float* slots, hipStream_t stream) {
  using G = CGeom<T>;
  static std::atomic<bool> attr[4][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const int BH = B * H, nch = (Tn + kBC - 1) / kBC, NR = bwd_ranges(B, H, Tn);
  const bool split = NR > BH;  // ranges cut sequences: increments and slots
  float* sslots = slots;
  float* rslots = slots + (size_t)NR * G::SLOT;
  float* dom_part = slots + (split ? 2 * (size_t)NR * G::SLOT : 0);  // [2 sides][NR ranges][2 segments][d]
  const T* q = static_cast<const T*>(phiq);
  const T* k = static_cast<const T*>(phik);
  const T* vv = static_cast<const T*>(v);
  const T* gg = static_cast<const T*>(g);
  hipError_t e;
  if ((e = set_lds_attr(bwd_chunk_kernel<T, 0>, G::lds, attr[1][dev])) != hipSuccess ||
      (e = set_lds_attr(bwd_chunk_kernel<T, 1>, G::lds, attr[3][dev])) != hipSuccess)
    return e;
  if (split && ((e = set_lds_attr(bwd_incr_kernel<T, 1>, G::lds, attr[0][dev])) != hipSuccess ||
                (e = set_lds_attr(bwd_incr_kernel<T, 2>, G::lds, attr[2][dev])) != hipSuccess))
    return e;
  auto incr = [&](int mode) {
    if (mode == 1)
      hipLaunchKernelGGL((bwd_incr_kernel<T, 1>), dim3(NR), dim3(256), G::lds, stream, q, k, vv, gg, stats, Tn, nch,
                         BH, NR, sslots);
    else
      hipLaunchKernelGGL((bwd_incr_kernel<T, 2>), dim3(NR), dim3(256), G::lds, stream, q, k, vv, gg, stats, Tn, nch,
                         BH, NR, rslots);
    return hipGetLastError();
  };
  auto chunks = [&](int dir) {
    if (dir == 0)
      hipLaunchKernelGGL((bwd_chunk_kernel<T, 0>), dim3(NR), dim3(256), G::lds, stream, q, k, vv, gg, stats, Tn, nch,
                         BH, NR, ceps, sslots, rslots, ja, static_cast<T*>(dq), static_cast<T*>(dk),
                         static_cast<T*>(dv), dom_part);
    else
      hipLaunchKernelGGL((bwd_chunk_kernel<T, 1>), dim3(NR), dim3(256), G::lds, stream, q, k, vv, gg, stats, Tn, nch,
                         BH, NR, ceps, sslots, rslots, ja, static_cast<T*>(dq), static_cast<T*>(dk),
                         static_cast<T*>(dv), dom_part);
    return hipGetLastError();
  };
  // S increments, the forward direction (which writes the statistics), R increments, the reverse direction, and
  // the per-sequence omega sums
  if (split && (e = incr(1)) != hipSuccess) return e;
  if ((e = chunks(0)) != hipSuccess) return e;
  if (split && (e = incr(2)) != hipSuccess) return e;
  if ((e = chunks(1)) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_domega_seg_kernel, dim3(2 * BH), dim3(64), 0, stream, dom_part, nch, BH, NR, seq_sum);
  return hipGetLastError();
}

}  // namespace

// Slots (two states per range when ranges cut sequences), then the omega partial rows (two sides, two per range)
size_t bwd_chunked_slot_bytes(int B, int H, int T) {
  const size_t NR = bwd_ranges(B, H, T);
  const bool split = NR > (size_t)B * H;
  return ((split ? 2 * NR * CGeom<float>::SLOT : 0) + 4 * NR * kD) * sizeof(float);
}

hipError_t launch_bwd_chunked(const void* phiq, const void* phik, const void* v, const void* g, float2* stats,
                              sanatan_dtype t, int B, int H, int T, float ceps, const void* q, const void* k,
                              const float* rho, const float* omega, int nph, float kr, void* dq, void* dk, void* dv,
                              float* seq_sum, float* slots, hipStream_t stream) {
  const JacArgs ja{q, k, rho, omega, nph, H, kr};
  return t == SANATAN_BF16
             ? launch_t<__bf16>(phiq, phik, v, g, stats, B, H, T, ceps, ja, dq, dk, dv, seq_sum, slots, stream)
             : launch_t<float>(phiq, phik, v, g, stats, B, H, T, ceps, ja, dq, dk, dv, seq_sum, slots, stream);
}

}  // namespace sanatan
