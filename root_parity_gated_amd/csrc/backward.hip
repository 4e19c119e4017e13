// backward.hip -- gradient of normalised causal power attention (p = 1 or 2) with respect to q, k, v and the
// root anchors omega.
//
// SANATAN reading notes: omega is learned (§2.2, root equation) and the method is trained, p = 2 first and
// then adapted to p = 1 (§4.1); the weights are w_ts = (kappa_ts / c)^p over s <= t (§2.6) with
// kappa_ts = <Phi(q_t), Phi(k_s)> (§2.3).  The chunked p = 1 prefill computes the same outputs, so this is its
// gradient as well.  For L = sum_t <g_t, o_t> (g = dout), in the kernels' scaled units (weights kappa^p,
// epsilon scaled by c^p, so Dn_t = sum_s kappa_ts^p + eps c^p):
//   G_ts = dL/dkappa_ts = p kappa_ts^(p-1) (<g_t, v_s> - delta_t) / Dn_t,   delta_t = <g_t, o_t>
//   dPhi(q_t) = sum_{s<=t} G_ts Phi(k_s),  dPhi(k_s) = sum_{t>=s} G_ts Phi(q_t),
//   dv_s = sum_{t>=s} kappa_ts^p g_t / Dn_t,
// then the feature map's Jacobian: with y = theta + t lambda and r' = dr/dtheta = dr/domega,
//   dtheta = r' (g_r + g_rc cos y + g_rs sin y) - sin y (g_c + r g_rc) + cos y (g_s + r g_rs),
//   du = dtheta pi / (1 + |u|)^2,  domega_a = sum over tokens of r' (g_r + g_rc cos y + g_rs sin y).
//
// Work split.  Phi(Q) and Phi(K) are featurized once into the workspace (element type of the call).  At p = 1
// the statistics, the feature gradients and dv come from the chunked recurrences of backward_chunked.hip.  At
// p = 2 a statistics pass (the forward kernel in its STATS mode) writes (1 / Dn_t, delta_t); then, flash-attention
// style, one kernel walks key blocks for each 32-query tile of a wave (dPhi(Q)), and one walks query blocks
// for each 32-key tile (dPhi(K) and dv); both recompute the score and <g, v> tiles on 32x32x16 bf16 MFMA
// (32x32x2 fp32 for fp32 inputs).  A wave keeps a 32 x 192 fp32 slice of its gradient in accumulators (32 x 128
// for fp32 inputs, whose operand fragments need twice the registers), so the feature gradients take two (three)
// passes, each recomputing the score tiles.  With bf16 operands, G enters the dPhi products as its bf16 rounding
// plus the bf16 rounding of the residual: a row of G nearly cancels (its weighted sum is ~0), so one rounding
// would leave an error of the order of the result.  The feature gradients go to an fp32 workspace; the Jacobian kernel turns them into
// du and per-block omega partials, which two small kernels sum in a fixed order (bitwise deterministic).
#include <atomic>

#include "feature_tiles.h"

namespace sanatan {

hipError_t launch_quadratic_stats(const void* q, const void* phik, const void* v, const void* g, sanatan_dtype t,
                                  int B, int H, int T, int p, const float* rho, const MethodConsts& mc, float2* stats,
                                  hipStream_t stream);
// backward_chunked.hip: the p = 1 feature gradients and dv as chunked recurrences (writing the per-sequence omega
// sums [2 sides][BH][d] to seq_sum), and the bytes of their slots and omega partials
size_t bwd_chunked_slot_bytes(int B, int H, int T);
hipError_t launch_bwd_chunked(const void* phiq, const void* phik, const void* v, const void* g, float2* stats,
                              sanatan_dtype t, int B, int H, int T, float ceps, const void* q, const void* k,
                              const float* rho, const float* omega, int nph, float kr, void* dq, void* dk, void* dv,
                              float* seq_sum, float* slots, hipStream_t stream);

// backward_quadratic.hip: the bf16 gradients at p = 2 (feature gradients, Jacobian and omega partials fused)
hipError_t launch_bwd_quadratic_bf16(const void* phiq, const void* phik, const void* v, const void* g,
                                     const float2* stats, int B, int H, int T, const void* q, const void* k,
                                     const float* rho, const float* omega, int nph, float kr, void* dq, void* dk,
                                     void* dv, float* dom_q, float* dom_k, hipStream_t stream);

namespace {

constexpr int kBlk = 32;  // tokens per staged block (and per wave tile)

template <typename T>
struct BGeom {
  static constexpr int FP = kF + 16 / (int)sizeof(T);   // feature tile pitch (elements): rows 16 bytes apart
  static constexpr int VP = kDV + 16 / (int)sizeof(T);  // value / gradient tile pitch
  static constexpr int f_bytes = kBlk * FP * (int)sizeof(T);
  static constexpr int v_bytes = kBlk * VP * (int)sizeof(T);
  static constexpr int st_bytes = kBlk * 8;
  static constexpr int lds = f_bytes + v_bytes + st_bytes;
  static constexpr int EL = 16 / (int)sizeof(T);        // elements per 16-byte piece
  static constexpr int FPIECES = kBlk * kF / EL / 256;  // 16-byte pieces per thread of one feature block
  static constexpr int VPIECES = kBlk * kDV / EL / 256;
};

// 8 consecutive elements of one row, in and out
__device__ __forceinline__ void ld8c(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void ld8c(const __bf16* p, float (&o)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; i++) o[i] = (float)v[i];
}
__device__ __forceinline__ void st8c(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void st8c(__bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = (__bf16)x[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}

// One staged block: 32 rows of features [32][384] and of a 64-wide operand (V or g), rows clamped to the
// sequence (rows past its end repeat the last row; the kernels mask them), and (dK kernel) the block's stats.
template <typename T>
struct BlockStage {
  using G = BGeom<T>;
  u32x4 pf[G::FPIECES], pv[G::VPIECES > 0 ? G::VPIECES : 1];
  float2 st;
  __device__ __forceinline__ void fetch(const T* feat, const T* val, const float2* stats, int s0, int Tn, int tid) {
#pragma unroll
    for (int p = 0; p < G::FPIECES; p++) {
      const int e = tid + 256 * p, row = e / (kF / G::EL), col = (e % (kF / G::EL)) * G::EL;
      pf[p] = *reinterpret_cast<const u32x4*>(feat + (size_t)min(s0 + row, Tn - 1) * kF + col);
    }
#pragma unroll
    for (int p = 0; p < G::VPIECES; p++) {
      const int e = tid + 256 * p, row = e / (kDV / G::EL), col = (e % (kDV / G::EL)) * G::EL;
      pv[p] = *reinterpret_cast<const u32x4*>(val + (size_t)min(s0 + row, Tn - 1) * kDV + col);
    }
    if (stats && tid < kBlk) st = stats[min(s0 + tid, Tn - 1)];
  }
  __device__ __forceinline__ void stash(char* smem, bool with_stats, int tid) const {
    T* F = reinterpret_cast<T*>(smem);
    T* V = reinterpret_cast<T*>(smem + G::f_bytes);
#pragma unroll
    for (int p = 0; p < G::FPIECES; p++) {
      const int e = tid + 256 * p, row = e / (kF / G::EL), col = (e % (kF / G::EL)) * G::EL;
      *reinterpret_cast<u32x4*>(F + row * G::FP + col) = pf[p];
    }
#pragma unroll
    for (int p = 0; p < G::VPIECES; p++) {
      const int e = tid + 256 * p, row = e / (kDV / G::EL), col = (e % (kDV / G::EL)) * G::EL;
      *reinterpret_cast<u32x4*>(V + row * G::VP + col) = pv[p];
    }
    if (with_stats && tid < kBlk) reinterpret_cast<float2*>(smem + G::f_bytes + G::v_bytes)[tid] = st;
  }
};

// Row operand: 8 consecutive elements of row `row` of a [rows][pitch] tile (LDS or global), from column col.
template <typename T>
__device__ __forceinline__ typename FragT<T>::type row_frag(const T* base, int pitch, int row, int col) {
  typedef typename FragT<T>::type Frag;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const Frag*>(base + (size_t)row * pitch + col);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(base + (size_t)row * pitch + col);
    const float4 b = *reinterpret_cast<const float4*>(base + (size_t)row * pitch + col + 4);
    Frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    return f;
  }
}

// dPhi(Q) for one 32-query tile per wave (four per workgroup), feature tiles FT0 .. FT0 + NFT - 1 (32 features
// each).  Tile layout: accumulator [s][t] (rows keys, columns queries), so a lane (query n32, half h) owns
// one query and its scalars (Dn_t, delta_t).
template <typename T, int P, int FT0, int NFT>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(const T* __restrict__ phiq, const T* __restrict__ phik,
                                                        const T* __restrict__ v, const T* __restrict__ g,
                                                        const float2* __restrict__ stats, float* __restrict__ dphiq,
                                                        int Tn, int BH, int nqb) {
  using G = BGeom<T>;
  typedef typename FragT<T>::type Frag;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);  // heaviest (latest) query tiles first
  const int bh = (int)(blockIdx.x % BH);
  const int row0 = qb * 128 + 32 * w;
  const size_t sq = (size_t)bh * Tn;
  const int t = row0 + n32, tc = min(t, Tn - 1);
  const T* F = reinterpret_cast<const T*>(smem);
  const T* Vt = reinterpret_cast<const T*>(smem + G::f_bytes);

  // the wave's query operands: Phi(q) K-steps 4..23 (channels 1..5; channel 0 enters as the splat d) and g
  Frag QF[20], GF[4];
#pragma unroll
  for (int j = 0; j < 20; j++) QF[j] = row_frag<T>(phiq + sq * kF, kF, tc, 64 + 16 * j + 8 * h);
#pragma unroll
  for (int j = 0; j < 4; j++) GF[j] = row_frag<T>(g + sq * kDV, kDV, tc, 16 * j + 8 * h);
  const float2 stt = stats[sq + tc];
  const float inv_dn = stt.x, delta = stt.y;

  f32x16 acc[NFT];
#pragma unroll
  for (int f = 0; f < NFT; f++) zero16(acc[f]);
  f32x16 c0;
#pragma unroll
  for (int i = 0; i < 16; i++) c0[i] = (float)kD;

  const int last_row = min(Tn - 1, qb * 128 + 127);
  const int nkb = last_row / kBlk + 1;          // key blocks the workgroup needs
  const int my_last = min(Tn - 1, row0 + 31);
  const int lastb = row0 < Tn ? my_last / kBlk : -1;  // this wave's last key block
  BlockStage<T> stg;
  stg.fetch(phik + sq * kF, v + sq * kDV, nullptr, 0, Tn, tid);
  for (int kb = 0; kb < nkb; kb++) {
    __syncthreads();  // the previous block's tiles are no longer read
    stg.stash(smem, false, tid);
    if (kb + 1 < nkb) stg.fetch(phik + sq * kF, v + sq * kDV, nullptr, (kb + 1) * kBlk, Tn, tid);
    __syncthreads();
    if (kb > lastb) continue;
    const int s0 = kb * kBlk;
    // scores kappa^T[s][t] and <v_s, g_t>
    f32x16 at = c0, gv;
    zero16(gv);
#pragma unroll
    for (int j = 0; j < 20; j++) mma32(at, row_frag<T>(F, G::FP, n32, 64 + 16 * j + 8 * h), QF[j]);
#pragma unroll
    for (int j = 0; j < 4; j++) mma32(gv, row_frag<T>(Vt, G::VP, n32, 16 * j + 8 * h), GF[j]);
    float gl[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int s = s0 + 8 * (i >> 2) + 4 * h + (i & 3);
      const float kap = at[i];
      const float dk = (P == 2 ? 2.0f * kap : 1.0f) * (gv[i] - delta) * inv_dn;
      gl[i] = (s > t || s >= Tn) ? 0.0f : dk;
    }
    float lo[8], hi8[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      lo[i] = gl[i];
      hi8[i] = gl[8 + i];
    }
    const Frag G0 = pack8f<T>(lo), G1 = pack8f<T>(hi8);
    // dPhi(q)^T[f][t] += Phi(K)^T[f][s] G^T[s][t].  With bf16 operands G also enters as its rounding residual
    // (a second bf16 term): a row of G nearly cancels, so its rounding error would weigh on the sum.
    Frag R0 = G0, R1 = G1;
    if constexpr (sizeof(T) == 2) R0 = residual8<T>(lo, G0), R1 = residual8<T>(hi8, G1);
#pragma unroll
    for (int f = 0; f < NFT; f++) {
      const Frag A0 = lds_tokfrag(F, G::FP, 0, 32 * (FT0 + f), l), A1 = lds_tokfrag(F, G::FP, 16, 32 * (FT0 + f), l);
      mma32(acc[f], A0, G0);
      mma32(acc[f], A1, G1);
      if constexpr (sizeof(T) == 2) {
        mma32(acc[f], A0, R0);
        mma32(acc[f], A1, R1);
      }
    }
  }
  if (t >= Tn) return;
  float* dst = dphiq + (sq + t) * kF;
#pragma unroll
  for (int f = 0; f < NFT; f++)
#pragma unroll
    for (int j = 0; j < 4; j++)
      *reinterpret_cast<float4*>(dst + 32 * (FT0 + f) + 8 * j + 4 * h) =
          make_float4(acc[f][4 * j], acc[f][4 * j + 1], acc[f][4 * j + 2], acc[f][4 * j + 3]);
}

// dPhi(K) (feature tiles FT0 .. FT0 + NFT - 1) and, with WITH_V, dv, for one 32-key tile per wave.  Tile layout:
// accumulator [t][s] (rows queries, columns keys): a lane (key n32, half h) owns one key; the per-query
// scalars of its 16 rows come from the staged block's stats.
template <typename T, int P, int FT0, int NFT, bool WITH_V>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(const T* __restrict__ phiq, const T* __restrict__ phik,
                                                         const T* __restrict__ v, const T* __restrict__ g,
                                                         const float2* __restrict__ stats, float* __restrict__ dphik,
                                                         T* __restrict__ dv, int Tn, int BH, int nkb_all) {
  using G = BGeom<T>;
  typedef typename FragT<T>::type Frag;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  const int kt = (int)(blockIdx.x / BH);  // heaviest (earliest) key tiles first
  const int bh = (int)(blockIdx.x % BH);
  const int row0 = kt * 128 + 32 * w;
  const size_t sq = (size_t)bh * Tn;
  const int s = row0 + n32, sc = min(s, Tn - 1);
  const T* F = reinterpret_cast<const T*>(smem);
  const T* Gt = reinterpret_cast<const T*>(smem + G::f_bytes);
  const float2* St = reinterpret_cast<const float2*>(smem + G::f_bytes + G::v_bytes);

  Frag KF[20], VF[4];
#pragma unroll
  for (int j = 0; j < 20; j++) KF[j] = row_frag<T>(phik + sq * kF, kF, sc, 64 + 16 * j + 8 * h);
#pragma unroll
  for (int j = 0; j < 4; j++) VF[j] = row_frag<T>(v + sq * kDV, kDV, sc, 16 * j + 8 * h);

  f32x16 acc[NFT], accv[2];
#pragma unroll
  for (int f = 0; f < NFT; f++) zero16(acc[f]);
  zero16(accv[0]);
  zero16(accv[1]);
  f32x16 c0;
#pragma unroll
  for (int i = 0; i < 16; i++) c0[i] = (float)kD;

  const int first_q = (kt * 128) / kBlk;                     // first query block the workgroup needs
  const int my_first = row0 < Tn ? row0 / kBlk : nkb_all;    // this wave's first query block
  BlockStage<T> stg;
  stg.fetch(phiq + sq * kF, g + sq * kDV, stats + sq, first_q * kBlk, Tn, tid);
  for (int tb = first_q; tb < nkb_all; tb++) {
    __syncthreads();
    stg.stash(smem, true, tid);
    if (tb + 1 < nkb_all) stg.fetch(phiq + sq * kF, g + sq * kDV, stats + sq, (tb + 1) * kBlk, Tn, tid);
    __syncthreads();
    if (tb < my_first) continue;
    const int t0 = tb * kBlk;
    f32x16 at = c0, gv;
    zero16(gv);
#pragma unroll
    for (int j = 0; j < 20; j++) mma32(at, row_frag<T>(F, G::FP, n32, 64 + 16 * j + 8 * h), KF[j]);
#pragma unroll
    for (int j = 0; j < 4; j++) mma32(gv, row_frag<T>(Gt, G::VP, n32, 16 * j + 8 * h), VF[j]);
    float gl[16], wl[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = 8 * (i >> 2) + 4 * h + (i & 3), t = t0 + r;
      const float2 st = St[r];
      const float inv_dn = st.x;
      const float kap = at[i];
      const bool keep = s <= t && t < Tn;
      gl[i] = keep ? (P == 2 ? 2.0f * kap : 1.0f) * (gv[i] - st.y) * inv_dn : 0.0f;
      wl[i] = keep ? (P == 2 ? kap * kap : kap) * inv_dn : 0.0f;
    }
    float lo[8], hi8[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      lo[i] = gl[i];
      hi8[i] = gl[8 + i];
    }
    const Frag G0 = pack8f<T>(lo), G1 = pack8f<T>(hi8);
    Frag R0 = G0, R1 = G1;  // bf16: G's rounding residual as a second term, as in the dPhi(q) kernel
    if constexpr (sizeof(T) == 2) R0 = residual8<T>(lo, G0), R1 = residual8<T>(hi8, G1);
#pragma unroll
    for (int f = 0; f < NFT; f++) {
      const Frag A0 = lds_tokfrag(F, G::FP, 0, 32 * (FT0 + f), l), A1 = lds_tokfrag(F, G::FP, 16, 32 * (FT0 + f), l);
      mma32(acc[f], A0, G0);
      mma32(acc[f], A1, G1);
      if constexpr (sizeof(T) == 2) {
        mma32(acc[f], A0, R0);
        mma32(acc[f], A1, R1);
      }
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo[i] = wl[i];
        hi8[i] = wl[8 + i];
      }
      const Frag W0 = pack8f<T>(lo), W1 = pack8f<T>(hi8);
#pragma unroll
      for (int vt = 0; vt < 2; vt++) {
        mma32(accv[vt], lds_tokfrag(Gt, G::VP, 0, 32 * vt, l), W0);
        mma32(accv[vt], lds_tokfrag(Gt, G::VP, 16, 32 * vt, l), W1);
      }
    }
  }
  if (s >= Tn) return;
  float* dst = dphik + (sq + s) * kF;
#pragma unroll
  for (int f = 0; f < NFT; f++)
#pragma unroll
    for (int j = 0; j < 4; j++)
      *reinterpret_cast<float4*>(dst + 32 * (FT0 + f) + 8 * j + 4 * h) =
          make_float4(acc[f][4 * j], acc[f][4 * j + 1], acc[f][4 * j + 2], acc[f][4 * j + 3]);
  if constexpr (WITH_V) {
    T* dvp = dv + (sq + s) * kDV;
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i4 = 0; i4 < 4; i4++) dvp[32 * vt + 8 * j + 4 * h + i4] = from_f32<T>(accv[vt][4 * j + i4]);
  }
}

// The feature map's Jacobian: dPhi [BH][T][6d] fp32 -> du [BH][T][d] (element type T), and per-block omega
// partials [block][d] (each block covers 32 tokens of one sequence; its partial is the sum over those tokens in
// a fixed order).  A thread owns 8 dims of one token; the recomputed angle, root and rotation follow
// featurize1 exactly (same hardware operations, same reduced phase).
template <typename T>
__global__ __launch_bounds__(256) void bwd_jacobian_kernel(const T* __restrict__ u, const float* __restrict__ dphi,
                                                           const float* __restrict__ rho,
                                                           const float* __restrict__ omega, int nph, int H, int Tn,
                                                           float kr, int ntiles, T* __restrict__ du,
                                                           float* __restrict__ dom_part) {
  __shared__ float red[32][kD + 1];
  const int bh = (int)(blockIdx.x / ntiles), tile = (int)(blockIdx.x % ntiles);
  const int j = threadIdx.x & 7, a0 = 8 * j, row = threadIdx.x >> 3;
  const int hd = bh % H;
  const int t = tile * 32 + row;
  float dom[8];
#pragma unroll
  for (int i = 0; i < 8; i++) dom[i] = 0.0f;
  if (t < Tn) {
    const size_t base = (size_t)bh * Tn + t;
    float x[8], rh[8], gch[6][8];  // gch[0] unused
    ld8c(u + base * kD + a0, x);
#pragma unroll
    for (int i = 0; i < 8; i++) rh[i] = rho[(size_t)t * kD + a0 + i];
#pragma unroll
    for (int c = 1; c < 6; c++) {  // channel 0 (the constant feature) has no derivative
      const float4 p0 = *reinterpret_cast<const float4*>(dphi + base * kF + c * kD + a0);
      const float4 p1 = *reinterpret_cast<const float4*>(dphi + base * kF + c * kD + a0 + 4);
      gch[c][0] = p0.x; gch[c][1] = p0.y; gch[c][2] = p0.z; gch[c][3] = p0.w;
      gch[c][4] = p1.x; gch[c][5] = p1.y; gch[c][6] = p1.z; gch[c][7] = p1.w;
    }
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float om4 = anchor_rev(omega[(size_t)(hd % nph) * kD + a0 + i]);
      feature_vjp(x[i], rh[i], om4, kr, gch[1][i], gch[2][i], gch[3][i], gch[4][i], gch[5][i], o[i], dom[i]);
    }
    st8c(du + base * kD + a0, o);
  }
#pragma unroll
  for (int i = 0; i < 8; i++) red[row][a0 + i] = dom[i];
  __syncthreads();
  if (threadIdx.x < kD) {
    float acc = 0.0f;
    for (int r = 0; r < 32; r++) acc += red[r][threadIdx.x];
    dom_part[(size_t)blockIdx.x * kD + threadIdx.x] = acc;
  }
}

// domega in two fixed-order stages.  Stage 1: per (side, sequence) the sum of its tiles' partials, eight
// independent partial sums per dim, combined in a fixed order.  Stage 2: per omega row, the sum over the q and k
// sides of every sequence whose head uses that row, in sequence order.
__global__ __launch_bounds__(64) void bwd_domega_seq_kernel(const float* __restrict__ part, int ntiles,
                                                            float* __restrict__ seq_sum) {
  const int sb = blockIdx.x, a = threadIdx.x;  // sb = side * BH + bh
  const float* p = part + (size_t)sb * ntiles * kD + a;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int t = 0;
  for (; t + 8 <= ntiles; t += 8)
#pragma unroll
    for (int u = 0; u < 8; u++) acc[u] += p[(size_t)(t + u) * kD];
  for (; t < ntiles; t++) acc[0] += p[(size_t)t * kD];
  seq_sum[(size_t)sb * kD + a] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}
__global__ __launch_bounds__(64) void bwd_domega_kernel(const float* __restrict__ seq_sum, int BH, int H, int nph,
                                                        float* __restrict__ domega) {
  const int prow = blockIdx.x, a = threadIdx.x;
  float acc = 0.0f;
  for (int bh = 0; bh < BH; bh++)
    if ((bh % H) % nph == prow) acc += seq_sum[(size_t)bh * kD + a] + seq_sum[((size_t)BH + bh) * kD + a];
  domega[(size_t)prow * kD + a] = acc;
}

// The statistics from a saved forward pass (fp32 output rows o [rows][d_v], then 1 / Dn [rows]):
// stats[r] = (1 / Dn_r, delta_r = <dout_r, o_r>), one row per thread, the dot product in fp32 in dimension order.
template <typename T>
__global__ __launch_bounds__(256) void bwd_saved_stats_kernel(const T* __restrict__ g, const float* __restrict__ saved,
                                                              size_t rows, float2* __restrict__ stats) {
  const size_t r = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const float* o = saved;
  const float* inv = saved + rows * kDV;
  float gv[8], ov[8], acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kDV / 8; j++) {
    ld8c(g + r * kDV + 8 * j, gv);
    ld8c(o + r * kDV + 8 * j, ov);
#pragma unroll
    for (int i = 0; i < 8; i++) acc = fmaf(gv[i], ov[i], acc);
  }
  stats[r] = make_float2(inv[r], acc);
}

template <typename Kern>
hipError_t set_lds(Kern k, int bytes, std::atomic<bool>& flag) {
  if (flag.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) flag.store(true, std::memory_order_release);
  return e;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t rho, phiq, phik, stats, dphiq, dphik, dom, slots, total;
};
BwdLayout bwd_layout(int B, int H, int T, sanatan_dtype t) {
  const size_t el = t == SANATAN_BF16 ? 2 : 4;
  const size_t BHT = (size_t)B * H * T;
  const size_t nblk = (size_t)B * H * ((T + 31) / 32);
  BwdLayout L;
  L.rho = 0;
  L.phiq = al256((size_t)T * kD * 4);
  L.phik = L.phiq + al256(BHT * kF * el);
  L.stats = L.phik + al256(BHT * kF * el);
  L.dphiq = L.stats + al256(BHT * 8);
  L.dphik = L.dphiq + al256(BHT * kF * 4);
  L.dom = L.dphik + al256(BHT * kF * 4);
  L.slots = L.dom + al256(2 * nblk * kD * 4) + al256((size_t)2 * B * H * kD * 4);
  L.total = L.slots + al256(bwd_chunked_slot_bytes(B, H, T));
  return L;
}

template <typename T, int P>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* g, int B, int H, int Tn,
                        int64_t pos0, const MethodConsts& mc, void* dq, void* dk, void* dv, float* domega, void* ws,
                        sanatan_dtype dt, hipStream_t stream, const float* saved) {
  using G = BGeom<T>;
  char* base = static_cast<char*>(ws);
  const BwdLayout L = bwd_layout(B, H, Tn, dt);
  float* rho = reinterpret_cast<float*>(base + L.rho);
  T* phiq = reinterpret_cast<T*>(base + L.phiq);
  T* phik = reinterpret_cast<T*>(base + L.phik);
  float2* stats = reinterpret_cast<float2*>(base + L.stats);
  float* dphiq = reinterpret_cast<float*>(base + L.dphiq);
  float* dphik = reinterpret_cast<float*>(base + L.dphik);
  float* dom = reinterpret_cast<float*>(base + L.dom);
  hipError_t e = launch_phase_table(rho, Tn, pos0, mc.log2_base, stream);
  if (e != hipSuccess) return e;
  if ((e = launch_featurize(q, dt, B, H, Tn, pos0, mc, phiq, dt, stream)) != hipSuccess) return e;
  if ((e = launch_featurize(k, dt, B, H, Tn, pos0, mc, phik, dt, stream)) != hipSuccess) return e;
  if constexpr (P == 1) {
    // p = 1: the statistics, the feature gradients and dv as chunked recurrences, linear in T
    // (the per-sequence omega sums go where the p = 2 path's stage 1 writes them)
    float* seq_sum = dom + (size_t)2 * B * H * ((Tn + 31) / 32) * kD;
    if ((e = launch_bwd_chunked(phiq, phik, v, g, stats, dt, B, H, Tn, mc.ceps, q, k, rho, mc.omega, mc.nph, mc.kr,
                                dq, dk, dv, seq_sum, reinterpret_cast<float*>(base + L.slots), stream)) != hipSuccess)
      return e;
  } else {
    if (saved) {  // the forward pass's saved output rows and normalisers replace the statistics pass
      const size_t rows = (size_t)B * H * Tn;
      hipLaunchKernelGGL((bwd_saved_stats_kernel<T>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                         static_cast<const T*>(g), saved, rows, stats);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if ((e = launch_quadratic_stats(q, phik, v, g, dt, B, H, Tn, P, rho, mc, stats, stream)) != hipSuccess) {
      return e;
    }

  // feature gradients over the feature tiles of channels 1..5 (tiles 2..11: channel 0 is the constant 1, whose
  // gradient the Jacobian does not use).  bf16 runs the pipelined one-pass kernels of backward_quadratic.hip;
  // fp32, whose operand fragments need twice the registers, takes 4 + 4 + 2 tiles in three passes here, dv
  // with the first dK pass.
  const int nqb = (Tn + 127) / 128, nkb_all = (Tn + kBlk - 1) / kBlk, BH = B * H;
  static std::atomic<bool> attr[8][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const dim3 grid(BH * nqb), blk(256);
  const T* cq = phiq;
  const T* ck = phik;
  const T* cv = static_cast<const T*>(v);
  const T* cg = static_cast<const T*>(g);
  auto pass = [&](auto Ft0, auto Nft, auto WithV, int slot) -> hipError_t {
    constexpr int FT0 = decltype(Ft0)::value, NFT = decltype(Nft)::value;
    constexpr bool WV = decltype(WithV)::value;
    hipError_t err = set_lds(bwd_dq_kernel<T, P, FT0, NFT>, G::lds, attr[2 * slot][dev]);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_dq_kernel<T, P, FT0, NFT>), grid, blk, G::lds, stream, cq, ck, cv, cg, stats, dphiq, Tn,
                       BH, nqb);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = set_lds(bwd_dkv_kernel<T, P, FT0, NFT, WV>, G::lds, attr[2 * slot + 1][dev])) != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_dkv_kernel<T, P, FT0, NFT, WV>), grid, blk, G::lds, stream, cq, ck, cv, cg, stats, dphik,
                       static_cast<T*>(dv), Tn, BH, nkb_all);
    return hipGetLastError();
  };
  if constexpr (sizeof(T) == 2) {
    const size_t side = (size_t)BH * nkb_all * kD;  // omega partial rows of one side
    if ((e = launch_bwd_quadratic_bf16(phiq, phik, v, g, stats, B, H, Tn, q, k, rho, mc.omega, mc.nph, mc.kr, dq, dk,
                                       dv, dom, dom + side, stream)) != hipSuccess)
      return e;
  } else {
    if ((e = pass(std::integral_constant<int, 2>(), std::integral_constant<int, 4>(), std::true_type(), 0)) !=
        hipSuccess)
      return e;
    if ((e = pass(std::integral_constant<int, 6>(), std::integral_constant<int, 4>(), std::false_type(), 1)) !=
        hipSuccess)
      return e;
    if ((e = pass(std::integral_constant<int, 10>(), std::integral_constant<int, 2>(), std::false_type(), 2)) !=
        hipSuccess)
      return e;
  }
  }
  const int BH = B * H, ntiles = (Tn + 31) / 32, nblk = BH * ntiles;
  const int nparts = ntiles;  // omega partial rows per (side, sequence)
  float* seq_sum = dom + (size_t)2 * nblk * kD;
  if constexpr (sizeof(T) == 4 && P != 1) {  // (bf16: the gradient kernels applied the Jacobian; p = 1: the chunk
                                            // kernels did, and wrote the per-sequence sums)
    hipLaunchKernelGGL((bwd_jacobian_kernel<T>), dim3(nblk), dim3(256), 0, stream, static_cast<const T*>(q), dphiq,
                       rho, mc.omega, mc.nph, H, Tn, mc.kr, ntiles, static_cast<T*>(dq), dom);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_jacobian_kernel<T>), dim3(nblk), dim3(256), 0, stream, static_cast<const T*>(k), dphik,
                       rho, mc.omega, mc.nph, H, Tn, mc.kr, ntiles, static_cast<T*>(dk),
                       dom + (size_t)nparts * BH * kD);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if constexpr (P != 1) {
    hipLaunchKernelGGL(bwd_domega_seq_kernel, dim3(2 * BH), dim3(64), 0, stream, dom, nparts, seq_sum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_domega_kernel, dim3(mc.nph), dim3(64), 0, stream, seq_sum, BH, H, mc.nph, domega);
  return hipGetLastError();
}

}  // namespace

size_t backward_ws_bytes(int B, int H, int T, sanatan_dtype t) { return bwd_layout(B, H, T, t).total; }

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* dout, sanatan_dtype t, int B,
                           int H, int T, int p, int64_t pos0, const MethodConsts& mc, void* dq, void* dk, void* dv,
                           float* domega, void* ws, hipStream_t stream, const float* si) {
  if (t == SANATAN_BF16)
    return p == 1 ? launch_bwd_t<__bf16, 1>(q, k, v, dout, B, H, T, pos0, mc, dq, dk, dv, domega, ws, t, stream, si)
                  : launch_bwd_t<__bf16, 2>(q, k, v, dout, B, H, T, pos0, mc, dq, dk, dv, domega, ws, t, stream, si);
  return p == 1 ? launch_bwd_t<float, 1>(q, k, v, dout, B, H, T, pos0, mc, dq, dk, dv, domega, ws, t, stream, si)
                : launch_bwd_t<float, 2>(q, k, v, dout, B, H, T, pos0, mc, dq, dk, dv, domega, ws, t, stream, si);
}

}  // namespace sanatan
