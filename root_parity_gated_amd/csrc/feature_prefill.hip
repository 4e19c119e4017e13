// feature_prefill.hip -- chunked causal p = 1 attention over materialized feature maps: the spectral-harmonic
// map and the unclipped four-channel map.
//
// SANATAN reading notes: the p = 1 recurrence S_t = S_{t-1} + Phi(k_t) v_t^T, z_t = z_{t-1} + Phi(k_t),
// o_t = Phi(q_t)^T S_t / (Phi(q_t)^T z_t + c eps) holds for any explicit feature map (§2.7).  Two maps besides
// the six-channel one are served here:
//   * spectral harmonics (the Appendix B outlook): per dim [1, cos n th, sin n th (n = 1..nh), r,
//     r cos n th, r sin n th (n = 1..nh)] of the rotated angle th, (2 + 4 nh) d features, state rows in that
//     channel-major order (nh = 1 is the six-channel map);
//   * the unclipped four-channel kernel (§2.5), per dim [1, r, r cos th, r sin th], kept compact like its decode
//     state: one shared channel-0 feature (1 for a key; d for a query, which stands for its d equal rows) and
//     r, r cos th, r sin th: 3d + 1 features.  The caller's state holds the shared row first; the workspace
//     holds it last (feature 3d), so that every thread's 8 dims of a channel are one aligned vector store.
// Phi(Q) and Phi(K) are featurized once into the workspace (element type of the call), padded to a multiple
// of 128 features with zeros.  The prefill kernel then walks each sequence in 32-token chunks with one
// workgroup of 4 waves per sequence: wave w owns feature tiles w, w + 4, ... (32 features each) and their
// 32 x 64 slices of S in MFMA accumulators; per chunk it forms its partial masked scores Phi(K) Phi(Q)^T over
// those features, the partial numerator V^T P + S^T Phi(Q)^T and denominator, and after the four partials
// meet in LDS (fixed order) the chunk's outputs are normalised; then S += Phi(K)^T V and z += Phi(K)^T 1.
// Operands: bf16 32x32x16 MFMA (fp32 32x32x2 for fp32 inputs), fp32 accumulation; S is rounded to the
// operand type only as the readout's operand.
// Sequence split: with fewer sequences than compute units, each sequence is cut into P pieces of whole chunks,
// one workgroup each.  Pass 1 (STATE_ONLY) runs pieces 0..P-2, each split into SPL parts of whole chunks, and
// writes each part's state increment to its slot (part 0 of piece 0 includes the caller's start state, which it
// also copies to the spare slot of piece P - 1); pass 3 then starts piece p from the sum of the slots of pieces
// 0..p-1 (piece 0 from that spare slot), so that no piece of pass 3 reads the caller's state while the final
// piece writes it back.
#include <atomic>

#include "feature_tiles.h"

namespace sanatan {
namespace {

constexpr int kFC = 32;  // chunk tokens

// The map's features of 8 consecutive dims a0 = 8 j .. 8 j + 7 of one token, in the padded feature layout:
// emit(row0, val) receives features row0 + a0 .. row0 + a0 + 7 of each channel (and zeros for the padding rows up
// to Fp).  KIND 0: harmonics n = 1..NH; KIND 1: four-channel compact, shared feature at 3d (IS_Q: it carries d
// instead of 1).  x: the raw components, rho: their phases (revolutions), om4: their anchors (anchor_rev).
template <int KIND, int NH, bool IS_Q, typename Emit>
__device__ __forceinline__ void ext_features8(const float (&x)[8], const float (&rho)[8], const float (&om4)[8],
                                              float kr, int j, int Fp, Emit&& emit) {
  float cr[8], sr[8], rr[8], y[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    featurize1(x[i], rho[i], om4[i], kr, cr[i], sr[i], rr[i]);
    y[i] = x[i] * rcp_hw(fmaf(fabsf(x[i]), 2.0f, 2.0f)) + rho[i];  // the rotated angle in revolutions, as featurize1
  }
  float tmp[8];
  if constexpr (KIND == 0) {
#pragma unroll
    for (int i = 0; i < 8; i++) tmp[i] = 1.0f;
    emit(0, tmp);
    emit((2 * NH + 1) * kD, rr);
#pragma unroll
    for (int n = 1; n <= NH; n++) {
      float c[8], sn[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        c[i] = n == 1 ? cr[i] : cos_rev((float)n * y[i]);
        sn[i] = n == 1 ? sr[i] : sin_rev((float)n * y[i]);
      }
      emit((2 * n - 1) * kD, c);
      emit((2 * n) * kD, sn);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        c[i] *= rr[i];
        sn[i] *= rr[i];
      }
      emit((2 * NH + 2 * n) * kD, c);
      emit((2 * NH + 2 * n + 1) * kD, sn);
    }
    // zero padding past (2 + 4 NH) d
    constexpr int Fr = (2 + 4 * NH) * kD;
#pragma unroll
    for (int i = 0; i < 8; i++) tmp[i] = 0.0f;
    for (int f = Fr; f < Fp; f += kD) emit(f, tmp);
  } else {
    // internal order r, r cos, r sin (d each), then the shared feature (d for a query, 1 for a key) and zero
    // padding; the caller's compact state keeps the shared row first, and the prefill maps rows between the two
    float rc[8], rs[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      rc[i] = rr[i] * cr[i];
      rs[i] = rr[i] * sr[i];
    }
    emit(0, rr);
    emit(kD, rc);
    emit(2 * kD, rs);
#pragma unroll
    for (int i = 0; i < 8; i++) tmp[i] = (j == 0 && i == 0) ? (IS_Q ? (float)kD : 1.0f) : 0.0f;
    emit(3 * kD, tmp);  // the shared feature, then zeros up to 3 d + 64
#pragma unroll
    for (int i = 0; i < 8; i++) tmp[i] = 0.0f;
    for (int f = 4 * kD; f < Fp; f += kD) emit(f, tmp);
  }
}

// 8 features as one 16-byte (bf16) or two 16-byte (fp32) stores
__device__ __forceinline__ void put8(__bf16* o, const float (&val)[8]) {
  bf16x8 w;
#pragma unroll
  for (int i = 0; i < 8; i++) w[i] = (__bf16)val[i];
  *reinterpret_cast<bf16x8*>(o) = w;
}
__device__ __forceinline__ void put8(float* o, const float (&val)[8]) {
  *reinterpret_cast<float4*>(o) = make_float4(val[0], val[1], val[2], val[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(val[4], val[5], val[6], val[7]);
}

// featurize one operand into the padded feature layout in global memory (the fp32 prefill's operands).  A thread
// owns 8 dims of one token.
template <typename TIn, typename TOut, int KIND, int NH, bool IS_Q>
__global__ __launch_bounds__(256) void featurize_ext_kernel(const TIn* __restrict__ u, TOut* __restrict__ phi, int H,
                                                            int T, int Fp, int64_t pos0,
                                                            const float* __restrict__ omega, int nph,
                                                            double log2_base, float kr, int ntiles) {
  const int bh = (int)(blockIdx.x / ntiles), tile = (int)(blockIdx.x % ntiles), j = threadIdx.x & 7, a0 = 8 * j;
  const int t = tile * 32 + (threadIdx.x >> 3);
  if (t >= T) return;
  const int hd = bh % H;
  const TIn* up = u + ((size_t)bh * T + t) * kD + a0;
  TOut* o = phi + ((size_t)bh * T + t) * Fp;
  float x[8], rho[8], om4[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    om4[i] = anchor_rev(omega[(size_t)(hd % nph) * kD + a0 + i]);
    rho[i] = phase_at(pos0 + t, phase_step(a0 + i, log2_base));
    x[i] = to_f32(up[i]);
  }
  ext_features8<KIND, NH, IS_Q>(x, rho, om4, kr, j, Fp, [&](int row0, const float (&val)[8]) { put8(o + row0 + a0, val); });
}

template <typename T, int NFT>
struct FGeom {
  static constexpr int Fp = 32 * NFT;
  static constexpr int KP = Fp + 16 / (int)sizeof(T);  // Phi(K) tile pitch (elements)
  static constexpr int VP = kDV + 16 / (int)sizeof(T);
  static constexpr int RP = 68;
  static constexpr int k_bytes = kFC * KP * (int)sizeof(T);
  static constexpr int v_bytes = kFC * VP * (int)sizeof(T);
  static constexpr int red_bytes = 4 * kFC * RP * 4;
  // bf16: the chunk's Phi(Q) rows are staged in LDS like Phi(K) (fp32 rows would not fit beside them; they are
  // read from global memory)
  static constexpr bool QLDS = sizeof(T) == 2;
  static constexpr int q_bytes = QLDS ? k_bytes : 0;
  static constexpr int lds = k_bytes + q_bytes + v_bytes + red_bytes + Fp * 4;
  static constexpr int EL = 16 / (int)sizeof(T);            // elements per 16-byte piece
  static constexpr int FPIECES = kFC * (Fp / EL) / 256;     // 16-byte pieces of a feature chunk per thread
  static constexpr int VPIECES = (kFC * (kDV / EL) + 255) / 256;
  static_assert(kFC * (Fp / EL) % 256 == 0, "a feature chunk is a whole number of pieces per thread");
};

// Raw operands of the fused staging: q and k rows [BH][T][d], the phase table [T][d] (revolutions), the anchors
// omega [nph][d] and the gate constant.
struct FuseIn {
  const __bf16* uq;
  const __bf16* uk;
  const float* rho;
  const float* omega;
  int nph, H;
  float kr;
};

// FUSED (bf16): Phi(Q) and Phi(K) are not read from the workspace; each thread featurizes 8 dims of one token of
// the chunk (map KIND, NH) straight into the LDS tiles while staging it.
template <typename T, int NFT, bool STATE_ONLY, bool FUSED = false, int KIND = 0, int NH = 0>
__global__ __launch_bounds__(256, 1) void feat_prefill_kernel(const T* __restrict__ phiq, const T* __restrict__ phik,
                                                              const T* __restrict__ v, T* __restrict__ out,
                                                              float* __restrict__ S, float* __restrict__ z, int Tn,
                                                              int Freal, float ceps, int P, int SPL,
                                                              float* __restrict__ slots, int shared_last, FuseIn fu) {
  using G = FGeom<T, NFT>;
  typedef typename FragT<T>::type Frag;
  static_assert(NFT % 4 == 0, "feature tiles are dealt to four waves");
  constexpr int NW = NFT / 4, Fp = G::Fp, KP = G::KP, VP = G::VP, RP = G::RP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* KT = reinterpret_cast<T*>(smem);
  T* QT = reinterpret_cast<T*>(smem + G::k_bytes);  // (bf16 only)
  T* VT = reinterpret_cast<T*>(smem + G::k_bytes + G::q_bytes);
  float* red = reinterpret_cast<float*>(smem + G::k_bytes + G::q_bytes + G::v_bytes);
  float* zs = reinterpret_cast<float*>(smem + G::k_bytes + G::q_bytes + G::v_bytes + G::red_bytes);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  // pass 1 (STATE_ONLY) runs part sp_ of SPL of every piece but the last (the final piece's state comes out of
  // pass 3), so consecutive workgroups, which go to different XCDs, all have work; pass 3 runs whole pieces
  const int bh = STATE_ONLY ? blockIdx.x / ((P - 1) * SPL) : blockIdx.x / P;
  const int p = STATE_ONLY ? (blockIdx.x / SPL) % (P - 1) : blockIdx.x % P;
  const int sp_ = STATE_ONLY ? blockIdx.x % SPL : 0;
  const int nch = (Tn + kFC - 1) / kFC;
  int t_lo = (int)((long long)p * nch / P) * kFC;
  int t_hi = min(Tn, (int)((long long)(p + 1) * nch / P) * kFC);
  if (STATE_ONLY) {  // never empty: every piece has at least SPL chunks
    const int pc = (t_hi - t_lo + kFC - 1) / kFC, base = t_lo;
    t_lo = base + (sp_ * pc / SPL) * kFC;
    t_hi = min(t_hi, base + ((sp_ + 1) * pc / SPL) * kFC);
  }
  constexpr size_t SLOT = (size_t)Fp * (kDV + 1);  // S [Fp][d_v], then z [Fp]
  auto slot = [&](int q, int part) { return slots + (((size_t)bh * P + q) * SPL + part) * SLOT; };
  const T* qp = phiq + (size_t)bh * Tn * Fp;
  const T* kp = phik + (size_t)bh * Tn * Fp;
  const T* vp = v + (size_t)bh * Tn * kDV;
  T* op = out + (size_t)bh * Tn * kDV;
  float* Sp = S ? S + (size_t)bh * Freal * kDV : nullptr;
  float* zp = z ? z + (size_t)bh * Freal : nullptr;

  // state slice: tile i of this wave is feature tile ft = w + 4 i; register 4 j + i4 of (i, vt) holds
  // S[32 ft + 8 j + 4 h + i4][32 vt + n32]
  f32x16 Sacc[NW][2];
#pragma unroll
  for (int i = 0; i < NW; i++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++) zero16(Sacc[i][vt]);
  for (int f = tid; f < Fp; f += 256) zs[f] = 0.0f;
  // add a state of `rows` rows ([rows][d_v] then [rows]) to the wave's tiles and to zs (each zs entry is
  // touched by the same thread here as in the zeroing above)
  // The caller's row of internal feature f: the four-channel map keeps its shared feature last internally
  // (feature 3 d) but first in the caller's compact state
  auto user_row = [&](int f) { return shared_last ? (f == Freal - 1 ? 0 : f + 1) : f; };
  auto add_state = [&](const float* s_, const float* z_, int rows, bool user) {
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int f = 32 * (w + 4 * i) + 8 * (r >> 2) + 4 * h + (r & 3);
          if (f < rows) Sacc[i][vt][r] += s_[(size_t)(user ? user_row(f) : f) * kDV + 32 * vt + n32];
        }
    for (int f = tid; f < rows; f += 256) zs[f] += z_[user ? user_row(f) : f];
  };
  // the same for a slot (all Fp rows, internal order): without the per-element guard the loads need not wait
  // for one another
  auto add_slot = [&](const float* s_) {
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int r = 0; r < 16; r++)
          Sacc[i][vt][r] += s_[(size_t)(32 * (w + 4 * i) + 8 * (r >> 2) + 4 * h + (r & 3)) * kDV + 32 * vt + n32];
    for (int f = tid; f < Fp; f += 256) zs[f] += s_[(size_t)Fp * kDV + f];
  };
  if (P == 1) {
    if (Sp) add_state(Sp, zp, Freal, true);
  } else if (STATE_ONLY) {
    if (p == 0 && sp_ == 0 && Sp) {
      add_state(Sp, zp, Freal, true);
      float* sp1 = slot(P - 1, 0);  // the start state of pass 3's piece 0, internal rows, padded with zeros
      for (int e = tid; e < Fp * kDV; e += 256) {
        const int f = e / kDV;
        sp1[e] = f < Freal ? Sp[(size_t)user_row(f) * kDV + e % kDV] : 0.0f;
      }
      for (int f = tid; f < Fp; f += 256) sp1[Fp * kDV + f] = f < Freal ? zp[user_row(f)] : 0.0f;
    }
  } else if (p == 0) {
    if (Sp) add_slot(slot(P - 1, 0));
  } else {
    for (int q = 0; q < p; q++)
      for (int part = 0; part < SPL; part++) add_slot(slot(q, part));
  }

  // Staging of a chunk's Phi(K) (and, bf16 output pass, Phi(Q)) and V rows, zero past its end.  With few pieces
  // per thread (PF) the next chunk's rows are loaded into registers while the current chunk computes; otherwise
  // the loads are issued in groups of GS pieces per operand before the group's LDS writes, so the staging waits
  // for memory once per group instead of once per piece.
  constexpr int EL = G::EL, FPC = Fp / EL;
  constexpr bool LQ = G::QLDS && !STATE_ONLY;
  constexpr int NPIECE = G::FPIECES * (LQ ? 2 : 1) + G::VPIECES;
  constexpr bool PF = FUSED || NPIECE <= 12;
  static_assert(!FUSED || sizeof(T) == 2, "the fused staging is for bf16 operands");
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 pk[PF && !FUSED ? G::FPIECES : 1], pq[PF && LQ && !FUSED ? G::FPIECES : 1], pv[PF ? G::VPIECES : 1];
  // (FUSED) this thread's token s = fs of a chunk and dims fa0 .. fa0 + 7: raw q and k pieces, their phases and
  // anchors
  const int fs = tid >> 3, fj = tid & 7, fa0 = 8 * fj;
  u32x4 fk = zero4, fq = zero4;
  float4 fr0 = make_float4(0.f, 0.f, 0.f, 0.f), fr1 = fr0;
  float fom[8];
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < 8; i++) fom[i] = anchor_rev(fu.omega[(size_t)((bh % fu.H) % fu.nph) * kD + fa0 + i]);
  }
  auto pf_load = [&](int c0, int cnv) {
    if constexpr (FUSED) {
      const size_t row = (size_t)(c0 + min(fs, cnv - 1));
      fk = *reinterpret_cast<const u32x4*>(fu.uk + ((size_t)bh * Tn + row) * kD + fa0);
      if constexpr (LQ) fq = *reinterpret_cast<const u32x4*>(fu.uq + ((size_t)bh * Tn + row) * kD + fa0);
      fr0 = *reinterpret_cast<const float4*>(fu.rho + row * kD + fa0);
      fr1 = *reinterpret_cast<const float4*>(fu.rho + row * kD + fa0 + 4);
    }
#pragma unroll
    for (int i = 0; i < (FUSED ? 0 : G::FPIECES); i++) {
      const int e = tid + 256 * i, s = e / FPC, c = (e % FPC) * EL;
      const size_t off = (size_t)(c0 + min(s, cnv - 1)) * Fp + c;
      pk[PF ? i : 0] = *reinterpret_cast<const u32x4*>(kp + off);
      if constexpr (LQ) pq[PF ? i : 0] = *reinterpret_cast<const u32x4*>(qp + off);
    }
#pragma unroll
    for (int i = 0; i < G::VPIECES; i++) {
      const int e = tid + 256 * i, s = e / (kDV / EL), c = (e % (kDV / EL)) * EL;
      if (e < kFC * (kDV / EL)) pv[PF ? i : 0] = *reinterpret_cast<const u32x4*>(vp + (size_t)(c0 + min(s, cnv - 1)) * kDV + c);
    }
  };
  auto pf_store = [&](int cnv) {
    if constexpr (FUSED) {
      const float rh[8] = {fr0.x, fr0.y, fr0.z, fr0.w, fr1.x, fr1.y, fr1.z, fr1.w};
      float x[8];
      const bf16x8 kb = __builtin_bit_cast(bf16x8, fk);
#pragma unroll
      for (int i = 0; i < 8; i++) x[i] = (float)kb[i];
      T* krow = KT + fs * KP + fa0;
      if (fs < cnv) {
        ext_features8<KIND, NH, false>(x, rh, fom, fu.kr, fj, Fp,
                                       [&](int row0, const float (&val)[8]) { put8(krow + row0, val); });
      } else {
        for (int f = 0; f < Fp; f += kD) *reinterpret_cast<u32x4*>(krow + f) = zero4;  // keys past the end
      }
      if constexpr (LQ) {
        const bf16x8 qb = __builtin_bit_cast(bf16x8, fq);
#pragma unroll
        for (int i = 0; i < 8; i++) x[i] = (float)qb[i];
        T* qrow_ = QT + fs * KP + fa0;
        ext_features8<KIND, NH, true>(x, rh, fom, fu.kr, fj, Fp,
                                      [&](int row0, const float (&val)[8]) { put8(qrow_ + row0, val); });
      }
    }
#pragma unroll
    for (int i = 0; i < (FUSED ? 0 : G::FPIECES); i++) {
      const int e = tid + 256 * i, s = e / FPC, c = (e % FPC) * EL;
      *reinterpret_cast<u32x4*>(KT + s * KP + c) = s < cnv ? pk[PF ? i : 0] : zero4;
      if constexpr (LQ) *reinterpret_cast<u32x4*>(QT + s * KP + c) = pq[PF ? i : 0];
    }
#pragma unroll
    for (int i = 0; i < G::VPIECES; i++) {
      const int e = tid + 256 * i, s = e / (kDV / EL), c = (e % (kDV / EL)) * EL;
      if (e < kFC * (kDV / EL)) *reinterpret_cast<u32x4*>(VT + s * VP + c) = s < cnv ? pv[PF ? i : 0] : zero4;
    }
  };
  if constexpr (PF) {
    if (t_lo < t_hi) pf_load(t_lo, min(kFC, t_hi - t_lo));
  }
  for (int t0 = t_lo; t0 < t_hi; t0 += kFC) {
    const int nv = min(kFC, t_hi - t0);
    if constexpr (PF) {
      pf_store(nv);
      __syncthreads();
      if (t0 + kFC < t_hi) pf_load(t0 + kFC, min(kFC, t_hi - t0 - kFC));
    } else {
      constexpr int GS = G::FPIECES < 4 ? G::FPIECES : 4;
#pragma unroll
      for (int g0 = 0; g0 < G::FPIECES; g0 += GS) {
        u32x4 kr[GS], qr[GS];
#pragma unroll
        for (int i = 0; i < GS; i++) {
          if (g0 + i < G::FPIECES) {
            const int e = tid + 256 * (g0 + i), s = e / FPC, c = (e % FPC) * EL, sc = t0 + min(s, nv - 1);
            kr[i] = *reinterpret_cast<const u32x4*>(kp + (size_t)sc * Fp + c);
            if constexpr (LQ) qr[i] = *reinterpret_cast<const u32x4*>(qp + (size_t)sc * Fp + c);
          }
        }
#pragma unroll
        for (int i = 0; i < GS; i++) {
          if (g0 + i < G::FPIECES) {
            const int e = tid + 256 * (g0 + i), s = e / FPC, c = (e % FPC) * EL;
            *reinterpret_cast<u32x4*>(KT + s * KP + c) = s < nv ? kr[i] : zero4;
            if constexpr (LQ) *reinterpret_cast<u32x4*>(QT + s * KP + c) = qr[i];
          }
        }
      }
      {
        u32x4 vr[G::VPIECES];
#pragma unroll
        for (int i = 0; i < G::VPIECES; i++) {
          const int e = tid + 256 * i, s = e / (kDV / EL), c = (e % (kDV / EL)) * EL;
          if (e < kFC * (kDV / EL)) vr[i] = *reinterpret_cast<const u32x4*>(vp + (size_t)(t0 + min(s, nv - 1)) * kDV + c);
        }
#pragma unroll
        for (int i = 0; i < G::VPIECES; i++) {
          const int e = tid + 256 * i, s = e / (kDV / EL), c = (e % (kDV / EL)) * EL;
          if (e < kFC * (kDV / EL)) *reinterpret_cast<u32x4*>(VT + s * VP + c) = s < nv ? vr[i] : zero4;
        }
      }
      __syncthreads();
    }

    if constexpr (!STATE_ONLY) {
    // this lane's query (column n32 of the transposed tiles), clamped into the chunk
    const int tc = t0 + min(n32, nv - 1);
    const T* qrow = G::QLDS ? QT + n32 * KP : qp + (size_t)tc * Fp;
    // per feature tile: its two query fragments feed the partial scores A^T[s][t] and, right away, the readout
    // against the state before this chunk (num^T += S^T Phi(Q)^T), so only two fragments are live at a time
    f32x16 at, num[2];
    zero16(at);
    zero16(num[0]);
    zero16(num[1]);
    float dz = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        const int base = 32 * (w + 4 * i) + 16 * kk;
        const Frag QF = slot_frag<T>(qrow, base, h);
        mma32(at, slot_frag<T>(KT + n32 * KP, base, h), QF);
#pragma unroll
        for (int s = 0; s < 8; s++) dz = fmaf((float)QF[s], zs[base + 8 * (s >> 2) + 4 * h + (s & 3)], dz);
#pragma unroll
        for (int vt = 0; vt < 2; vt++) {
          float x[8];
#pragma unroll
          for (int s = 0; s < 8; s++) x[s] = Sacc[i][vt][8 * kk + s];
          mma32(num[vt], pack8f<T>(x), QF);
        }
      }
    // masked partial scores (s <= t), their row sums, and V^T P
    float lo[8], hi8[8];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int s = 8 * (r >> 2) + 4 * h + (r & 3);
      const float a = s > n32 ? 0.0f : at[r];
      if (r < 8) lo[r] = a;
      else hi8[r - 8] = a;
    }
    const Frag P0 = pack8f<T>(lo), P1 = pack8f<T>(hi8);
    float den = frag_sum(P1, frag_sum(P0, dz));
#pragma unroll
    for (int vt = 0; vt < 2; vt++) {
      mma32(num[vt], lds_tokfrag(VT, VP, 0, 32 * vt, l), P0);
      mma32(num[vt], lds_tokfrag(VT, VP, 16, 32 * vt, l), P1);
    }
    den = xor32_sum(den);
    float* rw = red + (w * kFC + n32) * RP;
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        *reinterpret_cast<float4*>(rw + 32 * vt + 8 * j + 4 * h) =
            make_float4(num[vt][4 * j], num[vt][4 * j + 1], num[vt][4 * j + 2], num[vt][4 * j + 3]);
    if (h == 0) rw[64] = den;
    __syncthreads();
    {
      const int row = tid >> 3, c0 = 8 * (tid & 7);
      if (row < nv) {
        constexpr int WS = kFC * RP;
        const float* b0 = red + row * RP;
        const float dsum = ((b0[64] + b0[WS + 64]) + b0[2 * WS + 64]) + b0[3 * WS + 64];
        const float inv = 1.0f / (dsum + ceps);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; e++)
          o[e] = (((b0[c0 + e] + b0[WS + c0 + e]) + b0[2 * WS + c0 + e]) + b0[3 * WS + c0 + e]) * inv;
        if constexpr (sizeof(T) == 2) {
          bf16x8 ov;
#pragma unroll
          for (int e = 0; e < 8; e++) ov[e] = (__bf16)o[e];
          *reinterpret_cast<bf16x8*>(op + (size_t)(t0 + row) * kDV + c0) = ov;
        } else {
          float* dst = reinterpret_cast<float*>(op + (size_t)(t0 + row) * kDV + c0);
          *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    }
    }  // !STATE_ONLY
    // state update S += Phi(K)^T V and z += Phi(K)^T 1 over this wave's feature tiles
#pragma unroll
    for (int i = 0; i < NW; i++) {
      const int ft = w + 4 * i;
      float zsum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const Frag A = lds_tokfrag(KT, KP, 16 * ks, 32 * ft, l);
        zsum = frag_sum(A, zsum);
#pragma unroll
        for (int vt = 0; vt < 2; vt++) mma32(Sacc[i][vt], A, lds_tokfrag(VT, VP, 16 * ks, 32 * vt, l));
      }
      zsum = xor32_sum(zsum);
      // every wave read zs for this chunk's readout before the reduction barrier; each wave updates its own tiles
      if (h == 0) zs[32 * ft + n32] += zsum;
    }
    __syncthreads();  // tiles and the reduction buffer are reused by the next chunk
  }
  auto store_state = [&](float* s_, float* z_, int rows, bool user) {
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int f = 32 * (w + 4 * i) + 8 * (r >> 2) + 4 * h + (r & 3);
          if (f < rows) s_[(size_t)(user ? user_row(f) : f) * kDV + 32 * vt + n32] = Sacc[i][vt][r];
        }
    for (int f = tid; f < rows; f += 256) z_[user ? user_row(f) : f] = zs[f];
  };
  if (STATE_ONLY) store_state(slot(p, sp_), slot(p, sp_) + Fp * kDV, Fp, false);
  else if (Sp && p == P - 1) store_state(Sp, zp, Freal, true);
}

// Pieces per sequence: as many as keep every sequence's pieces on distinct compute units (at most 8, at most
// one per chunk); 1 (no split) when there are at least as many sequences as compute units.
int ext_pieces(int B, int H, int Tn) {
  const long long BH = (long long)B * H, nch = (Tn + kFC - 1) / kFC;
  long long P = device_cus() / BH;
  if (P > 8) P = 8;
  if (P > nch) P = nch;
  return P < 1 ? 1 : (int)P;
}

// Workgroups per piece in pass 1: only P - 1 pieces of a sequence have a state to hand on, so each one's chunks
// are split over this many workgroups (each writes a slot of its own, and pass 3 sums them) to keep the compute
// units busy: at most 8, and never more than the chunks of the smallest piece.
int ext_split(int B, int H, int Tn) {
  const int P = ext_pieces(B, H, Tn);
  if (P < 2) return 1;
  const long long BH = (long long)B * H, nch = (Tn + kFC - 1) / kFC;
  long long S = device_cus() / (BH * (P - 1));
  if (S > 8) S = 8;
  if (S > nch / P) S = nch / P;
  return S < 1 ? 1 : (int)S;
}

template <typename Kern>
hipError_t set_lds_once(Kern k, int bytes, std::atomic<bool>& flag) {
  if (flag.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) flag.store(true, std::memory_order_release);
  return e;
}

// bytes of the position phase table [T][d] fp32 at the front of a bf16 call's workspace (256-byte aligned)
size_t ext_rho_bytes(int T) { return ((size_t)T * kD * sizeof(float) + 255) & ~(size_t)255; }

template <typename TIn, int KIND, int NH, int NFT>
hipError_t launch_fp_t(const void* q, const void* k, const void* v, int B, int H, int Tn, int64_t pos0,
                       const MethodConsts& mc, float* S, float* z, void* out, void* ws, int Freal,
                       hipStream_t stream) {
  using G = FGeom<TIn, NFT>;
  // bf16 featurizes while staging (FUSED); fp32 materializes Phi(Q) and Phi(K) first (its tiles would not fit
  // in LDS side by side)
  constexpr bool FUSED = sizeof(TIn) == 2;
  const int BH = B * H, ntiles = (Tn + 31) / 32;
  TIn* phiq = nullptr;
  TIn* phik = nullptr;
  float* rho = nullptr;
  float* slots = nullptr;
  hipError_t e = hipSuccess;
  if constexpr (FUSED) {
    rho = static_cast<float*>(ws);
    slots = reinterpret_cast<float*>(static_cast<char*>(ws) + ext_rho_bytes(Tn));
    if ((e = launch_phase_table(rho, Tn, pos0, mc.log2_base, stream)) != hipSuccess) return e;
  } else {
    phiq = static_cast<TIn*>(ws);
    phik = phiq + (size_t)BH * Tn * G::Fp;
    slots = reinterpret_cast<float*>(phik + (size_t)BH * Tn * G::Fp);
    const dim3 fgrid((unsigned)((long long)BH * ntiles)), fblk(256);
    hipLaunchKernelGGL((featurize_ext_kernel<TIn, TIn, KIND, NH, true>), fgrid, fblk, 0, stream,
                       static_cast<const TIn*>(q), phiq, H, Tn, G::Fp, pos0, mc.omega, mc.nph, mc.log2_base, mc.kr,
                       ntiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((featurize_ext_kernel<TIn, TIn, KIND, NH, false>), fgrid, fblk, 0, stream,
                       static_cast<const TIn*>(k), phik, H, Tn, G::Fp, pos0, mc.omega, mc.nph, mc.log2_base, mc.kr,
                       ntiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const FuseIn fu{reinterpret_cast<const __bf16*>(q), reinterpret_cast<const __bf16*>(k), rho, mc.omega, mc.nph, H,
                  mc.kr};
  static std::atomic<bool> attr[64], attr1[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if ((e = set_lds_once(feat_prefill_kernel<TIn, NFT, false, FUSED, KIND, NH>, G::lds, attr[dev])) != hipSuccess)
    return e;
  const int P = ext_pieces(B, H, Tn), SPL = ext_split(B, H, Tn);
  if (P > 1) {
    if ((e = set_lds_once(feat_prefill_kernel<TIn, NFT, true, FUSED, KIND, NH>, G::lds, attr1[dev])) != hipSuccess)
      return e;
    hipLaunchKernelGGL((feat_prefill_kernel<TIn, NFT, true, FUSED, KIND, NH>), dim3(BH * (P - 1) * SPL), dim3(256),
                       G::lds, stream, phiq, phik, static_cast<const TIn*>(v), static_cast<TIn*>(out), S, z, Tn,
                       Freal, mc.ceps, P, SPL, slots, KIND == 1 ? 1 : 0, fu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((feat_prefill_kernel<TIn, NFT, false, FUSED, KIND, NH>), dim3(BH * P), dim3(256), G::lds,
                     stream, phiq, phik, static_cast<const TIn*>(v), static_cast<TIn*>(out), S, z, Tn, Freal, mc.ceps,
                     P, SPL, slots, KIND == 1 ? 1 : 0, fu);
  return hipGetLastError();
}

}  // namespace

// padded feature count of a map: harmonics (2 + 4 nh) d, four-channel 3 d + 1, rounded up to 128
int ext_features_padded(int nh_or_zero) {
  const int f = nh_or_zero > 0 ? (2 + 4 * nh_or_zero) * kD : 3 * kD + 1;
  return (f + 127) / 128 * 128;
}

size_t ext_prefill_ws_bytes(int B, int H, int T, sanatan_dtype t, int nh_or_zero) {
  const size_t Fp = ext_features_padded(nh_or_zero);
  const int P = ext_pieces(B, H, T);
  const size_t slots = P > 1 ? (size_t)B * H * P * ext_split(B, H, T) * Fp * (kDV + 1) * sizeof(float) : 0;
  // bf16: the phase table, then the piece slots; fp32: Phi(Q), Phi(K), then the piece slots (Phi's bytes are a
  // multiple of 4: Fp is a multiple of 128)
  if (t == SANATAN_BF16) return ext_rho_bytes(T) + slots;
  return 2 * (size_t)B * H * T * Fp * sizeof(float) + slots;
}

// nh_or_zero: 1 or 2 harmonics, or 0 for the four-channel compact map
hipError_t launch_ext_prefill(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                              int nh_or_zero, int64_t pos0, const MethodConsts& mc, float* S, float* z, void* out,
                              void* ws, hipStream_t stream) {
  const bool bf = t == SANATAN_BF16;
  switch (nh_or_zero) {
    case 0:
      return bf ? launch_fp_t<__bf16, 1, 0, 8>(q, k, v, B, H, T, pos0, mc, S, z, out, ws, 3 * kD + 1, stream)
                : launch_fp_t<float, 1, 0, 8>(q, k, v, B, H, T, pos0, mc, S, z, out, ws, 3 * kD + 1, stream);
    case 1:
      return bf ? launch_fp_t<__bf16, 0, 1, 12>(q, k, v, B, H, T, pos0, mc, S, z, out, ws, 6 * kD, stream)
                : launch_fp_t<float, 0, 1, 12>(q, k, v, B, H, T, pos0, mc, S, z, out, ws, 6 * kD, stream);
    case 2:
      return bf ? launch_fp_t<__bf16, 0, 2, 20>(q, k, v, B, H, T, pos0, mc, S, z, out, ws, 10 * kD, stream)
                : launch_fp_t<float, 0, 2, 20>(q, k, v, B, H, T, pos0, mc, S, z, out, ws, 10 * kD, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sanatan
