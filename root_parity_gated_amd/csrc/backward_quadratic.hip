// backward_quadratic.hip -- the feature gradients and dv of normalised causal power attention in quadratic form,
// bf16 operands, software-pipelined.
//
// SANATAN reading notes: the weights are w_ts = (kappa_ts / c)^p over s <= t (§2.6) with
// kappa_ts = <Phi(q_t), Phi(k_s)> (§2.3); the model is trained at p = 2 first (§4.1), which has no small-state
// recurrence, so its gradient runs over query-key tiles.  In the kernels' scaled units (weights kappa^p,
// Dn_t = sum_s kappa_ts^p + eps c^p, delta_t = <g_t, o_t>):
//   G_ts = p kappa_ts^(p-1) (<g_t, v_s> - delta_t) / Dn_t,
//   dPhi(q_t) = sum_{s<=t} G_ts Phi(k_s),  dPhi(k_s) = sum_{t>=s} G_ts Phi(q_t),  dv_s = sum_{t>=s} kappa_ts^p g_t / Dn_t.
//
// One kernel per side.  SIDE 0 (dPhi(q)): a wave owns 32 queries and walks the key blocks up to its own; SIDE 1
// (dPhi(k), dv): a wave owns 32 keys and walks the query blocks from its own to the end.  Four waves (128 owned
// tokens) per workgroup, one per SIMD, so that a wave holds all ten 32 x 32 fp32 gradient tiles of feature
// channels 1..5 in accumulators (channel 0 is the constant 1: it adds exactly d to every score and has no
// derivative), next to its 20 feature and 4 value fragments.  Per streamed block of 32 tokens:
//   scores:   kappa tile = 20 K-steps of 32x32x16 bf16 MFMA (+ d), and the <g, v> tile (4 K-steps);
//   weights:  G (and W = kappa^p / Dn on SIDE 1) formed in registers; with bf16 operands G enters the gradient
//             products as its bf16 rounding plus the bf16 rounding of the residual, since a row of G nearly
//             cancels (Phi(q_t) . dPhi(q_t) is ~0), so one rounding would leave an error of the order of the result;
//   products: dPhi += Phi^T G over the ten tiles (40 MFMAs), dv^T += g^T W (4 MFMAs, SIDE 1).
// The scores of block b + 1 are issued between the weight arithmetic of block b, so the matrix cores have
// independent work while that VALU runs.  The streamed tiles live in three LDS buffers (block b, b + 1 being
// read, b + 2 being written), so one barrier per block suffices; the rows of block b + 3 are loaded into
// registers meanwhile, through buffer loads whose range check returns zeros past the sequence's end.
#include <atomic>

#include "feature_tiles.h"

namespace sanatan {
namespace {

constexpr int kQB = 32;  // tokens per streamed block and per owned tile

struct Q2Geom {
  static constexpr int NF = kF - kD;         // staged features: channels 1..5
  static constexpr int NJ = NF / 16;         // K-steps of the score product
  static constexpr int NT = NF / 32;         // 32-feature gradient tiles
  static constexpr int FP = NF + 8;          // feature tile pitch (elements): rows 656 bytes apart
  static constexpr int VP = kDV + 16;        // value / gradient tile pitch: rows 160 bytes apart
  static constexpr int f_bytes = kQB * FP * 2;
  static constexpr int v_bytes = kQB * VP * 2;
  static constexpr int s_bytes = 3 * kQB * 4;  // SIDE 1: per query row a = p / Dn, -a delta, 1 / Dn
  static constexpr int buf_bytes = f_bytes + v_bytes + s_bytes;
  static constexpr int lds = 3 * buf_bytes;
  static constexpr int FPT = kQB * NF / 8 / 256;   // 16-byte feature pieces per thread and block
  static constexpr int VPT = kQB * kDV / 8 / 256;  // 16-byte value pieces per thread and block
  static_assert(FPT * 256 * 8 == kQB * NF && VPT * 256 * 8 == kQB * kDV, "pieces must divide evenly");
  static_assert(buf_bytes % 16 == 0, "buffers must stay 16-byte aligned");
};

// LDS read distances: score fragments kPD K-steps ahead of their MFMA; gradient-side fragments kRB - 1 tiles
// (two MFMAs each) ahead
constexpr int kPD = 4, kRB = 3;
constexpr int RB = kRB;

constexpr int kRawBufferWord3 = 0x00020000;

// Inputs of the fused Jacobian: the owned side's raw rows u [BH][T][d], the phase table [T][d] (revolutions),
// the anchors omega [nph][d] and the gate constant.
struct JacIn {
  const __bf16* u;
  const float* rho;
  const float* omega;
  int nph, H;
  float kr;
};  // descriptor word 3: the gfx9-family raw-buffer format

// Transposing reads of a token-major bf16 tile (the operand of lds_tokfrag): the lane's part of the byte
// address, fixed per lane, so that a read at (tok0, col0) only adds a constant to it.
__device__ __forceinline__ int tok_lane_bytes(int pitch, int l) {
  const int b = l >> 4, L = l & 15;
  return ((4 * (b >> 1) + (L >> 2)) * pitch + 16 * (b & 1) + 4 * (L & 3)) * 2;
}
typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
// lane (row l % 32, h) gets column col0 + l % 32 at tokens tok0 + 8 (i / 4) + 4 h + i % 4 (as lds_tokfrag);
// p = tile base + tok_lane_bytes(pitch, l)
__device__ __forceinline__ bf16x8 tokfrag_at(lds_cchar* p, int pitch, int tok0, int col0) {
  const u32x2 lo = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + (tok0 * pitch + col0) * 2)));
  const u32x2 hi = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + ((tok0 + 8) * pitch + col0) * 2)));
  const u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, r);
}

template <int P, int SIDE>
__global__ __launch_bounds__(256, 1) void bwd_quad_kernel(const __bf16* __restrict__ phiq,
                                                          const __bf16* __restrict__ phik,
                                                          const __bf16* __restrict__ v, const __bf16* __restrict__ g,
                                                          const float2* __restrict__ stats, JacIn jin,
                                                          __bf16* __restrict__ du, float* __restrict__ dom_part,
                                                          __bf16* __restrict__ dv, int Tn, int BH, int nqb) {
  using G = Q2Geom;
  constexpr int NJ = G::NJ, NT = G::NT, FP = G::FP, VP = G::VP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  // SIDE 0: heaviest (latest) query tiles first; SIDE 1: heaviest (earliest) key tiles first
  const int tile = SIDE == 0 ? nqb - 1 - (int)(blockIdx.x / BH) : (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const size_t sq = (size_t)bh * Tn;
  const int row0 = tile * 128 + 32 * w;  // this wave's first owned token
  const int own = row0 + n32, oc = min(own, Tn - 1);
  const int nblk = (Tn + kQB - 1) / kQB;
  // streamed blocks of the workgroup [bbeg, bend) and of this wave [alo, ahi]
  int bbeg, bend, alo, ahi;
  if constexpr (SIDE == 0) {
    bbeg = 0;
    bend = min(Tn - 1, tile * 128 + 127) / kQB + 1;
    alo = 0;
    ahi = row0 < Tn ? row0 / kQB : -1;
  } else {
    bbeg = tile * 4;
    bend = nblk;
    alo = row0 < Tn ? row0 / kQB : nblk;
    ahi = nblk - 1;
  }
  const __bf16* sfeat = (SIDE == 0 ? phik : phiq) + sq * kF + kD;  // streamed features, from channel 1
  const __bf16* sval = (SIDE == 0 ? v : g) + sq * kDV;             // streamed 64-wide rows
  const __bf16* ofeat = (SIDE == 0 ? phiq : phik) + sq * kF + kD;  // owned features
  const __bf16* oval = (SIDE == 0 ? g : v) + sq * kDV;             // owned 64-wide rows

  // ---- staging: block b's rows -> registers (buffer loads, zeros past the end) -> LDS buffer (b - bbeg) % 3
  u32x4 rf[G::FPT], rv[G::VPT];
  float2 rs = make_float2(0.0f, 0.0f);
  unsigned foff[G::FPT], voff[G::VPT];
#pragma unroll
  for (int p = 0; p < G::FPT; p++) {
    const int e = tid + 256 * p;
    foff[p] = (unsigned)(((e / (G::NF / 8)) * kF + (e % (G::NF / 8)) * 8) * 2);
  }
#pragma unroll
  for (int p = 0; p < G::VPT; p++) {
    const int e = tid + 256 * p;
    voff[p] = (unsigned)(((e / (kDV / 8)) * kDV + (e % (kDV / 8)) * 8) * 2);
  }
  auto fetch = [&](int b) {
    const int s0 = b * kQB;
    const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(sfeat + (size_t)s0 * kF), (short)0, (int)(((long long)(Tn - s0) * kF - kD) * 2), kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(sval + (size_t)s0 * kDV), (short)0, (int)((long long)(Tn - s0) * kDV * 2), kRawBufferWord3);
#pragma unroll
    for (int p = 0; p < G::FPT; p++) rf[p] = __builtin_amdgcn_raw_buffer_load_b128(fr, foff[p], 0, 0);
#pragma unroll
    for (int p = 0; p < G::VPT; p++) rv[p] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[p], 0, 0);
    if constexpr (SIDE == 1)
      if (tid < kQB) rs = s0 + tid < Tn ? stats[sq + s0 + tid] : make_float2(0.0f, 0.0f);
  };
  auto buf = [&](int b) { return smem + ((b - bbeg) % 3) * G::buf_bytes; };
  auto stash = [&](int b) {
    char* B_ = buf(b);
    __bf16* F = reinterpret_cast<__bf16*>(B_);
    __bf16* V = reinterpret_cast<__bf16*>(B_ + G::f_bytes);
#pragma unroll
    for (int p = 0; p < G::FPT; p++) {
      const int e = tid + 256 * p;
      *reinterpret_cast<u32x4*>(F + (e / (G::NF / 8)) * FP + (e % (G::NF / 8)) * 8) = rf[p];
    }
#pragma unroll
    for (int p = 0; p < G::VPT; p++) {
      const int e = tid + 256 * p;
      *reinterpret_cast<u32x4*>(V + (e / (kDV / 8)) * VP + (e % (kDV / 8)) * 8) = rv[p];
    }
    if constexpr (SIDE == 1) {
      if (tid < kQB) {
        // rows past the end carry 1 / Dn = 0: their weights are zero
        float* S = reinterpret_cast<float*>(B_ + G::f_bytes + G::v_bytes);
        const float a = (float)P * rs.x;
        S[tid] = a;
        S[kQB + tid] = -a * rs.y;
        S[2 * kQB + tid] = rs.x;
      }
    }
  };

  fetch(bbeg);
  // the owned operands: features of channels 1..5 (K-step j = 16 features) and the 64-wide rows
  bf16x8 XF[NJ], YF[4];
#pragma unroll
  for (int j = 0; j < NJ; j++)
    XF[j] = *reinterpret_cast<const bf16x8*>(ofeat + (size_t)oc * kF + 16 * j + 8 * h);
#pragma unroll
  for (int j = 0; j < 4; j++) YF[j] = *reinterpret_cast<const bf16x8*>(oval + (size_t)oc * kDV + 16 * j + 8 * h);
  float la = 0.0f, lnb = 0.0f;  // SIDE 0: the owned query's p / Dn and -(p / Dn) delta
  if constexpr (SIDE == 0) {
    const float2 st = stats[sq + oc];
    la = (float)P * st.x;
    lnb = -la * st.y;
  }
  stash(bbeg);
  if (bbeg + 1 < bend) {
    fetch(bbeg + 1);
    stash(bbeg + 1);
  }
  if (bbeg + 2 < bend) fetch(bbeg + 2);
  __syncthreads();

  f32x16 acc[NT], accv[2];
#pragma unroll
  for (int f = 0; f < NT; f++) zero16(acc[f]);
  zero16(accv[0]);
  zero16(accv[1]);
  // score and <g, v> tiles of two consecutive blocks, by block parity
  f32x16 sc[2], gv[2];
  f32x16 cz;
#pragma unroll
  for (int i = 0; i < 16; i++) cz[i] = 0.0f;

  // Weights of the current block.  Register i of a tile is row r = 8 (i / 4) + 4 h + i % 4 of the block, column
  // n32 (the owned token).  SIDE 1 reads the per-row scalars of registers 2 jj and 2 jj + 1 (rows 8 (jj / 2) +
  // 4 h + 2 (jj % 2) + 0..1) a little ahead of their use.
  bf16x8 G0, G1, R0, R1, W0, W1;
  float gw[16], ww[16];
  float2 qa[8], qn[8], qc[8];
  auto ldq = [&](const char* Bc, int jj) {
    const float* S = reinterpret_cast<const float*>(Bc + G::f_bytes + G::v_bytes);
    const int r = 8 * (jj >> 1) + 4 * h + 2 * (jj & 1);
    qa[jj] = *reinterpret_cast<const float2*>(S + r);
    qn[jj] = *reinterpret_cast<const float2*>(S + kQB + r);
    qc[jj] = *reinterpret_cast<const float2*>(S + 2 * kQB + r);
  };
  auto weight = [&](const f32x16& sct, const f32x16& gvt, int i, bool diag) {
    const int r = 8 * (i >> 2) + 4 * h + (i & 3);
    const float kap = sct[i] + (float)kD;  // channel 0 adds exactly d
    const float kp1 = P == 2 ? kap : 1.0f;
    float a, nb;
    if constexpr (SIDE == 0) {
      a = la;
      nb = lnb;
    } else {
      a = (i & 1) ? qa[i >> 1].y : qa[i >> 1].x;
      nb = (i & 1) ? qn[i >> 1].y : qn[i >> 1].x;
    }
    float gg = kp1 * fmaf(a, gvt[i], nb);
    // the diagonal block: SIDE 0 drops keys after the query, SIDE 1 queries before the key
    const bool drop = SIDE == 0 ? r > n32 : r < n32;
    gw[i] = diag && drop ? 0.0f : gg;
    if constexpr (SIDE == 1) {
      const float wt = (P == 2 ? kap * kap : kap) * ((i & 1) ? qc[i >> 1].y : qc[i >> 1].x);
      ww[i] = diag && drop ? 0.0f : wt;
    }
  };
  // pack registers o .. o + 7 of the weights: G (and its residual) and W
  auto pack_half = [&](int o, bf16x8& Gh, bf16x8& Rh, bf16x8& Wh) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; i++) x[i] = gw[o + i];
    Gh = pack8f<__bf16>(x);
    Rh = residual8<__bf16>(x, Gh);
    if constexpr (SIDE == 1) {
#pragma unroll
      for (int i = 0; i < 8; i++) x[i] = ww[o + i];
      Wh = pack8f<__bf16>(x);
    }
  };

  // Phase A: the score tiles of block bn (buffer Bn) into parity par ^ 1 (with NXT), and (with CUR) registers
  // 0..7 of block bc's weights (parity par) formed between their MFMAs, one register per K-step.
  auto phase_a = [&](auto Par, auto Nxt, auto Cur, const char* Bn, const char* Bc, bool diag) {
    constexpr int par = decltype(Par)::value;
    constexpr bool nxt = decltype(Nxt)::value, cur = decltype(Cur)::value;
    lds_cchar* frow = (lds_cchar*)Bn + (n32 * FP + 8 * h) * 2;
    lds_cchar* vrow = (lds_cchar*)Bn + G::f_bytes + (n32 * VP + 8 * h) * 2;
    asm volatile("" : "+v"(frow), "+v"(vrow));
    constexpr int PD = kPD;  // feature fragments are read PD K-steps ahead of their MFMA
    bf16x8 Ar[PD];
    if constexpr (nxt) {
#pragma unroll
      for (int j = 0; j < PD; j++) Ar[j] = *(lds_bf16x8*)(frow + 32 * j);
    }
    if constexpr (cur && SIDE == 1) {
      ldq(Bc, 0);
      ldq(Bc, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJ + 4; j++) {
      if constexpr (nxt) {
        if (j < NJ) {
          const bf16x8 A = Ar[j % PD];
          if (j == 0)
            sc[par ^ 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, XF[0], cz, 0, 0, 0);
          else
            mma32(sc[par ^ 1], A, XF[j]);
          if (j + PD < NJ) Ar[j % PD] = *(lds_bf16x8*)(frow + 32 * (j + PD));
        } else {
          const bf16x8 Vf = *(lds_bf16x8*)(vrow + 32 * (j - NJ));
          if (j == NJ)
            gv[par ^ 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Vf, YF[0], cz, 0, 0, 0);
          else
            mma32(gv[par ^ 1], Vf, YF[j - NJ]);
        }
      }
      if constexpr (cur) {
        if (j < 8) {
          if (SIDE == 1 && (j & 1) && (j >> 1) + 2 < 4) ldq(Bc, (j >> 1) + 2);
          weight(sc[par], gv[par], j, diag);
        } else if (j == 8) {
          pack_half(0, G0, R0, W0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int tf_lane = tok_lane_bytes(FP, l), tv_lane = tok_lane_bytes(VP, l);
  // Phase B: the gradient products of block bc, first over its keys 0..15 (G0, R0) for all ten tiles, with
  // registers 8..15 of the weights formed between them, then over keys 16..31 (G1, R1).
  auto phase_b = [&](auto Par, const char* Bc, bool diag) {
    constexpr int par = decltype(Par)::value;
    // (opaque to the optimiser, so that every read adds its constant in the instruction's offset field
    // instead of the loop keeping one hoisted address register per read)
    lds_cchar* F = (lds_cchar*)Bc + tf_lane;
    lds_cchar* V = (lds_cchar*)Bc + G::f_bytes + tv_lane;
    asm volatile("" : "+v"(F), "+v"(V));
    // Phi^T fragments (tokens tok0.. of the block as K-slots, feature column n32 of tile f), RB - 1 tiles ahead
    bf16x8 A[RB];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const int tok0 = 16 * hf;
#pragma unroll
      for (int f = 0; f < RB - 1; f++) A[f] = tokfrag_at(F, FP, tok0, 32 * f);
      if (hf == 0 && SIDE == 1) {
        ldq(Bc, 4);
        ldq(Bc, 5);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NT; f++) {
        if (f + RB - 1 < NT) A[(f + RB - 1) % RB] = tokfrag_at(F, FP, tok0, 32 * (f + RB - 1));
        mma32(acc[f], A[f % RB], hf ? G1 : G0);
        mma32(acc[f], A[f % RB], hf ? R1 : R0);
        if (hf == 0) {
          if (f < 8) {
            if (SIDE == 1 && (f & 1) && (f >> 1) + 6 < 8) ldq(Bc, (f >> 1) + 6);
            weight(sc[par], gv[par], 8 + f, diag);
          } else if (f == 8) {
            pack_half(8, G1, R1, W1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (SIDE == 1) {
#pragma unroll
      for (int vt = 0; vt < 2; vt++) {
        mma32(accv[vt], tokfrag_at(V, VP, 0, 32 * vt), W0);
        mma32(accv[vt], tokfrag_at(V, VP, 16, 32 * vt), W1);
      }
    }
  };
  auto active = [&](int b) { return b >= alo && b <= ahi; };
  // one step per streamed block b; the parity names the score tiles of block b at compile time
  auto step = [&](auto Par, int b) {
    constexpr int par = decltype(Par)::value;
    if (b + 2 < bend) stash(b + 2);
    if (b + 3 < bend) fetch(b + 3);
    const bool cur = active(b), nxt = b + 1 < bend && active(b + 1);
    const bool diag = SIDE == 0 ? b == ahi : b == alo;
    const char* Bc = buf(b);
    const char* Bn = buf(b + 1);
    if (nxt && cur)
      phase_a(Par, std::true_type(), std::true_type(), Bn, Bc, diag);
    else if (nxt)
      phase_a(Par, std::true_type(), std::false_type(), Bn, Bc, diag);
    else if (cur)
      phase_a(Par, std::false_type(), std::true_type(), Bn, Bc, diag);
    if (cur) phase_b(Par, Bc, diag);
    __syncthreads();
  };
  // the first block's scores (parity 0)
  if (active(bbeg))
    phase_a(std::integral_constant<int, 1>(), std::true_type(), std::false_type(), buf(bbeg), buf(bbeg), false);
  for (int b = bbeg; b < bend; b += 2) {
    step(std::integral_constant<int, 0>(), b);
    if (b + 1 >= bend) break;
    step(std::integral_constant<int, 1>(), b + 1);
  }

  // ---- the feature map's Jacobian, fused: lane (n32, h) holds, for its owned token, the gradient of channel c
  // (1..5) at dim 32 e + 8 (i / 4) + 4 h + i % 4 in register i of tile 2 (c - 1) + e.  It writes du for those dims
  // and the wave sums the omega gradients of its 32 tokens per dim in a fixed order (through a wave-private LDS
  // tile), one partial row per 32-token tile of the sequence.
  const bool valid = own < Tn;
  float* red = reinterpret_cast<float*>(smem) + w * (kQB * (kD + 1));
  const int hd = bh % jin.H;
  const float* omrow = jin.omega + (size_t)(hd % jin.nph) * kD;
  const __bf16* urow = jin.u + (sq + oc) * kD;
  const float* rrow = jin.rho + (size_t)oc * kD;
  __syncthreads();  // the streamed-block buffers are free
#pragma unroll
  for (int e = 0; e < 2; e++) {
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int a0 = 32 * e + 8 * m + 4 * h;
      const u32x2 uw = *reinterpret_cast<const u32x2*>(urow + a0);
      const bf16x4 ub = __builtin_bit_cast(bf16x4, uw);
      const float4 rh = *reinterpret_cast<const float4*>(rrow + a0);
      const float4 om = *reinterpret_cast<const float4*>(omrow + a0);
      const float rha[4] = {rh.x, rh.y, rh.z, rh.w}, oma[4] = {om.x, om.y, om.z, om.w};
      float dus[4];
#pragma unroll
      for (int i4 = 0; i4 < 4; i4++) {
        const int i = 4 * m + i4;
        float dom;
        feature_vjp((float)ub[i4], rha[i4], anchor_rev(oma[i4]), jin.kr, acc[e][i], acc[2 + e][i], acc[4 + e][i],
                    acc[6 + e][i], acc[8 + e][i], dus[i4], dom);
        red[n32 * (kD + 1) + a0 + i4] = valid ? dom : 0.0f;
      }
      if (valid) {
        const u32x2 o = {pack_bf16x2(dus[0], dus[1]), pack_bf16x2(dus[2], dus[3])};
        *reinterpret_cast<u32x2*>(du + (sq + own) * kD + a0) = o;
      }
    }
  }
  __syncthreads();
  if (row0 < Tn) {
    float sum = 0.0f;
    for (int r = 0; r < kQB; r++) sum += red[r * (kD + 1) + l];
    dom_part[((size_t)bh * nblk + row0 / kQB) * kD + l] = sum;
  }
  if (!valid) return;
  if constexpr (SIDE == 1) {
    __bf16* dvp = dv + (sq + own) * kDV;
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const unsigned lo = pack_bf16x2(accv[vt][4 * j], accv[vt][4 * j + 1]);
        const unsigned hi = pack_bf16x2(accv[vt][4 * j + 2], accv[vt][4 * j + 3]);
        *reinterpret_cast<u32x2*>(dvp + 32 * vt + 8 * j + 4 * h) = (u32x2){lo, hi};
      }
  }
}

template <typename Kern>
hipError_t set_lds_attr(Kern k, int bytes, std::atomic<bool>& flag) {
  if (flag.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) flag.store(true, std::memory_order_release);
  return e;
}

template <int P>
hipError_t launch_t(const __bf16* phiq, const __bf16* phik, const __bf16* v, const __bf16* g, const float2* stats,
                    int B, int H, int Tn, const __bf16* q, const __bf16* k, const float* rho, const float* omega,
                    int nph, float kr, __bf16* dq, __bf16* dk, __bf16* dv, float* dom_q, float* dom_k,
                    hipStream_t stream) {
  static std::atomic<bool> attr[2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const int BH = B * H, nqb = (Tn + 127) / 128;
  hipError_t e = set_lds_attr(bwd_quad_kernel<P, 0>, Q2Geom::lds, attr[0][dev]);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_quad_kernel<P, 0>), dim3(BH * nqb), dim3(256), Q2Geom::lds, stream, phiq, phik, v, g,
                     stats, JacIn{q, rho, omega, nph, H, kr}, dq, dom_q, (__bf16*)nullptr, Tn, BH, nqb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = set_lds_attr(bwd_quad_kernel<P, 1>, Q2Geom::lds, attr[1][dev])) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_quad_kernel<P, 1>), dim3(BH * nqb), dim3(256), Q2Geom::lds, stream, phiq, phik, v, g,
                     stats, JacIn{k, rho, omega, nph, H, kr}, dk, dom_k, dv, Tn, BH, nqb);
  return hipGetLastError();
}

}  // namespace

// dq, dk (through the feature map's Jacobian), dv (bf16 [BH][T][d]) and the omega partials (fp32, one row of d per
// (side, sequence, 32-token tile): dom_q and dom_k each [BH][ceil(T / 32)][d]) from the featurized operands and
// the statistics (1 / Dn_t, delta_t) of the forward pass, p = 2.  rho is the position phase table [T][d].
hipError_t launch_bwd_quadratic_bf16(const void* phiq, const void* phik, const void* v, const void* g,
                                     const float2* stats, int B, int H, int T, const void* q, const void* k,
                                     const float* rho, const float* omega, int nph, float kr, void* dq, void* dk,
                                     void* dv, float* dom_q, float* dom_k, hipStream_t stream) {
  return launch_t<2>(static_cast<const __bf16*>(phiq), static_cast<const __bf16*>(phik),
                     static_cast<const __bf16*>(v), static_cast<const __bf16*>(g), stats, B, H, T,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), rho, omega, nph, kr,
                     static_cast<__bf16*>(dq), static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), dom_q, dom_k,
                     stream);
}

}  // namespace sanatan
