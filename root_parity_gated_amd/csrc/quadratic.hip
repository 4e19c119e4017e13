// quadratic.hip -- normalised causal power attention in masked quadratic form (p = 1 or 2).
//
// SANATAN reading notes §2.6: w_ts = (kappa_ts / c)^p for s <= t, o_t = sum w v_s / (sum w + eps);
// kappa_ts = <Phi(q_t), Phi(k_s)> (§2.3).  p = 2 has no small-state recurrence (§2.6, §4.1), so
// this is the training/parallel form.  For the six-channel kernel 0 <= kappa <= 4d = c, so every
// weight lies in [0, 1] and no running maximum is needed (unlike softmax): partial sums over key
// blocks just add.  The unclipped four-channel instantiation (C0 = 3) has kappa4 in [-d, 3d]: its
// p = 1 weights and denominators can be negative or near zero, and its p = 2 weights give
// strongly mismatched pairs large positive weight; partial sums still just add (no maximum is
// needed for bounded weights), but the p = 2 result is not the clipped four-channel attention.
//
// Phi(K) is featurized once into the workspace (element type of the call), after the position
// phase table.  A workgroup is 4 waves and two workgroups share a CU (two waves per SIMD hide each
// other's latencies); each wave owns MQ tiles of 32 query rows and featurizes them once into
// 32x32x16 MFMA operand registers (K-step j = 16 features).  Per block of 32 keys, Phi(K)
// (channels 1..5: channel 0 is the constant 1 and contributes exactly d = 64 to every score) and
// V are staged token-major in LDS, two slots each, K one block ahead of V, and every wave forms its
// transposed score tiles A^T[s][t].  The masked, powered tile is the B operand of V^T P (V^T read
// with the transposing LDS load), and its row sums (v_dot2) accumulate the denominator.  A wave
// issues the score MFMAs of block kb + 1 with the weight VALU and V^T P MFMAs of block kb between
// them (software pipelining across key blocks).
#include <atomic>

#include "prefill_common.h"

namespace sanatan {
namespace {

// C0: the first staged feature channel.  1 for the six-channel kernel (channels 1..5), 3 for the unclipped
// four-channel kernel of the notes' §2.5, whose features per dim are [1, r, r cos, r sin] (channels 0, 3, 4, 5
// of the six-channel layout): the score then sums 1 + r_q r_k (1 + cos dtheta) per dim.
template <typename T, int C0 = 1>
struct QGeom {
  static constexpr int MQ = 1;                        // 32-row query tiles per wave
  static constexpr int QROWS = 4 * 32 * MQ;          // query rows per workgroup
  static constexpr int KB = 32;                       // keys per block
  static constexpr int NF = kF - C0 * kD;             // staged features: channels C0..5
  static constexpr int NJ = NF / 16;                  // K-steps of the score product
  static constexpr int KP = NF + 16 / (int)sizeof(T); // Phi(K) tile pitch (elements)
  // V tile pitch: bf16 rows of 160 bytes (40 banks apart, 8 mod 32), so the four token rows that 16 lanes
  // of a transposing read cover (eight banks each) fall on disjoint banks; fp32 rows 4 words apart
  static constexpr int VP = kDV + (sizeof(T) == 2 ? 16 : 4);
  static constexpr int k_bytes = KB * KP * (int)sizeof(T);
  static constexpr int v_bytes = KB * VP * (int)sizeof(T);
  static constexpr int buf_bytes = k_bytes + v_bytes;
  static constexpr int lds = 2 * buf_bytes;
  static constexpr int EL = 16 / (int)sizeof(T);     // elements per 16-byte piece
  static constexpr int KPIECES = KB * NF / EL;        // 16-byte pieces of one Phi(K) block
  static constexpr int VPIECES = KB * kDV / EL;
  static constexpr int PIECES = (KPIECES + VPIECES + 255) / 256;  // per thread
};

// Two workgroups per CU for bf16; the fp32 operand fragments take the registers of one.
// STATS (the backward pass's forward statistics): instead of o, write per query row the denominator
// 1 / Dn (Dn = sum_s kappa^p + eps c^p) and delta = <g_t, o_t> with g = dout, as float2 stats[bh][t].
template <typename T, int P, int C0, bool STATS = false>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void quadratic_kernel(
    const T* __restrict__ q, const T* __restrict__ phik, const T* __restrict__ v, T* __restrict__ out,
    const float* __restrict__ rho, const float* __restrict__ omega, int nph, int H, int Tn, int BH, int nqb, float kr,
    float eps_cp, const T* __restrict__ gout = nullptr, float2* __restrict__ stats = nullptr,
    float* __restrict__ inv_out = nullptr) {
  using G = QGeom<T, C0>;
  typedef typename FragT<T>::type Frag;
  constexpr int MQ = G::MQ, KB = G::KB, NF = G::NF, NJ = G::NJ, KP = G::KP, VP = G::VP, EL = G::EL;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, h = l >> 5, n32 = l & 31;
  // heaviest (latest) query blocks first across all sequences
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int hd = bh % H;
  const int row0 = qb * G::QROWS + w * 32 * MQ;  // this wave's first query row
  const T* qp = q + (size_t)bh * Tn * kD;
  const T* kp = phik + (size_t)bh * Tn * kF + C0 * kD;  // skip the channels below C0
  const T* vp = v + (size_t)bh * Tn * kDV;
  T* op = out + (size_t)bh * Tn * kDV;

  // ---- key blocks: staged Phi(K) (channels 1..5) and V, double-buffered.  A block is KB rows of NF
  // features and KB rows of d_v values: exactly KPT + VPT 16-byte pieces per thread, whose offsets do
  // not depend on the block.
  constexpr int KPT = G::KPIECES / 256, VPT = G::VPIECES / 256;
  static_assert(KPT * 256 == G::KPIECES && VPT * 256 == G::VPIECES, "pieces must divide evenly");
  const int last_row = min(Tn - 1, qb * G::QROWS + G::QROWS - 1);
  const int nkb = last_row / KB + 1;
  const int my_last = min(Tn - 1, row0 + 32 * MQ - 1);
  // this wave's last key block: the only one that can reach past one of its queries
  const int lastb = my_last / KB;
  u32x4 pk[KPT], pv[VPT];
  auto krow_of = [&](int p) { return (tid + 256 * p) / (NF / EL); };
  auto kcol_of = [&](int p) { return ((tid + 256 * p) % (NF / EL)) * EL; };
  auto vrow_of = [&](int p) { return (tid + 256 * p) / (kDV / EL); };
  auto vcol_of = [&](int p) { return ((tid + 256 * p) % (kDV / EL)) * EL; };
  // This thread's pieces of key block kb -> registers, through buffer loads: the block's descriptor starts
  // at its first row and covers the rows up to the sequence's end, so the hardware's range check returns
  // zeros for rows past the end, and each piece's offset from the descriptor's start is fixed per thread
  // (no address arithmetic per block).  Descriptor word 3: the gfx9-family raw-buffer format.  Callers
  // fetch only blocks kb < nkb, whose first row lies inside the sequence.
  unsigned koff[KPT], voff[VPT];
#pragma unroll
  for (int p = 0; p < KPT; p++) koff[p] = (unsigned)((krow_of(p) * kF + kcol_of(p)) * (int)sizeof(T));
#pragma unroll
  for (int p = 0; p < VPT; p++) voff[p] = (unsigned)((vrow_of(p) * kDV + vcol_of(p)) * (int)sizeof(T));
  constexpr int kRawBufferWord3 = 0x00020000;
  auto fetch_k = [&](int kb, u32x4 (&dst)[KPT]) {
    const int s0 = kb * KB;
    // Phi(K) rows start at channel C0 (kp skips the channels below), so the last row ends C0 kD elements
    // short of kF
    const __amdgpu_buffer_rsrc_t kr_ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kp + (size_t)s0 * kF), (short)0, (int)(((long long)(Tn - s0) * kF - C0 * kD) * (long long)sizeof(T)),
        kRawBufferWord3);
#pragma unroll
    for (int p = 0; p < KPT; p++) dst[p] = __builtin_amdgcn_raw_buffer_load_b128(kr_, koff[p], 0, 0);
  };
  auto fetch_v = [&](int kb) {
    const int s0 = kb * KB;
    const __amdgpu_buffer_rsrc_t vr_ = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vp + (size_t)s0 * kDV), (short)0, (int)((long long)(Tn - s0) * kDV * (long long)sizeof(T)),
        kRawBufferWord3);
#pragma unroll
    for (int p = 0; p < VPT; p++) pv[p] = __builtin_amdgcn_raw_buffer_load_b128(vr_, voff[p], 0, 0);
  };
  // LDS: two Phi(K) slots, then two V slots.  Key block kb lives in K slot kb % 2 and V slot kb % 2.
  auto kslot = [&](int s) { return reinterpret_cast<T*>(smem + s * G::k_bytes); };
  auto vslot = [&](int s) { return reinterpret_cast<T*>(smem + 2 * G::k_bytes + s * G::v_bytes); };
  auto stash_k = [&](int s, const u32x4 (&src)[KPT]) {
    T* Ks = kslot(s);
#pragma unroll
    for (int p = 0; p < KPT; p++)
      *reinterpret_cast<u32x4*>(__builtin_assume_aligned(Ks + krow_of(p) * KP + kcol_of(p), 16)) = src[p];
  };
  auto stash_v = [&](int s) {
    T* Vs = vslot(s);
#pragma unroll
    for (int p = 0; p < VPT; p++)
      *reinterpret_cast<u32x4*>(__builtin_assume_aligned(Vs + vrow_of(p) * VP + vcol_of(p), 16)) = pv[p];
  };

  f32x16 num[MQ][2];
  float rs[MQ];
#pragma unroll
  for (int mq = 0; mq < MQ; mq++) {
    zero16(num[mq][0]);
    zero16(num[mq][1]);
    rs[mq] = 0.0f;
  }
  // in flight while the queries are featurized
  u32x4 pk1[KPT];
  fetch_k(0, pk);
  fetch_v(0);
  if (nkb > 1) fetch_k(1, pk1);
  // ---- Phi(q) operands: K-step j = channel C0 + j/4, dims 16 (j%4) + 8h + i (slot i)
  Frag QF[MQ][NJ];
#pragma unroll
  for (int mq = 0; mq < MQ; mq++) {
    const int t = min(row0 + 32 * mq + n32, Tn - 1);
#pragma unroll
    for (int m = 0; m < 4; m++) {
      float cr[8], sr[8], rr[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int a = 16 * m + 8 * h + i;
        const float om4 = anchor_rev(omega[(size_t)(hd % nph) * kD + a]);
        featurize1(to_f32(qp[(size_t)t * kD + a]), rho[(size_t)t * kD + a], om4, kr, cr[i], sr[i], rr[i]);
      }
      float ch[5][8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        ch[0][i] = cr[i];
        ch[1][i] = sr[i];
        ch[2][i] = rr[i];
        ch[3][i] = rr[i] * cr[i];
        ch[4][i] = rr[i] * sr[i];
      }
#pragma unroll
      for (int c = 0; c < 6 - C0; c++) QF[mq][4 * c + m] = pack8f<T>(ch[C0 - 1 + c]);
    }
  }

  stash_k(0, pk);
  stash_v(0);
  if (nkb > 1) stash_k(1, pk1);
  if (nkb > 2) fetch_k(2, pk);
  if (nkb > 1) fetch_v(1);
  __syncthreads();

  // Score tiles of two consecutive key blocks, indexed by block parity: A^T[s][t] (rows = keys, cols =
  // queries) in MFMA accumulator layout, lane (query n32, half h) holding keys 8(i/4) + 4h + i%4.
  f32x16 at[2][MQ];
  // Channel 0 (the constant 1 in both feature maps) adds exactly d to every score: the first MFMA of each
  // tile starts from this splat instead of from zero.  (The empty asm keeps it in registers, so it is not
  // rebuilt for every tile.)
  f32x16 c0;
#pragma unroll
  for (int i = 0; i < 16; i++) c0[i] = (float)kD;
  asm volatile("" : "+v"(c0));
  // weights of one score tile (kappa^p; the 1 / c^p of the pages' weights cancels against the scaled
  // epsilon of the normalisation)
  auto power = [&](float a) { return P == 2 ? a * a : a; };
  // the weights of block kb (score tile sc, V slot vs) times V, masked where the block reaches past a query
  auto weigh = [&](const f32x16 (&sc)[MQ], const T* Vs, int kb) {
    const int s0 = kb * KB;
    const bool diag = s0 + KB - 1 > row0;
#pragma unroll
    for (int mq = 0; mq < MQ; mq++) {
      const int tq = row0 + 32 * mq + n32;  // this lane's query
      float wv[16];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        // (an empty asm keeps the compiler from hoisting these powers above the branch that leads
        // here, where the other path forms them again between its MFMAs)
        float a = sc[mq][i];
        asm volatile("" : "+v"(a));
        wv[i] = power(a);
      }
      if (diag) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int s = s0 + 8 * (i >> 2) + 4 * h + (i & 3);
          wv[i] = (s > tq) ? 0.0f : wv[i];
        }
      }
      float lo[8], hi8[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        lo[i] = wv[i];
        hi8[i] = wv[8 + i];
      }
      const Frag P0 = pack8f<T>(lo), P1 = pack8f<T>(hi8);
      rs[mq] = frag_sum(P1, frag_sum(P0, rs[mq]));
#pragma unroll
      for (int vt = 0; vt < 2; vt++) {
        mma32(num[mq][vt], lds_tokfrag(Vs, VP, 0, 32 * vt, l), P0);
        mma32(num[mq][vt], lds_tokfrag(Vs, VP, 16, 32 * vt, l), P1);
      }
    }
  };
  // Score tiles of key block kb (K slot kb % 2) into at[kb % 2].  With `prev`, the weights of block kb - 1
  // (never a block that reaches past a query: only a wave's last block does) are formed in the same
  // instruction stream: powered, packed and summed between the score MFMAs, then multiplied with their V
  // (V slot (kb - 1) % 2), so the matrix cores have independent work while that VALU runs.
  auto scores = [&](auto Par, auto Prev) {
    constexpr int par = decltype(Par)::value;
    constexpr bool prev = decltype(Prev)::value;
    const T* Ks = kslot(par);
    const T* Vs = vslot(par ^ 1);
    f32x16(&cur)[MQ] = at[par];
    const f32x16(&old)[MQ] = at[par ^ 1];
    const T* krow = Ks + n32 * KP + 8 * h;
    auto ldA = [&](int j) {
      Frag A;
      if constexpr (sizeof(T) == 2) {
        A = *reinterpret_cast<const Frag*>(krow + 16 * j);
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) A[i] = krow[16 * j + i];
      }
      return A;
    };
    // Phi(K) fragments are read PD K-steps ahead of their MFMA, so LDS latency stays hidden
    constexpr int PD = 4;
    // the previous block's work, spread over the K-steps: powers over the first PW steps, then packing (2),
    // the V fragments (1), the row sums (1) and the four V^T P MFMAs
    constexpr int PW = NJ >= 16 ? 8 : 4;
    static_assert(NJ >= PW + 8, "not enough K-steps to spread the previous block's work over");
    Frag Ar[PD];
#pragma unroll
    for (int j = 0; j < PD; j++) Ar[j] = ldA(j);
    float wv[MQ][16];
    Frag P0[MQ], P1[MQ], Vf[2][2];
    __builtin_amdgcn_sched_barrier(0);  // (fences keep the compiler from shortening the distances)
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const Frag A = Ar[j % PD];
#pragma unroll
      for (int mq = 0; mq < MQ; mq++) {
        if (j == 0)
          mma32c(cur[mq], A, QF[mq][0], c0);
        else
          mma32(cur[mq], A, QF[mq][j]);
      }
      if (j + PD < NJ) Ar[j % PD] = ldA(j + PD);
      if constexpr (prev) {
        if (j < PW) {
          constexpr int E = 16 / PW;
#pragma unroll
          for (int mq = 0; mq < MQ; mq++)
#pragma unroll
            for (int e = 0; e < E; e++) wv[mq][E * j + e] = power(old[mq][E * j + e]);
        } else if (j == PW || j == PW + 1) {
#pragma unroll
          for (int mq = 0; mq < MQ; mq++) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; i++) x[i] = wv[mq][8 * (j - PW) + i];
            (j == PW ? P0[mq] : P1[mq]) = pack8f<T>(x);
          }
        } else if (j == PW + 2) {
#pragma unroll
          for (int vt = 0; vt < 2; vt++) {
            Vf[vt][0] = lds_tokfrag(Vs, VP, 0, 32 * vt, l);
            Vf[vt][1] = lds_tokfrag(Vs, VP, 16, 32 * vt, l);
          }
        } else if (j == PW + 3) {
#pragma unroll
          for (int mq = 0; mq < MQ; mq++) rs[mq] = frag_sum(P1[mq], frag_sum(P0[mq], rs[mq]));
        } else if (j >= PW + 4 && j < PW + 8) {
          const int vt = (j - PW - 4) >> 1, hf = (j - PW - 4) & 1;
#pragma unroll
          for (int mq = 0; mq < MQ; mq++) mma32(num[mq][vt], Vf[vt][hf], hf ? P1[mq] : P0[mq]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One step per key block kb: the scores of block kb + 1 together with the weights of block kb, or, on
  // the wave's last block, its masked weights alone; then the staging of K(kb + 2) and V(kb + 1), whose
  // slots were last read before the previous barrier.  The loop below alternates the parities
  // explicitly, so each copy of this body names its slots and tiles at compile time.
  auto step = [&](auto Par, int kb) {
    constexpr int par = decltype(Par)::value;
    if (kb < lastb) scores(std::integral_constant<int, par ^ 1>(), std::true_type());
    if (kb == lastb) weigh(at[par], vslot(par), kb);
    if (kb + 2 < nkb) stash_k(par, pk);
    if (kb + 1 < nkb) stash_v(par ^ 1);
    if (kb + 3 < nkb) fetch_k(kb + 3, pk);
    if (kb + 2 < nkb) fetch_v(kb + 2);
    __syncthreads();
  };
  scores(std::integral_constant<int, 0>(), std::false_type());  // every wave has key block 0
  __syncthreads();  // K slot 0 is restaged in the first step
  for (int kb = 0; kb < nkb; kb += 2) {
    step(std::integral_constant<int, 0>(), kb);
    if (kb + 1 >= nkb) break;
    step(std::integral_constant<int, 1>(), kb + 1);
  }

  // ---- o = num / (den + eps): lane (query n32, half h) holds value rows 32 vt + 8 j + 4 h + i4
#pragma unroll
  for (int mq = 0; mq < MQ; mq++) {
    const int t = row0 + 32 * mq + n32;
    const float den = xor32_sum(rs[mq]);
    if constexpr (STATS) {
      const int tc = min(t, Tn - 1);
      const T* gp = gout + ((size_t)bh * Tn + tc) * kDV;
      float dot = 0.0f;
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int i4 = 0; i4 < 4; i4++) dot = fmaf(to_f32(gp[32 * vt + 8 * j + 4 * h + i4]), num[mq][vt][4 * j + i4], dot);
      dot = xor32_sum(dot);
      const float dn = den + eps_cp;
      if (t < Tn && h == 0) stats[(size_t)bh * Tn + t] = make_float2(1.0f / dn, dot / dn);
      continue;
    }
    if (t < Tn) {
      // weights are kappa^p here, so epsilon is scaled by c^p: o = sum w v / (sum w + eps c^p)
      const float inv = 1.0f / (den + eps_cp);
      // saved for the backward pass: the fp32 output row ([BH][T][d_v]) then 1 / Dn ([BH][T])
      float* sv = inv_out ? inv_out + ((size_t)bh * Tn + t) * kDV : nullptr;
      if (inv_out && h == 0) inv_out[(size_t)BH * Tn * kDV + (size_t)bh * Tn + t] = inv;
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
#pragma unroll
          for (int i4 = 0; i4 < 4; i4++)
            op[(size_t)t * kDV + 32 * vt + 8 * j + 4 * h + i4] = from_f32<T>(num[mq][vt][4 * j + i4] * inv);
          if (sv)
            *reinterpret_cast<float4*>(sv + 32 * vt + 8 * j + 4 * h) =
                make_float4(num[mq][vt][4 * j] * inv, num[mq][vt][4 * j + 1] * inv, num[mq][vt][4 * j + 2] * inv,
                            num[mq][vt][4 * j + 3] * inv);
        }
    }
  }
}

size_t rho_bytes_q(int T) { return (((size_t)T * kD * sizeof(float)) + 255) & ~(size_t)255; }

template <typename T, int P, int C0>
hipError_t launch_quad_t(const void* q, const void* k, const void* v, int B, int H, int Tn, int64_t pos0,
                         const MethodConsts& mc, void* out, void* ws, sanatan_dtype t, float* inv_out,
                         hipStream_t stream) {
  float* rho = static_cast<float*>(ws);
  void* phik = static_cast<char*>(ws) + rho_bytes_q(Tn);
  hipError_t e = launch_phase_table(rho, Tn, pos0, mc.log2_base, stream);
  if (e != hipSuccess) return e;
  e = launch_featurize(k, t, B, H, Tn, pos0, mc, phik, t, stream);
  if (e != hipSuccess) return e;
  using G = QGeom<T, C0>;
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void*)quadratic_kernel<T, P, C0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            G::lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  const int nqb = (Tn + G::QROWS - 1) / G::QROWS;
  const int BH = B * H;
  hipLaunchKernelGGL((quadratic_kernel<T, P, C0>), dim3(BH * nqb), dim3(256), G::lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(phik), static_cast<const T*>(v),
                     static_cast<T*>(out), rho, mc.omega, mc.nph, H, Tn, BH, nqb, mc.kr,
                     P == 2 ? (float)((double)mc.ceps / (double)mc.inv_c) : mc.ceps, nullptr, nullptr, inv_out);
  return hipGetLastError();
}

template <typename T, int P>
hipError_t launch_quad_stats_t(const void* q, const void* phik, const void* v, const void* g, int B, int H, int Tn,
                               const float* rho, const MethodConsts& mc, float2* stats, hipStream_t stream) {
  using G = QGeom<T, 1>;
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute((const void*)quadratic_kernel<T, P, 1, true>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, G::lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  const int nqb = (Tn + G::QROWS - 1) / G::QROWS;
  const int BH = B * H;
  hipLaunchKernelGGL((quadratic_kernel<T, P, 1, true>), dim3(BH * nqb), dim3(256), G::lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(phik), static_cast<const T*>(v), nullptr, rho,
                     mc.omega, mc.nph, H, Tn, BH, nqb, mc.kr,
                     P == 2 ? (float)((double)mc.ceps / (double)mc.inv_c) : mc.ceps, static_cast<const T*>(g), stats);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quadratic_stats(const void* q, const void* phik, const void* v, const void* g, sanatan_dtype t,
                                  int B, int H, int T, int p, const float* rho, const MethodConsts& mc, float2* stats,
                                  hipStream_t stream) {
  if (t == SANATAN_BF16)
    return p == 1 ? launch_quad_stats_t<__bf16, 1>(q, phik, v, g, B, H, T, rho, mc, stats, stream)
                  : launch_quad_stats_t<__bf16, 2>(q, phik, v, g, B, H, T, rho, mc, stats, stream);
  return p == 1 ? launch_quad_stats_t<float, 1>(q, phik, v, g, B, H, T, rho, mc, stats, stream)
                : launch_quad_stats_t<float, 2>(q, phik, v, g, B, H, T, rho, mc, stats, stream);
}

size_t quadratic_ws_bytes(int B, int H, int T, sanatan_dtype t) {
  const size_t el = (t == SANATAN_BF16) ? 2 : 4;
  return rho_bytes_q(T) + (size_t)B * H * T * kF * el;
}

template <int C0>
static hipError_t launch_quad_c(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                                int p, int64_t pos0, const MethodConsts& mc, void* out, void* ws, float* inv_out,
                                hipStream_t stream) {
  if (t == SANATAN_BF16)
    return p == 1 ? launch_quad_t<__bf16, 1, C0>(q, k, v, B, H, T, pos0, mc, out, ws, t, inv_out, stream)
                  : launch_quad_t<__bf16, 2, C0>(q, k, v, B, H, T, pos0, mc, out, ws, t, inv_out, stream);
  return p == 1 ? launch_quad_t<float, 1, C0>(q, k, v, B, H, T, pos0, mc, out, ws, t, inv_out, stream)
                : launch_quad_t<float, 2, C0>(q, k, v, B, H, T, pos0, mc, out, ws, t, inv_out, stream);
}

hipError_t launch_quadratic(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                            int p, bool four_channel, int64_t pos0, const MethodConsts& mc, void* out, void* ws,
                            hipStream_t stream, float* inv_out) {
  return four_channel ? launch_quad_c<3>(q, k, v, t, B, H, T, p, pos0, mc, out, ws, inv_out, stream)
                      : launch_quad_c<1>(q, k, v, t, B, H, T, p, pos0, mc, out, ws, inv_out, stream);
}

}  // namespace sanatan
