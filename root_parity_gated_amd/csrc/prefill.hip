// prefill.hip -- chunked causal p = 1 SANATAN attention on gfx950 MFMA: host plan, dispatch,
// the boundary scan, and the 4-wave kernel for fp32 inputs.  The bf16 kernels (one wave per feature
// group) are in prefill_grp.hip.
//
// Exact regrouping of the recurrence of the SANATAN reading notes §2.7 (sum over s <= t of
// kappa(t,s) v_s with kappa = <Phi(q_t), Phi(k_s)>, §2.3).  For a chunk with the state (S, z) of
// all earlier tokens:
//     num_t = sum_{s in chunk, s <= t} A_ts v_s + Phi(q_t)^T S,       A = Phi(Q) Phi(K)^T
//     den_t = sum_{s in chunk, s <= t} A_ts     + Phi(q_t)^T z,       o_t = num_t / (den_t + c eps)
// then S += Phi(K)^T V and z += Phi(K)^T 1.
//
// Work split (MI355X-first):
//   * G = #CUs workgroups (one resident per CU) split the flattened (sequence, chunk) list into
//     equal contiguous ranges.  A range's part of one sequence is a "piece": pass 1 computes each
//     non-final piece's state increment, the scan (fused into pass 3 when a sequence has few pieces)
//     gives each piece its exclusive prefix, pass 3 runs the chunks.  The update is purely
//     additive (no decay, as the notes stress), so pieces compose by addition.
//   * Features are split across waves by content dims (see prefill_common.h).  Lanes featurize
//     straight into the K-slots of the 32x32x16 MFMA; Phi never leaves the CU.  Phi(K) is kept
//     token-major in LDS for the intra product and read through the gfx950 transposing LDS load
//     (ds_read_b64_tr_b16) as the token-consecutive operand of the state update; V likewise.
//   * Accumulator tiles are directly the next product's operands: A^T tiles (rows s, cols t) are the
//     B operand of num^T = V^T A^T, and S tiles (rows f, cols v) the A operand of the readout
//     num^T += S^T Phi(Q)^T.  The state slice stays in accumulators for a whole piece; z lives in LDS.
//     The denominator is computed on VALU (row sums of the masked A^T tiles with v_dot2, and
//     Phi(q) . z), far cheaper than a 32-column MFMA tile for one column.
//   * Partial (num, den) over feature groups are added through LDS in a fixed order (bitwise
//     deterministic) before the division.
#include <atomic>

#include "prefill_common.h"

namespace sanatan {

template <typename T, int CH>
struct Geom4 {
  static constexpr int TB = (CH + 31) / 32;   // 32-token blocks per chunk
  static constexpr int CT = 32 * TB;          // tile tokens
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VP = 64 + 16 / ES;     // Vs pitch (elements): +16 B keeps alignment, skews banks
  static constexpr int KP = 96 + 16 / ES;     // KS pitch
  static constexpr int RP = 68;               // red pitch (floats): 64 values, den at 64
  static constexpr size_t vs_bytes = (size_t)CT * VP * ES;
  static constexpr size_t ks_bytes = (size_t)4 * CT * KP * ES;
  static constexpr size_t red_bytes = (size_t)4 * 32 * RP * 4;
  static constexpr size_t z_bytes = 4 * 96 * 4;
  static constexpr size_t stage_bytes = (size_t)(kF * kDV + kF) * 4;
  static constexpr size_t body(bool state_only) { return vs_bytes + ks_bytes + (state_only ? 0 : red_bytes); }
  static constexpr size_t lds(bool state_only) {
    return (body(state_only) > stage_bytes ? body(state_only) : stage_bytes) + z_bytes;
  }
};

template <typename T, int CH, bool STATE_ONLY, bool RAGGED>
__global__ __launch_bounds__(256, 1) void prefill4_kernel(const PrefillArgs args) {
  using G = Geom4<T, CH>;
  using Frag = typename FragT<T>::type;
  constexpr int TB = G::TB, CT = G::CT, VP = G::VP, KP = G::KP, RP = G::RP;
  constexpr size_t LDS = G::lds(STATE_ONLY);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* Vs = reinterpret_cast<T*>(smem);                                       // [CT][VP] V
  T* KS = reinterpret_cast<T*>(smem + G::vs_bytes);                         // [4][CT][KP] Phi(K)
  float* red = reinterpret_cast<float*>(smem + G::vs_bytes + G::ks_bytes);  // [4][32][RP]
  float* stage = reinterpret_cast<float*>(smem);                            // state staging (aliases)
  float* Zb = reinterpret_cast<float*>(smem + LDS - G::z_bytes);            // [4][96] z

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n32 = l & 31;
  const int g = range_of_block(args);
  const int Tn = args.T;
  T* KSw = KS + w * CT * KP;
  float* Zw = Zb + w * 96;
  const int dbase = 16 * w + 4 * h;  // this lane's dims: dbase + {0..3, 8..11}

  const long long total = call_chunks<RAGGED>(args);
  const long long hi = range_lo(g + 1, total, args.G);
  for (long long c = range_lo(g, total, args.G); c < hi;) {
    const SeqSpan sp = seq_span<RAGGED>(c, args);
    if (RAGGED && sp.bh < 0) break;
    const int bh = sp.bh;
    const long long seq_c0 = sp.c0;
    const long long seq_end = sp.c1;
    const long long pend = hi < seq_end ? hi : seq_end;
    const bool last_piece = (pend == seq_end);
    const int t_begin = (int)(c - seq_c0) * CH;
    const int t_end = min(sp.len, (int)(pend - seq_c0) * CH);
    c = pend;
    if (STATE_ONLY && last_piece) continue;
    const int hh = bh % args.H;
    const T* __restrict__ qp = static_cast<const T*>(args.q) + (size_t)bh * Tn * kD;
    const T* __restrict__ kp = static_cast<const T*>(args.k) + (size_t)bh * Tn * kD;
    const T* __restrict__ vp = static_cast<const T*>(args.v) + (size_t)bh * Tn * kDV;
    T* __restrict__ op = static_cast<T*>(args.out) + (size_t)bh * Tn * kDV;
    float* slot = args.ws_state + (size_t)(bh + g) * kStateFloats;

    float om4[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      om4[i] = anchor_rev(args.omega[(size_t)(hh % args.nph) * kD + dbase + (i & 3) + 8 * (i >> 2)]);

    // ---- initial state of the piece
    f32x16 Sacc[2][3];
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int ft = 0; ft < 3; ft++) zero16(Sacc[vt][ft]);
    for (int m = l; m < 96; m += 64) Zw[m] = 0.0f;
    if (!STATE_ONLY) {
      auto add_slot = [&](const float* s, const float* zz) {
        __syncthreads();
        stage_in<256>(stage, s, zz);
        __syncthreads();
        stage_add_tile(Sacc[0], stage, w, 0, l);
        stage_add_tile(Sacc[1], stage, w, 1, l);
        for (int m = l; m < 96; m += 64) Zw[m] += stage[kStageS + w * 96 + m];
      };
      if (args.multi && args.scanned) {
        // (a ragged call's scan leaves the head piece's slot unwritten when there is no caller state)
        if (!RAGGED || args.S || g != range_of_chunk(seq_c0, total, args.G)) add_slot(slot, slot + kF * kDV);
      } else {
        if (args.S) add_slot(args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF);
        if (!RAGGED && args.multi) {  // few pieces per sequence: add the earlier pieces' increments here
          // (a uniform plan has no empty ranges: every slot gf..g-1 was written by pass 1)
          const int gf = range_of_chunk(seq_c0, total, args.G);
          for (int gg = gf; gg < g; gg++) {
            const float* sj = args.ws_state + (size_t)(bh + gg) * kStateFloats;
            add_slot(sj, sj + kF * kDV);
          }
        }
      }
      __syncthreads();  // the staging area is reused by the tiles
    }

    // Raw K, Q and V rows of a chunk are loaded into registers one chunk ahead of their use (each set is
    // refilled as soon as it is consumed), so the global-load latency is not exposed at the chunk start.
    constexpr int EPL = 16 / G::ES, PER_TOK = kDV / EPL;
    constexpr int NVP = (CT * PER_TOK + 255) / 256;  // 16-byte pieces of V per thread
    Raw8<T> rk[TB], rq[TB];
    uint4 rv[NVP];
    auto fetch_kv = [&](int tc0) {
      const int nv = min(CH, t_end - tc0);
#pragma unroll
      for (int j = 0; j < NVP; j++) {
        const int idx = tid + 256 * j, s = idx / PER_TOK, col = (idx % PER_TOK) * EPL;
        if (idx < CT * PER_TOK) rv[j] = *reinterpret_cast<const uint4*>(vp + (size_t)(tc0 + min(s, nv - 1)) * kDV + col);
      }
#pragma unroll
      for (int sb = 0; sb < TB; sb++) load_raw8(kp + (size_t)(tc0 + min(32 * sb + n32, nv - 1)) * kD + dbase, rk[sb]);
    };
    auto fetch_q = [&](int tc0, int tb) {
      const int nv = min(CH, t_end - tc0);
      load_raw8(qp + (size_t)(tc0 + min(32 * tb + n32, nv - 1)) * kD + dbase, rq[tb]);
    };
    fetch_kv(t_begin);
    if (!STATE_ONLY) {
#pragma unroll
      for (int tb = 0; tb < TB; tb++) fetch_q(t_begin, tb);
    }

    for (int t0 = t_begin; t0 < t_end; t0 += CH) {
      const int nvalid = min(CH, t_end - t0);
      const int tn = t0 + CH < t_end ? t0 + CH : t0;  // the next chunk (or this one again at the end)

      // (a) V tile -> LDS (token-major), zero beyond nvalid (loads clamped in bounds).
#pragma unroll
      for (int j = 0; j < NVP; j++) {
        const int idx = tid + 256 * j, s = idx / PER_TOK, col = (idx % PER_TOK) * EPL;
        if (idx < CT * PER_TOK)
          *reinterpret_cast<uint4*>(Vs + s * VP + col) = s < nvalid ? rv[j] : make_uint4(0u, 0u, 0u, 0u);
      }
      // (b) Phi(K) of the chunk -> this wave's token-major LDS tile (zero rows beyond nvalid)
      float ku[TB][8];
#pragma unroll
      for (int sb = 0; sb < TB; sb++) unpack8(rk[sb], ku[sb]);
      fetch_kv(tn);
#pragma unroll
      for (int sb = 0; sb < TB; sb++) {
        const int sl = 32 * sb + n32;
        const int sc = t0 + min(sl, nvalid - 1);
        float rh[8];
        const float (&u)[8] = ku[sb];
        load8(args.rho + (size_t)sc * kD + dbase, rh);
        float ch[6][8];
        featurize8(u, rh, om4, args.kr, ch);
        const float keep = sl < nvalid ? 1.0f : 0.0f;
#pragma unroll
        for (int cc = 0; cc < 6; cc++) {
          T* p = KSw + sl * KP + 16 * cc + 4 * h;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            p[i] = (T)(ch[cc][i] * keep);
            p[8 + i] = (T)(ch[cc][4 + i] * keep);
          }
        }
      }
      __syncthreads();

      if (!STATE_ONLY) {
        // readout operands S^T (rows v, K = features) from the state before this chunk
        Frag SA[2][6];
#pragma unroll
        for (int vt = 0; vt < 2; vt++)
#pragma unroll
          for (int cc = 0; cc < 6; cc++) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; i++) x[i] = Sacc[vt][cc >> 1][8 * (cc & 1) + i];
            SA[vt][cc] = pack8f<T>(x);
          }
#pragma unroll
        for (int tb = 0; tb < TB; tb++) {
          // Phi(Q) of query block tb, and the readout part of the denominator, Phi(q) . z
          const int tl = 32 * tb + n32;
          const int tc = t0 + min(tl, nvalid - 1);
          float u[8], rh[8];
          unpack8(rq[tb], u);
          fetch_q(tn, tb);
          load8(args.rho + (size_t)tc * kD + dbase, rh);
          float ch[6][8];
          featurize8(u, rh, om4, args.kr, ch);
          Frag QF[6];
          float den = 0.0f;
#pragma unroll
          for (int cc = 0; cc < 6; cc++) {
            QF[cc] = pack8f<T>(ch[cc]);
            const float4 za = *reinterpret_cast<const float4*>(Zw + 16 * cc + 4 * h);
            const float4 zb = *reinterpret_cast<const float4*>(Zw + 16 * cc + 8 + 4 * h);
            den = fmaf(ch[cc][0], za.x, den);
            den = fmaf(ch[cc][1], za.y, den);
            den = fmaf(ch[cc][2], za.z, den);
            den = fmaf(ch[cc][3], za.w, den);
            den = fmaf(ch[cc][4], zb.x, den);
            den = fmaf(ch[cc][5], zb.y, den);
            den = fmaf(ch[cc][6], zb.z, den);
            den = fmaf(ch[cc][7], zb.w, den);
          }
          f32x16 numT[2];
          zero16(numT[0]);
          zero16(numT[1]);
          // intra-chunk: A^T tiles (rows s, cols t) over this wave's 96 features, masked s <= t,
          // straight into num^T = V^T A^T as the B operand
#pragma unroll
          for (int sb = 0; sb <= tb; sb++) {
            f32x16 at;
            zero16(at);
#pragma unroll
            for (int cc = 0; cc < 6; cc++) mma32(at, lds_rowfrag<T>(KSw, KP, 32 * sb + n32, cc, h), QF[cc]);
            float lo[8], hi2[8];
#pragma unroll
            for (int i = 0; i < 16; i++) {
              const int sl = 8 * (i >> 2) + 4 * h + (i & 3);
              const float a = (sb == tb && sl > n32) ? 0.0f : at[i];
              if (i < 8) lo[i] = a;
              else hi2[i - 8] = a;
            }
            const Frag P0 = pack8f<T>(lo), P1 = pack8f<T>(hi2);
            den = frag_sum(P1, frag_sum(P0, den));  // row sum of the values the A.V product sees
#pragma unroll
            for (int vt = 0; vt < 2; vt++) {
              mma32(numT[vt], lds_tokfrag(Vs, VP, 32 * sb, 32 * vt, l), P0);
              mma32(numT[vt], lds_tokfrag(Vs, VP, 32 * sb + 16, 32 * vt, l), P1);
            }
          }
          // inter-chunk readout: num^T += S^T Phi(Q)^T
#pragma unroll
          for (int cc = 0; cc < 6; cc++)
#pragma unroll
            for (int vt = 0; vt < 2; vt++) mma32(numT[vt], SA[vt][cc], QF[cc]);
          den += __shfl_xor(den, 32);
          // this wave's partial (num, den) -> LDS: row t, 64 value columns, den at column 64
          float* rw = red + w * 32 * RP + n32 * RP;
#pragma unroll
          for (int vt = 0; vt < 2; vt++)
#pragma unroll
            for (int j = 0; j < 4; j++)
              *reinterpret_cast<float4*>(rw + 32 * vt + 8 * j + 4 * h) =
                  make_float4(numT[vt][4 * j], numT[vt][4 * j + 1], numT[vt][4 * j + 2], numT[vt][4 * j + 3]);
          if (h == 0) rw[64] = den;
          __syncthreads();
          {
            const int row = tid >> 3, v0 = 8 * (tid & 7);
            const int t_out = 32 * tb + row;
            if (t_out < nvalid) {
              constexpr int WS = 32 * RP;
              const float dsum = ((red[row * RP + 64] + red[WS + row * RP + 64]) + red[2 * WS + row * RP + 64]) +
                                 red[3 * WS + row * RP + 64];
              const float inv = 1.0f / (dsum + args.ceps);
              T o[8];
#pragma unroll
              for (int hv = 0; hv < 2; hv++) {
                const float4 a0 = *reinterpret_cast<const float4*>(red + row * RP + v0 + 4 * hv);
                const float4 a1 = *reinterpret_cast<const float4*>(red + WS + row * RP + v0 + 4 * hv);
                const float4 a2 = *reinterpret_cast<const float4*>(red + 2 * WS + row * RP + v0 + 4 * hv);
                const float4 a3 = *reinterpret_cast<const float4*>(red + 3 * WS + row * RP + v0 + 4 * hv);
                o[4 * hv + 0] = from_f32<T>((((a0.x + a1.x) + a2.x) + a3.x) * inv);
                o[4 * hv + 1] = from_f32<T>((((a0.y + a1.y) + a2.y) + a3.y) * inv);
                o[4 * hv + 2] = from_f32<T>((((a0.z + a1.z) + a2.z) + a3.z) * inv);
                o[4 * hv + 3] = from_f32<T>((((a0.w + a1.w) + a2.w) + a3.w) * inv);
              }
              uint4* dst = reinterpret_cast<uint4*>(op + (size_t)(t0 + t_out) * kDV + v0);
              const uint4* src = reinterpret_cast<const uint4*>(o);
#pragma unroll
              for (int i = 0; i < (int)sizeof(o) / 16; i++) dst[i] = src[i];
            }
          }
          __syncthreads();
        }
      }

      // (c) state update S += Phi(K)^T V (this wave's 96 feature rows) and z += Phi(K)^T 1
      float zadd[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int ft = 0; ft < 3; ft++) {
#pragma unroll
        for (int ks = 0; ks < 2 * TB; ks++) {
          const Frag A = lds_tokfrag(KSw, KP, 16 * ks, 32 * ft, l);
          zadd[ft] = frag_sum(A, zadd[ft]);
#pragma unroll
          for (int vt = 0; vt < 2; vt++) mma32(Sacc[vt][ft], A, lds_tokfrag(Vs, VP, 16 * ks, 32 * vt, l));
        }
      }
#pragma unroll
      for (int ft = 0; ft < 3; ft++) zadd[ft] += __shfl_xor(zadd[ft], 32);
      if (h == 0) {
#pragma unroll
        for (int ft = 0; ft < 3; ft++) Zw[32 * ft + n32] += zadd[ft];
      }
      __syncthreads();
    }

    float* dst_s = STATE_ONLY ? slot : (last_piece && args.S ? args.S + (size_t)bh * kF * kDV : nullptr);
    float* dst_z = STATE_ONLY ? slot + kF * kDV : (last_piece && args.S ? args.z + (size_t)bh * kF : nullptr);
    if (dst_s) {
      __syncthreads();
      stage_put_tile(Sacc[0], stage, w, 0, l);
      stage_put_tile(Sacc[1], stage, w, 1, l);
      for (int m = l; m < 96; m += 64) stage[kStageS + w * 96 + m] = Zw[m];
      __syncthreads();
      stage_out<256>(stage, dst_s, dst_z);
    }
    __syncthreads();  // Zw and the staging area are reused by the next piece
  }
}

// Exclusive prefix over the pieces of each sequence, in place: slot(bh, g) <- S0 + increments of the
// earlier pieces of sequence bh.  Block (x, bh) covers every gridDim.x-th group of 256 state elements of
// sequence bh (gridDim.x = scan_slices()); the sequence's piece range is worked out once per block, not once
// per element (its 64-bit divisions would otherwise dominate the kernel).
constexpr int kScanMaxFlags = 4096;  // ragged calls: ranges of one sequence whose emptiness is looked up in LDS
__global__ __launch_bounds__(256) void prefill_scan_kernel(const PrefillArgs args, int BH) {
  const int bh = blockIdx.y;
  if (bh >= BH) return;
  const SeqSpan sp = seq_span_of(bh, args);
  if (sp.c1 == sp.c0) return;  // a ragged length of 0: no piece, the caller's state stays as it is
  const long long total = args.lens ? call_chunks<true>(args) : call_chunks<false>(args);
  const int gf = range_of_chunk(sp.c0, total, args.G);
  const int gl = range_of_chunk(sp.c1 - 1, total, args.G);
  // A ragged call may have more ranges than chunks: an empty range between gf and gl holds no piece, so pass 1
  // never wrote its slot and it adds nothing.  A uniform call's plan has no empty ranges.
  __shared__ unsigned char piece[kScanMaxFlags];
  const bool ragged = args.lens != nullptr;
  if (ragged) {
    for (int i = threadIdx.x; i <= gl - gf && i < kScanMaxFlags; i += 256)
      piece[i] = range_lo(gf + i + 1, total, args.G) > range_lo(gf + i, total, args.G);
    __syncthreads();
  }
  auto has_piece = [&](int gg) {
    if (!ragged) return true;
    const int i = gg - gf;
    return i < kScanMaxFlags ? piece[i] != 0 : range_lo(gg + 1, total, args.G) > range_lo(gg, total, args.G);
  };
  for (int e = blockIdx.x * 256 + threadIdx.x; e < kStateFloats; e += gridDim.x * 256) {
    float run = 0.0f;
    if (args.S) run = (e < kF * kDV) ? args.S[(size_t)bh * kF * kDV + e] : args.z[(size_t)bh * kF + (e - kF * kDV)];
    // U slots' increments are loaded at once, then replaced by their prefixes in order
    constexpr int U = 8;
    for (int g0 = gf; g0 <= gl; g0 += U) {
      float d[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int gg = g0 + u;
        d[u] = (gg < gl && has_piece(gg)) ? args.ws_state[(size_t)(bh + gg) * kStateFloats + e] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int gg = g0 + u;
        if (gg <= gl) {
          // a ragged call's pass 3 starts a head piece without a caller state from zero, not from its slot
          if (!ragged || args.S || gg != gf) args.ws_state[(size_t)(bh + gg) * kStateFloats + e] = run;
          run += d[u];
        }
      }
    }
  }
}

// Blocks per sequence of the scan: about eight per workgroup of the call in all, 8 to one per 256 elements.
static int scan_slices(const PrefillArgs& a, int BH) {
  const int want = (8 * a.G + BH - 1) / BH;
  const int most = (kStateFloats + 255) / 256;
  return want < 8 ? 8 : (want > most ? most : want);
}

// ------------------------------------------------------------------------------- host side
bool prefill_chunk_supported(int chunk, sanatan_dtype t) {
  if (chunk == 16 || chunk == 32 || chunk == 64) return true;
  return chunk == 128 && t == SANATAN_BF16;
}

// Compute units of the current device, cached per device (the cache is written once per device; a racing
// first call on two threads stores the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Pieces per sequence above which the separate scan kernel is cheaper than letting each pass-3
// workgroup add up its predecessors' increments.
static constexpr int kFusedScanMaxPieces = 4;

bool prefill_plan(int B, int H, int T, int chunk, int workgroups, bool with_state, PrefillPlan* plan) {
  if (B <= 0 || H <= 0 || T <= 0 || chunk <= 0 || workgroups < 0) return false;
  const long long BH = (long long)B * H;
  const long long ncs = (T + chunk - 1) / chunk;
  const long long total = BH * ncs;
  long long G = workgroups > 0 ? workgroups : device_cus();
  if (G > total) G = total;
  plan->chunk = chunk;
  plan->ncs = (int)ncs;
  plan->G = (int)G;
  plan->total = total;
  plan->rho_bytes = (((size_t)T * kD * sizeof(float)) + 255) & ~(size_t)255;
  plan->state_bytes = (size_t)(BH + G - 1) * kStateFloats * sizeof(float);
  plan->total_bytes = plan->rho_bytes + plan->state_bytes;
  int max_pieces = 1;
  for (long long bh = 0; bh < BH; bh++) {
    const long long c0 = bh * ncs, c1 = c0 + ncs - 1;
    const int np = (int)(((c1 + 1) * G - 1) / total - ((c0 + 1) * G - 1) / total) + 1;
    if (np > max_pieces) max_pieces = np;
  }
  plan->multi = max_pieces > 1;
  // With a caller state and a sequence in several pieces, the state must be read before any piece's
  // final state is written back.  Pass 3 cannot guarantee that (the final piece of a sequence may run
  // on another workgroup before the head piece starts), so the scan kernel, an earlier launch, reads it.
  plan->scanned = max_pieces > kFusedScanMaxPieces || (plan->multi && with_state);
  return true;
}

template <typename T, int CH, bool RAGGED>
static hipError_t launch_prefill4_r(const PrefillArgs& a, int BH, hipStream_t stream) {
  using G = Geom4<T, CH>;
  static_assert(G::lds(false) <= 160 * 1024, "LDS budget");
  if (a.multi) {
    const size_t lds1 = G::lds(true);
    hipError_t e = hipFuncSetAttribute((const void*)prefill4_kernel<T, CH, true, RAGGED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill4_kernel<T, CH, true, RAGGED>), dim3(a.G), dim3(256), lds1, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.scanned) {
      hipLaunchKernelGGL(prefill_scan_kernel, dim3(scan_slices(a, BH), BH), dim3(256), 0, stream, a, BH);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const size_t lds3 = G::lds(false);
  hipError_t e = hipFuncSetAttribute((const void*)prefill4_kernel<T, CH, false, RAGGED>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill4_kernel<T, CH, false, RAGGED>), dim3(a.G), dim3(256), lds3, stream, a);
  return hipGetLastError();
}

template <typename T, int CH>
static hipError_t launch_prefill4_t(const PrefillArgs& a, int BH, hipStream_t stream) {
  return a.lens ? launch_prefill4_r<T, CH, true>(a, BH, stream) : launch_prefill4_r<T, CH, false>(a, BH, stream);
}

hipError_t launch_prefill_scan(const PrefillArgs& a, int BH, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_scan_kernel, dim3(scan_slices(a, BH), BH), dim3(256), 0, stream, a, BH);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                          int64_t pos0, const MethodConsts& mc, float* S, float* z, void* out, void* ws,
                          const PrefillPlan& plan, hipStream_t stream, const int* lens) {
  float* rho = static_cast<float*>(ws);
  hipError_t e = launch_phase_table(rho, T, pos0, mc.log2_base, stream);
  if (e != hipSuccess) return e;
  PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.omega = mc.omega; a.S = S; a.z = z;
  a.ws_state = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.rho_bytes);
  a.rho = rho;
  a.total = plan.total;
  a.lens = lens;
  a.G = plan.G; a.ncs = plan.ncs; a.nph = mc.nph; a.B = B; a.H = H; a.T = T; a.chunk = plan.chunk;
  a.chunk_log2 = 0;
  while ((1 << a.chunk_log2) < plan.chunk) a.chunk_log2++;
  a.multi = plan.multi; a.scanned = plan.scanned;
  if (lens && plan.G > 1) {
    // the pieces depend on lengths the host does not see: any sequence may span several, and a caller
    // state must be read by the scan kernel before any final piece writes it back
    a.multi = 1;
    a.scanned = 1;
  }
  a.kr = mc.kr; a.ceps = mc.ceps;
  const int BH = B * H;
  if (t == SANATAN_BF16) {
    switch (plan.chunk) {
      case 16:
      case 32:
      case 64:
      case 128: return launch_prefill_grp(a, plan.chunk, BH, stream);
    }
  } else {
    switch (plan.chunk) {
      case 16: return launch_prefill4_t<float, 16>(a, BH, stream);
      case 32: return launch_prefill4_t<float, 32>(a, BH, stream);
      case 64: return launch_prefill4_t<float, 64>(a, BH, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sanatan
