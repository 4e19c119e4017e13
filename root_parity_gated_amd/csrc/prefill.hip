// prefill.hip -- chunked causal p = 1 SANATAN attention on bf16 / fp32 MFMA.
//
// Exact regrouping of the recurrence of the SANATAN reading notes §2.7 (sum over s <= t of
// kappa(t,s) v_s, kappa = <Phi(q_t), Phi(k_s)>, §2.3): for a chunk of C tokens with the state
// (S, z) of everything before it,
//     num_t = sum_{s in chunk, s <= t} A_ts v_s + Phi(q_t)^T S,   A = Phi(Q) Phi(K)^T,
//     den_t = sum_{s in chunk, s <= t} A_ts     + Phi(q_t)^T z,   o_t = num_t / (den_t + c eps),
// then S += Phi(K)^T V, z += Phi(K)^T 1.  The denominator rides along as a 65th value column
// (V' = [V | 1], state S' = [S | z]), padded to a fifth 16-wide MFMA tile.
//
// Work split (MI355X-first):
//   * G = #CUs workgroups (4 waves each, one resident per CU) split the flattened (sequence,
//     chunk) list into equal contiguous ranges, so every CU runs the same number of chunks in
//     one round.  A range covering part of a sequence is a "piece": pass 1 computes each
//     non-final piece's state increment, a scan turns them into exclusive prefixes per sequence,
//     pass 3 runs each piece's chunks in order starting from its prefix.  The update is purely
//     additive (the notes stress there is no decay or forgetting), so piece summaries compose
//     by addition.
//   * Wave w owns content dims 16w..16w+15, i.e. 96 of the 384 features (6 channels x 16 dims).
//     Each lane featurizes 4 dims of one token per 16-row block, straight into MFMA operand
//     registers -- Phi never goes to HBM or LDS except one transposed copy of Phi(K) for the
//     state update.  The wave's 96 x 80 slice of S' lives in MFMA accumulators for the whole
//     segment.  Every product is split over waves along the feature axis, so the four waves'
//     partial (num, den) are summed through LDS in a fixed order (deterministic) before the
//     division.
//   * 16x16 MFMA tiles (v_mfma_f32_16x16x32_bf16, or 8 x v_mfma_f32_16x16x4_f32 for fp32 inputs)
//     with token and feature K-slot permutations chosen so that an accumulator tile is directly
//     the next product's operand: A^T tiles feed the A.V product and S' tiles feed the readout
//     without any data movement.
#include <stdlib.h>

#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

// Work partition: the B*H sequences are cut into chunks of C tokens and the flattened
// (sequence, chunk) list is split into G equal contiguous ranges, one per workgroup.  A range
// that crosses sequence boundaries is processed as several "pieces" (one per sequence touched).
// Piece (bh, g) owns boundary-state slot bh + g; slots are disjoint and increasing in (bh, g).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* omega;
  float* S;          // user state [BH][6d][dv] or null
  float* z;          // user state [BH][6d] or null
  float* ws_state;   // [BH + G - 1][kStateFloats] boundary states (pieces' exclusive prefixes)
  const float* rho;  // [T][64] position phases
  long long total;   // BH * ncs chunks
  int G;             // workgroups in the partition
  int ncs;           // chunks per sequence
  int nph, H, T;
  int multi;         // 1 if some sequence spans more than one piece (pass 1 + scan ran)
  float kr, ceps;
};

__device__ __forceinline__ long long range_lo(long long g, const PrefillArgs& a) { return g * a.total / a.G; }

template <typename T, int NB>
struct PrefillGeom {
  static constexpr int C = NB * 16;                    // chunk tokens
  static constexpr int CP = ((C + 31) / 32) * 32;      // padded to whole 32-token K-steps
  static constexpr int NM = CP / 32;                   // token K-steps per chunk
  static constexpr int PITCH = CP + 16 / (int)sizeof(T);  // LDS row pitch (elements); the pad breaks bank aliasing
  static constexpr int QG = NB < 2 ? NB : 2;  // query row-blocks per group (bounds live registers)
  static constexpr size_t vt_bytes = (size_t)kDV * PITCH * sizeof(T);
  static constexpr size_t kt_bytes = (size_t)4 * 96 * PITCH * sizeof(T);
  static constexpr size_t red_bytes = (size_t)4 * QG * 16 * 65 * sizeof(float);
  static constexpr size_t lds_bytes(bool state_only) { return vt_bytes + kt_bytes + (state_only ? 0 : red_bytes); }
};

// Add a state slot ([6d][dv] then z[6d]) into the wave's accumulator slice.
__device__ __forceinline__ void add_state(f32x4 (&Sacc)[6][5], const float* __restrict__ s,
                                          const float* __restrict__ zz, int a0, int r) {
#pragma unroll
  for (int c = 0; c < 6; c++) {
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) Sacc[c][nt][i] += s[(size_t)(c * kD + a0 + i) * kDV + 16 * nt + r];
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < 4; i++) Sacc[c][4][i] += zz[c * kD + a0 + i];
    }
  }
}

__device__ __forceinline__ void store_state(const f32x4 (&Sacc)[6][5], float* __restrict__ s,
                                            float* __restrict__ zz, int a0, int r) {
#pragma unroll
  for (int c = 0; c < 6; c++) {
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) s[(size_t)(c * kD + a0 + i) * kDV + 16 * nt + r] = Sacc[c][nt][i];
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < 4; i++) zz[c * kD + a0 + i] = Sacc[c][4][i];
    }
  }
}

// Featurize 4 dims of one token (validity-masked) into the three operand fragments
// (channels {0,1}, {2,3}, {4,5}); optionally also return the six channel values.
template <typename T>
__device__ __forceinline__ void featurize_frag(const float (&u)[4], const float (&rh)[4], const float (&om4)[4],
                                               float kr, bool valid, typename FragT<T>::type (&F)[3],
                                               float (&ch)[6][4]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float cr, sr, rr;
    featurize1(u[i], rh[i], om4[i], kr, cr, sr, rr);
    ch[0][i] = valid ? 1.0f : 0.0f;
    ch[1][i] = valid ? cr : 0.0f;
    ch[2][i] = valid ? sr : 0.0f;
    ch[3][i] = valid ? rr : 0.0f;
    ch[4][i] = ch[3][i] * ch[1][i];
    ch[5][i] = ch[3][i] * ch[2][i];
  }
  F[0] = pack8<T>(ch[0], ch[1]);
  F[1] = pack8<T>(ch[2], ch[3]);
  F[2] = pack8<T>(ch[4], ch[5]);
}

// Operand fragment of a transposed [row][token] LDS buffer: row `row`, token K-step m, lane quarter qd.
// Slots 0..3: tokens 32m + 4qd + i; slots 4..7: tokens 32m + 16 + 4qd + i.
template <typename T>
__device__ __forceinline__ typename FragT<T>::type lds_tok_frag(const T* __restrict__ buf, int pitch, int row, int m,
                                                                int qd) {
  typename FragT<T>::type f;
  const T* p = buf + row * pitch + 32 * m + 4 * qd;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[i] = p[i];
    f[4 + i] = p[16 + i];
  }
  return f;
}

template <typename T, int NB, bool STATE_ONLY>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const PrefillArgs args) {
  using G = PrefillGeom<T, NB>;
  using Frag = typename FragT<T>::type;
  constexpr int C = G::C, CP = G::CP, NM = G::NM, PITCH = G::PITCH, QG = G::QG;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* Vt = reinterpret_cast<T*>(smem);                         // [64][PITCH]   V^T of the chunk
  T* KT = reinterpret_cast<T*>(smem + G::vt_bytes);           // [4][96][PITCH] Phi(K)^T per wave
  float* red = reinterpret_cast<float*>(smem + G::vt_bytes + G::kt_bytes);  // [4][QG*16][65]

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, qd = l >> 4;
  const int g = blockIdx.x;
  const int Tn = args.T;
  const int a0 = 16 * w + 4 * qd;  // this lane's 4 content dims
  const float kr = args.kr;

  T* KTw = KT + w * 96 * PITCH;
  if (CP > C) {  // padding token columns of Phi(K)^T stay zero for the whole kernel
    for (int idx = l; idx < 96 * (CP - C); idx += 64) KTw[(idx / (CP - C)) * PITCH + C + idx % (CP - C)] = (T)0.0f;
  }
  Frag ONES;  // B operand of the denominator column: column 0 of the fifth tile is all ones
#pragma unroll
  for (int i = 0; i < 8; i++) ONES[i] = (T)(r == 0 ? 1.0f : 0.0f);

  const long long hi = range_lo(g + 1, args);
  for (long long c = range_lo(g, args); c < hi;) {
    const int bh = (int)(c / args.ncs);
    const long long seq_end = (long long)(bh + 1) * args.ncs;
    const long long pend = hi < seq_end ? hi : seq_end;
    const bool last_piece = (pend == seq_end);
    const int t_begin = (int)(c - (long long)bh * args.ncs) * C;
    const int t_end = min(Tn, (int)(pend - (long long)bh * args.ncs) * C);
    c = pend;
    if (STATE_ONLY && last_piece) continue;
    const int h = bh % args.H;
    const T* __restrict__ qp = static_cast<const T*>(args.q) + (size_t)bh * Tn * kD;
    const T* __restrict__ kp = static_cast<const T*>(args.k) + (size_t)bh * Tn * kD;
    const T* __restrict__ vp = static_cast<const T*>(args.v) + (size_t)bh * Tn * kDV;
    T* __restrict__ op = static_cast<T*>(args.out) + (size_t)bh * Tn * kDV;
    float* slot = args.ws_state + (size_t)(bh + g) * kStateFloats;

    float om4[4];
#pragma unroll
    for (int i = 0; i < 4; i++) om4[i] = anchor_rev(args.omega[(size_t)(h % args.nph) * kD + a0 + i]);

    f32x4 Sacc[6][5];
#pragma unroll
    for (int cc = 0; cc < 6; cc++)
#pragma unroll
      for (int nt = 0; nt < 5; nt++) Sacc[cc][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!STATE_ONLY) {
      if (args.multi) add_state(Sacc, slot, slot + kF * kDV, a0, r);
      else if (args.S) add_state(Sacc, args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF, a0, r);
    }

    for (int t0 = t_begin; t0 < t_end; t0 += C) {
      const int nvalid = min(C, t_end - t0);

      // (a) V chunk -> LDS, transposed to [value col][token]; tokens >= nvalid are zero.
      {
        constexpr int E = 16 / (int)sizeof(T);
        constexpr int TPT = kDV / E;
        constexpr int TOKS = 256 / TPT;
        const int n0 = (tid % TPT) * E;
        for (int s = tid / TPT; s < CP; s += TOKS) {
          T vals[E];
          if (s < nvalid) {
            const uint4 raw = *reinterpret_cast<const uint4*>(vp + (size_t)(t0 + s) * kDV + n0);
            const T* rv = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int j = 0; j < E; j++) vals[j] = rv[j];
          } else {
#pragma unroll
            for (int j = 0; j < E; j++) vals[j] = (T)0.0f;
          }
#pragma unroll
          for (int j = 0; j < E; j++) Vt[(n0 + j) * PITCH + s] = vals[j];
        }
      }

      // (b) Phi(K): operand fragments in registers + transposed copy in this wave's LDS slice.
      Frag KF[NB][3];
#pragma unroll
      for (int rb = 0; rb < NB; rb++) {
        const int sl = 16 * rb + r;
        const bool valid = sl < nvalid;
        float u[4] = {0.f, 0.f, 0.f, 0.f}, rh[4] = {0.f, 0.f, 0.f, 0.f};
        if (valid) {
          load4(kp + (size_t)(t0 + sl) * kD + a0, u);
          load4(args.rho + (size_t)(t0 + sl) * kD + a0, rh);
        }
        float ch[6][4];
        featurize_frag<T>(u, rh, om4, kr, valid, KF[rb], ch);
#pragma unroll
        for (int c = 0; c < 6; c++)
#pragma unroll
          for (int i = 0; i < 4; i++) KTw[(c * 16 + 4 * qd + i) * PITCH + sl] = (T)ch[c][i];
      }
      __syncthreads();

      if (!STATE_ONLY) {
#pragma unroll
        for (int qg = 0; qg < NB; qg += QG) {
          // Phi(Q) for query row-blocks g .. g+QG-1
          Frag QF[QG][3];
#pragma unroll
          for (int tbl = 0; tbl < QG; tbl++) {
            const int tl = 16 * (qg + tbl) + r;
            const bool valid = (qg + tbl < NB) && tl < nvalid;
            float u[4] = {0.f, 0.f, 0.f, 0.f}, rh[4] = {0.f, 0.f, 0.f, 0.f};
            if (valid) {
              load4(qp + (size_t)(t0 + tl) * kD + a0, u);
              load4(args.rho + (size_t)(t0 + tl) * kD + a0, rh);
            }
            float ch[6][4];
            featurize_frag<T>(u, rh, om4, kr, valid, QF[tbl], ch);
          }
          f32x4 num[QG][5];
#pragma unroll
          for (int tbl = 0; tbl < QG; tbl++)
#pragma unroll
            for (int nt = 0; nt < 5; nt++) num[tbl][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

          // intra-chunk: A^T tiles (rows s, cols t) over this wave's 96 features, masked s <= t,
          // then straight into the A.V' product as the A operand.
#pragma unroll
          for (int tbl = 0; tbl < QG; tbl++) {
            const int tb = qg + tbl;
            if (tb >= NB) continue;
#pragma unroll
            for (int m = 0; 2 * m <= tb; m++) {
              const int sb0 = 2 * m, sb1 = 2 * m + 1;
              f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int j = 0; j < 3; j++) mma(d0, KF[sb0][j], QF[tbl][j]);
              if (sb1 <= tb) {
#pragma unroll
                for (int j = 0; j < 3; j++) mma(d1, KF[sb1][j], QF[tbl][j]);
              }
              if (sb0 == tb) {
#pragma unroll
                for (int i = 0; i < 4; i++) d0[i] = (4 * qd + i > r) ? 0.0f : d0[i];
              }
              if (sb1 == tb) {
#pragma unroll
                for (int i = 0; i < 4; i++) d1[i] = (4 * qd + i > r) ? 0.0f : d1[i];
              }
              const Frag P = pack8v<T>(d0, d1);
#pragma unroll
              for (int nt = 0; nt < 4; nt++) mma(num[tbl][nt], P, lds_tok_frag<T>(Vt, PITCH, 16 * nt + r, m, qd));
              mma(num[tbl][4], P, ONES);
            }
          }
          // inter-chunk readout with the state before this chunk: num += Phi(Q) S'
#pragma unroll
          for (int j = 0; j < 3; j++) {
#pragma unroll
            for (int nt = 0; nt < 5; nt++) {
              const Frag SB = pack8v<T>(Sacc[2 * j][nt], Sacc[2 * j + 1][nt]);
#pragma unroll
              for (int tbl = 0; tbl < QG; tbl++)
                if (qg + tbl < NB) mma(num[tbl][nt], QF[tbl][j], SB);
            }
          }
          // cross-wave sum of the partial (num, den) in a fixed order, then divide and store.
          float* redw = red + (size_t)w * QG * 16 * 65;
#pragma unroll
          for (int tbl = 0; tbl < QG; tbl++) {
#pragma unroll
            for (int nt = 0; nt < 4; nt++)
#pragma unroll
              for (int i = 0; i < 4; i++) redw[(16 * tbl + 4 * qd + i) * 65 + 16 * nt + r] = num[tbl][nt][i];
            if (r == 0) {
#pragma unroll
              for (int i = 0; i < 4; i++) redw[(16 * tbl + 4 * qd + i) * 65 + 64] = num[tbl][4][i];
            }
          }
          __syncthreads();
          {
            constexpr int ROWS = QG * 16;
            constexpr int CPT = ROWS * kDV / 256;
            constexpr int TPR = kDV / CPT;
            const int row = tid / TPR;
            const int c0 = (tid % TPR) * CPT;
            const int tl = 16 * qg + row;
            if (tl < nvalid) {
              constexpr int WS = QG * 16 * 65;
              const float den = ((red[row * 65 + 64] + red[WS + row * 65 + 64]) + red[2 * WS + row * 65 + 64]) +
                                red[3 * WS + row * 65 + 64];
              const float inv = 1.0f / (den + args.ceps);
              T o[CPT];
#pragma unroll
              for (int cc = 0; cc < CPT; cc++) {
                const int idx = row * 65 + c0 + cc;
                const float s = ((red[idx] + red[WS + idx]) + red[2 * WS + idx]) + red[3 * WS + idx];
                o[cc] = from_f32<T>(s * inv);
              }
              T* dst = op + (size_t)(t0 + tl) * kDV + c0;
#pragma unroll
              for (int cc = 0; cc < CPT; cc++) dst[cc] = o[cc];
            }
          }
          __syncthreads();
        }
      }

      // state update S' += Phi(K)^T V' (this wave's 96 feature rows), after this chunk's readout.
#pragma unroll
      for (int c = 0; c < 6; c++) {
#pragma unroll
        for (int m = 0; m < NM; m++) {
          const Frag A = lds_tok_frag<T>(KTw, PITCH, c * 16 + r, m, qd);
#pragma unroll
          for (int nt = 0; nt < 4; nt++) mma(Sacc[c][nt], A, lds_tok_frag<T>(Vt, PITCH, 16 * nt + r, m, qd));
          mma(Sacc[c][4], A, ONES);
        }
      }
      __syncthreads();
    }

    if (STATE_ONLY) {
      store_state(Sacc, slot, slot + kF * kDV, a0, r);
    } else if (last_piece && args.S) {
      store_state(Sacc, args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF, a0, r);
    }
  }  // pieces
}

// Exclusive prefix over the pieces of each sequence, in place: slot(bh, g) <- S0 + sum of the
// increments of the earlier pieces of sequence bh.  One thread per (sequence, state element).
__global__ __launch_bounds__(256) void prefill_scan_kernel(const PrefillArgs args, int BH) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= kStateFloats || bh >= BH) return;
  const long long c0 = (long long)bh * args.ncs, c1 = c0 + args.ncs - 1;
  const int gf = (int)(((c0 + 1) * args.G - 1) / args.total);
  const int gl = (int)(((c1 + 1) * args.G - 1) / args.total);
  float run = 0.0f;
  if (args.S) run = (e < kF * kDV) ? args.S[(size_t)bh * kF * kDV + e] : args.z[(size_t)bh * kF + (e - kF * kDV)];
  for (int g = gf; g <= gl; g++) {
    float* p = args.ws_state + (size_t)(bh + g) * kStateFloats + e;
    const float d = (g < gl) ? *p : 0.0f;
    *p = run;
    run += d;
  }
}

// ------------------------------------------------------------------------------- host side
bool prefill_chunk_supported(int chunk, sanatan_dtype t) {
  if (chunk == 16 || chunk == 32 || chunk == 64) return true;
  return chunk == 128 && t == SANATAN_BF16;
}

static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

bool prefill_plan(int B, int H, int T, int chunk, PrefillPlan* plan) {
  if (B <= 0 || H <= 0 || T <= 0 || chunk <= 0) return false;
  const long long BH = (long long)B * H;
  const long long ncs = (T + chunk - 1) / chunk;
  const long long total = BH * ncs;
  // One resident workgroup per CU: G = #CUs equal ranges fill the chip in one round.
  long long G = device_cus();
  const char* env = getenv("SANATAN_PREFILL_WGS");
  if (env && atoll(env) > 0) G = atoll(env);
  if (G > total) G = total;
  plan->chunk = chunk;
  plan->ncs = (int)ncs;
  plan->G = (int)G;
  plan->total = total;
  plan->rho_bytes = (((size_t)T * kD * sizeof(float)) + 255) & ~(size_t)255;
  plan->state_bytes = (size_t)(BH + G - 1) * kStateFloats * sizeof(float);
  plan->total_bytes = plan->rho_bytes + plan->state_bytes;
  // Does any sequence span more than one range?  (then pass 1 and the scan are needed)
  plan->multi = 0;
  for (long long bh = 0; bh < BH && !plan->multi; bh++) {
    const long long c0 = bh * ncs, c1 = c0 + ncs - 1;
    if (((c0 + 1) * G - 1) / total != ((c1 + 1) * G - 1) / total) plan->multi = 1;
  }
  return true;
}

template <typename T, int NB>
static hipError_t launch_prefill_t(const PrefillArgs& a, int BH, hipStream_t stream) {
  using G = PrefillGeom<T, NB>;
  if (a.multi) {
    const size_t lds1 = G::lds_bytes(true);
    hipError_t e = hipFuncSetAttribute((const void*)prefill_kernel<T, NB, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_kernel<T, NB, true>), dim3(a.G), dim3(256), lds1, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_scan_kernel, dim3((kStateFloats + 255) / 256, BH), dim3(256), 0, stream, a, BH);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds3 = G::lds_bytes(false);
  hipError_t e = hipFuncSetAttribute((const void*)prefill_kernel<T, NB, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<T, NB, false>), dim3(a.G), dim3(256), lds3, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, sanatan_dtype t, int B, int H, int T,
                          int64_t pos0, const MethodConsts& mc, float* S, float* z, void* out, void* ws,
                          const PrefillPlan& plan, hipStream_t stream) {
  float* rho = static_cast<float*>(ws);
  float* ws_state = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.rho_bytes);
  hipError_t e = launch_phase_table(rho, T, pos0, mc.log2_base, stream);
  if (e != hipSuccess) return e;
  PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.omega = mc.omega; a.S = S; a.z = z; a.ws_state = ws_state; a.rho = rho;
  a.total = plan.total; a.G = plan.G; a.ncs = plan.ncs; a.multi = plan.multi;
  a.nph = mc.nph; a.H = H; a.T = T;
  a.kr = mc.kr; a.ceps = mc.ceps;
  const int BH = B * H;
  const int nb = plan.chunk / 16;
  if (t == SANATAN_BF16) {
    switch (nb) {
      case 1: return launch_prefill_t<__bf16, 1>(a, BH, stream);
      case 2: return launch_prefill_t<__bf16, 2>(a, BH, stream);
      case 4: return launch_prefill_t<__bf16, 4>(a, BH, stream);
      case 8: return launch_prefill_t<__bf16, 8>(a, BH, stream);
    }
  } else {
    switch (nb) {
      case 1: return launch_prefill_t<float, 1>(a, BH, stream);
      case 2: return launch_prefill_t<float, 2>(a, BH, stream);
      case 4: return launch_prefill_t<float, 4>(a, BH, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace sanatan
