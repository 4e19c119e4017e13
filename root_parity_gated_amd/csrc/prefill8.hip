// prefill8.hip -- 8-wave bf16 chunked causal p = 1 prefill for chunks of 16, 32 or 64 tokens.
//
// Same mathematics and work partition as prefill.hip (exact chunked regrouping of the recurrence
// of the SANATAN reading notes §2.7).  What changes is the wave layout, chosen so that two waves
// share each SIMD and hide each other's LDS / memory latency:
//   * wave (g, role), g = feature group 0..3 (content dims 16g..16g+15 = 96 features), role 0/1.
//   * role 0 featurizes the chunk's keys into the token-major tile KS[g], role 1 its queries into
//     QS[g] (and the readout part of the denominator, Phi(q) . z).  Both roles form the same
//     intra-chunk A^T tiles from those tiles (the duplicated 18 MFMAs per chunk are cheaper than
//     an exchange), and each role owns one 32-column value tile: role r accumulates
//     num^T[v in 32r..32r+31] and keeps rows of S (96 x 32) for those columns in accumulators.
//   * per-wave registers stay under 256 (VGPR + AGPR), so the 8 waves of one workgroup give two
//     waves per SIMD; the next chunk's q/k/v rows and phases are prefetched into registers while
//     the current chunk computes.
#include "prefill_common.h"

namespace sanatan {

template <int CH>
struct Geom8 {
  static constexpr int TB = (CH + 31) / 32;   // 32-token blocks per chunk
  static constexpr int CT = 32 * TB;          // tile tokens
  static constexpr int VP = 72;               // Vs pitch (bf16 elements)
  static constexpr int KP = 104;              // KS / QS pitch (bf16 elements)
  static constexpr int RP = 68;               // red pitch (floats): 64 values, row sum at 64
  static constexpr size_t vs_bytes = (size_t)CT * VP * 2;
  static constexpr size_t ks_bytes = (size_t)4 * CT * KP * 2;
  static constexpr size_t red_bytes = (size_t)4 * 32 * RP * 4;
  static constexpr size_t dz_bytes = (size_t)4 * CT * 4;
  static constexpr size_t z_bytes = 4 * 96 * 4;
  static constexpr size_t stage_bytes = (size_t)(kF * kDV + kF) * 4;
  static constexpr size_t body(bool state_only) { return vs_bytes + ks_bytes + (state_only ? 0 : ks_bytes + red_bytes); }
  static constexpr size_t lds(bool state_only) {
    return (body(state_only) > stage_bytes ? body(state_only) : stage_bytes) + dz_bytes + z_bytes;
  }
};

template <int CH, bool STATE_ONLY>
__global__ __launch_bounds__(512, 2) void prefill8_kernel(const PrefillArgs args) {
  using G = Geom8<CH>;
  typedef bf16x8 Frag;
  constexpr int TB = G::TB, CT = G::CT, VP = G::VP, KP = G::KP, RP = G::RP;
  constexpr size_t LDS = G::lds(STATE_ONLY);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __bf16* Vs = reinterpret_cast<__bf16*>(smem);                             // [CT][VP] V
  __bf16* KS = reinterpret_cast<__bf16*>(smem + G::vs_bytes);               // [4][CT][KP] Phi(K)
  __bf16* QS = reinterpret_cast<__bf16*>(smem + G::vs_bytes + G::ks_bytes);  // [4][CT][KP] Phi(Q)
  float* red = reinterpret_cast<float*>(smem + G::vs_bytes + 2 * G::ks_bytes);  // [4][32][RP]
  float* stage = reinterpret_cast<float*>(smem);                                 // state staging (aliases)
  float* Zb = reinterpret_cast<float*>(smem + LDS - G::z_bytes);                 // [4][96] z
  float* DZ = reinterpret_cast<float*>(smem + LDS - G::z_bytes - G::dz_bytes);   // [4][CT] Phi(q).z parts

  const int tid = threadIdx.x, w8 = tid >> 6, grp = w8 & 3, role = w8 >> 2;
  const int l = tid & 63, h = l >> 5, n32 = l & 31;
  const int g = blockIdx.x;
  const int Tn = args.T;
  __bf16* KSg = KS + grp * CT * KP;
  __bf16* QSg = QS + grp * CT * KP;
  float* Zg = Zb + grp * 96;
  float* DZg = DZ + grp * CT;
  const int dbase = 16 * grp + 4 * h;  // this lane's dims: dbase + {0..3, 8..11}
  // token blocks this wave featurizes: pass 3 -> role 0 keys, role 1 queries (all blocks);
  // pass 1 -> keys, blocks split between the roles.
  constexpr int NF = STATE_ONLY ? (TB + 1) / 2 : TB;

  const long long hi = range_lo(g + 1, args);
  for (long long c = range_lo(g, args); c < hi;) {
    const int bh = (int)(c / args.ncs);
    const long long seq_c0 = (long long)bh * args.ncs;
    const long long seq_end = seq_c0 + args.ncs;
    const long long pend = hi < seq_end ? hi : seq_end;
    const bool last_piece = (pend == seq_end);
    const int t_begin = (int)(c - seq_c0) * CH;
    const int t_end = min(Tn, (int)(pend - seq_c0) * CH);
    c = pend;
    if (STATE_ONLY && last_piece) continue;
    const int hh = bh % args.H;
    const bool feat_q = !STATE_ONLY && role == 1;
    const __bf16* __restrict__ src = static_cast<const __bf16*>(feat_q ? args.q : args.k) + (size_t)bh * Tn * kD;
    const __bf16* __restrict__ vp = static_cast<const __bf16*>(args.v) + (size_t)bh * Tn * kDV;
    __bf16* __restrict__ op = static_cast<__bf16*>(args.out) + (size_t)bh * Tn * kDV;
    float* slot = args.ws_state + (size_t)(bh + g) * kStateFloats;

    float om4[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      om4[i] = anchor_rev(args.omega[(size_t)(hh % args.nph) * kD + dbase + (i & 3) + 8 * (i >> 2)]);

    // ---- initial state of the piece: this wave's value tile of its group's S, and z (role 0)
    f32x16 Sacc[3];
#pragma unroll
    for (int ft = 0; ft < 3; ft++) zero16(Sacc[ft]);
    if (role == 0)
      for (int m = l; m < 96; m += 64) Zg[m] = 0.0f;
    if (!STATE_ONLY) {
      auto add_slot = [&](const float* s, const float* zz) {
        __syncthreads();
        stage_in<512>(stage, s, zz);
        __syncthreads();
        stage_add_tile(Sacc, stage, grp, role, l);
        if (role == 0)
          for (int m = l; m < 96; m += 64) Zg[m] += stage[kStageS + grp * 96 + m];
      };
      if (args.multi && args.scanned) {
        add_slot(slot, slot + kF * kDV);
      } else {
        if (args.S) add_slot(args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF);
        if (args.multi) {  // few pieces per sequence: add the earlier pieces' increments here
          const int gf = range_of_chunk(seq_c0, args);
          for (int gg = gf; gg < g; gg++) {
            const float* sj = args.ws_state + (size_t)(bh + gg) * kStateFloats;
            add_slot(sj, sj + kF * kDV);
          }
        }
      }
    }
    __syncthreads();  // the staging area is reused by the tiles; Zg initialised

    // ---- register prefetch of one chunk: this wave's rows + phases, and one 16-byte piece of V
    bf16x4 pu[NF][2];
    float4 pr[NF][2];
    uint4 pv;
    auto prefetch = [&](int t0) {
      const int nv = min(CH, t_end - t0);
#pragma unroll
      for (int f = 0; f < NF; f++) {
        const int blk = STATE_ONLY ? 2 * f + role : f;
        const int tc = t0 + min(32 * blk + n32, nv - 1);
        const __bf16* pu_src = src + (size_t)tc * kD + dbase;
        const float* pr_src = args.rho + (size_t)tc * kD + dbase;
        pu[f][0] = *reinterpret_cast<const bf16x4*>(pu_src);
        pu[f][1] = *reinterpret_cast<const bf16x4*>(pu_src + 8);
        pr[f][0] = *reinterpret_cast<const float4*>(pr_src);
        pr[f][1] = *reinterpret_cast<const float4*>(pr_src + 8);
      }
      const int s = tid >> 3, col = 8 * (tid & 7);
      if (s < CT) pv = *reinterpret_cast<const uint4*>(vp + (size_t)(t0 + min(s, nv - 1)) * kDV + col);
    };
    prefetch(t_begin);

    for (int t0 = t_begin; t0 < t_end; t0 += CH) {
      const int nvalid = min(CH, t_end - t0);

      // (a) V piece -> LDS; featurize this wave's rows into its token-major tile
      {
        const int s = tid >> 3, col = 8 * (tid & 7);
        if (s < CT) *reinterpret_cast<uint4*>(Vs + s * VP + col) = (s < nvalid) ? pv : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int f = 0; f < NF; f++) {
        const int blk = STATE_ONLY ? 2 * f + role : f;
        if (blk >= TB) continue;
        const int sl = 32 * blk + n32;
        float u[8], rh[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          u[i] = (float)pu[f][0][i];
          u[4 + i] = (float)pu[f][1][i];
        }
        rh[0] = pr[f][0].x; rh[1] = pr[f][0].y; rh[2] = pr[f][0].z; rh[3] = pr[f][0].w;
        rh[4] = pr[f][1].x; rh[5] = pr[f][1].y; rh[6] = pr[f][1].z; rh[7] = pr[f][1].w;
        float ch[6][8];
        featurize8(u, rh, om4, args.kr, ch);
        if (feat_q) {
          // readout part of the denominator: Phi(q) . z for this group's features
          float dz = 0.0f;
#pragma unroll
          for (int cc = 0; cc < 6; cc++) {
            const float4 za = *reinterpret_cast<const float4*>(Zg + 16 * cc + 4 * h);
            const float4 zb = *reinterpret_cast<const float4*>(Zg + 16 * cc + 8 + 4 * h);
            dz = fmaf(ch[cc][0], za.x, dz); dz = fmaf(ch[cc][1], za.y, dz);
            dz = fmaf(ch[cc][2], za.z, dz); dz = fmaf(ch[cc][3], za.w, dz);
            dz = fmaf(ch[cc][4], zb.x, dz); dz = fmaf(ch[cc][5], zb.y, dz);
            dz = fmaf(ch[cc][6], zb.z, dz); dz = fmaf(ch[cc][7], zb.w, dz);
          }
          dz += __shfl_xor(dz, 32);
          if (h == 0) DZg[sl] = dz;
        }
        const bool keep = feat_q || sl < nvalid;  // key rows beyond the chunk end are zero
        __bf16* row = (feat_q ? QSg : KSg) + sl * KP + 4 * h;
#pragma unroll
        for (int cc = 0; cc < 6; cc++) {
          bf16x4 a, b;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            a[i] = (__bf16)(keep ? ch[cc][i] : 0.0f);
            b[i] = (__bf16)(keep ? ch[cc][4 + i] : 0.0f);
          }
          *reinterpret_cast<bf16x4*>(row + 16 * cc) = a;
          *reinterpret_cast<bf16x4*>(row + 16 * cc + 8) = b;
        }
      }
      if (t0 + CH < t_end) prefetch(t0 + CH);  // next chunk's loads fly while this one computes
      __syncthreads();

      if (!STATE_ONLY) {
        // readout operands S^T (rows v of this wave's tile, K = features) from the state before this chunk
        Frag SA[6];
#pragma unroll
        for (int cc = 0; cc < 6; cc++) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] = Sacc[cc >> 1][8 * (cc & 1) + i];
          SA[cc] = pack8f<__bf16>(x);
        }
#pragma unroll
        for (int tb = 0; tb < TB; tb++) {
          Frag QF[6];
#pragma unroll
          for (int cc = 0; cc < 6; cc++) QF[cc] = lds_rowfrag<__bf16>(QSg, KP, 32 * tb + n32, cc, h);
          f32x16 numT;
          zero16(numT);
          float rs = 0.0f;
#pragma unroll
          for (int sb = 0; sb <= tb; sb++) {
            f32x16 at;
            zero16(at);
#pragma unroll
            for (int cc = 0; cc < 6; cc++) mma32(at, lds_rowfrag<__bf16>(KSg, KP, 32 * sb + n32, cc, h), QF[cc]);
            float lo[8], hi2[8];
#pragma unroll
            for (int i = 0; i < 16; i++) {
              const int sl = 8 * (i >> 2) + 4 * h + (i & 3);
              const float a = (sb == tb && sl > n32) ? 0.0f : at[i];
              if (i < 8) lo[i] = a;
              else hi2[i - 8] = a;
            }
            const Frag P0 = pack8f<__bf16>(lo), P1 = pack8f<__bf16>(hi2);
            if (role == 0) rs = frag_sum(P1, frag_sum(P0, rs));
            mma32(numT, lds_tokfrag(Vs, VP, 32 * sb, 32 * role, l), P0);
            mma32(numT, lds_tokfrag(Vs, VP, 32 * sb + 16, 32 * role, l), P1);
          }
#pragma unroll
          for (int cc = 0; cc < 6; cc++) mma32(numT, SA[cc], QF[cc]);
          float* rw = red + grp * 32 * RP + n32 * RP + 32 * role;
#pragma unroll
          for (int j = 0; j < 4; j++)
            *reinterpret_cast<float4*>(rw + 8 * j + 4 * h) =
                make_float4(numT[4 * j], numT[4 * j + 1], numT[4 * j + 2], numT[4 * j + 3]);
          if (role == 0) {
            rs += __shfl_xor(rs, 32);
            if (h == 0) red[grp * 32 * RP + n32 * RP + 64] = rs;
          }
          __syncthreads();
          {
            const int row = tid >> 4, v0 = 4 * (tid & 15);
            const int t_out = 32 * tb + row;
            if (t_out < nvalid) {
              constexpr int WS = 32 * RP;
              const int ri = row * RP;
              const float den = ((((red[ri + 64] + DZ[32 * tb + row]) + (red[WS + ri + 64] + DZ[CT + 32 * tb + row])) +
                                  (red[2 * WS + ri + 64] + DZ[2 * CT + 32 * tb + row])) +
                                 (red[3 * WS + ri + 64] + DZ[3 * CT + 32 * tb + row]));
              const float inv = 1.0f / (den + args.ceps);
              const float4 a0 = *reinterpret_cast<const float4*>(red + ri + v0);
              const float4 a1 = *reinterpret_cast<const float4*>(red + WS + ri + v0);
              const float4 a2 = *reinterpret_cast<const float4*>(red + 2 * WS + ri + v0);
              const float4 a3 = *reinterpret_cast<const float4*>(red + 3 * WS + ri + v0);
              bf16x4 o;
              o[0] = (__bf16)((((a0.x + a1.x) + a2.x) + a3.x) * inv);
              o[1] = (__bf16)((((a0.y + a1.y) + a2.y) + a3.y) * inv);
              o[2] = (__bf16)((((a0.z + a1.z) + a2.z) + a3.z) * inv);
              o[3] = (__bf16)((((a0.w + a1.w) + a2.w) + a3.w) * inv);
              *reinterpret_cast<bf16x4*>(op + (size_t)(t0 + t_out) * kDV + v0) = o;
            }
          }
          __syncthreads();
        }
      }

      // state update: S[:, this wave's value tile] += Phi(K)^T V; role 0 also z += Phi(K)^T 1
      float zadd[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2 * TB; ks++) {
        const Frag B = lds_tokfrag(Vs, VP, 16 * ks, 32 * role, l);
#pragma unroll
        for (int ft = 0; ft < 3; ft++) {
          const Frag A = lds_tokfrag(KSg, KP, 16 * ks, 32 * ft, l);
          if (role == 0) zadd[ft] = frag_sum(A, zadd[ft]);
          mma32(Sacc[ft], A, B);
        }
      }
      if (role == 0) {
#pragma unroll
        for (int ft = 0; ft < 3; ft++) zadd[ft] += __shfl_xor(zadd[ft], 32);
        if (h == 0) {
#pragma unroll
          for (int ft = 0; ft < 3; ft++) Zg[32 * ft + n32] += zadd[ft];
        }
      }
      __syncthreads();
    }

    float* dst_s = STATE_ONLY ? slot : (last_piece && args.S ? args.S + (size_t)bh * kF * kDV : nullptr);
    float* dst_z = STATE_ONLY ? slot + kF * kDV : (last_piece && args.S ? args.z + (size_t)bh * kF : nullptr);
    if (dst_s) {
      stage_put_tile(Sacc, stage, grp, role, l);
      if (role == 0)
        for (int m = l; m < 96; m += 64) stage[kStageS + grp * 96 + m] = Zg[m];
      __syncthreads();
      stage_out<512>(stage, dst_s, dst_z);
    }
    __syncthreads();  // Zg and the staging area are reused by the next piece
  }
}

template <int CH>
static hipError_t launch8_t(const PrefillArgs& a, int BH, hipStream_t stream) {
  using G = Geom8<CH>;
  static_assert(G::lds(false) <= 160 * 1024, "LDS budget");
  if (a.multi) {
    const size_t lds1 = G::lds(true);
    hipError_t e = hipFuncSetAttribute((const void*)prefill8_kernel<CH, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill8_kernel<CH, true>), dim3(a.G), dim3(512), lds1, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.scanned) {
      e = launch_prefill_scan(a, BH, stream);
      if (e != hipSuccess) return e;
    }
  }
  const size_t lds3 = G::lds(false);
  hipError_t e = hipFuncSetAttribute((const void*)prefill8_kernel<CH, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill8_kernel<CH, false>), dim3(a.G), dim3(512), lds3, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill8(const PrefillArgs& a, int chunk, int BH, hipStream_t stream) {
  switch (chunk) {
    case 16: return launch8_t<16>(a, BH, stream);
    case 32: return launch8_t<32>(a, BH, stream);
    case 64: return launch8_t<64>(a, BH, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sanatan
