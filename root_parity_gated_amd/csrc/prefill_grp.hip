// prefill_grp.hip -- bf16 chunked causal p = 1 prefill, one wave per feature group.
//
// Mathematics: the chunked regrouping of the recurrence of the SANATAN reading notes §2.7 (intra-chunk
// masked Phi(Q) Phi(K)^T V, inter-chunk readout Phi(Q) S and Phi(Q) . z, state update S += Phi(K)^T V,
// z += Phi(K)^T 1), with the work partition of prefill.hip (pieces of the flattened chunk list, pass 1 =
// increments of non-final pieces, pass 3 = outputs).
//
// Layout.  A workgroup is 4 waves, one per SIMD; wave g owns feature group g = content dims 16g..16g+15,
// i.e. the 96 features (channel c, dim) of those dims, and the 96 x 64 slice of S for them (6 accumulator
// tiles of 32 x 32 fp32, 96 AGPR/VGPR per lane).  Lane (n32 = l % 32, h = l / 32) featurizes token n32 of
// each 32-token block, dims 16g + 8h .. 16g + 8h + 7: exactly the 8 K-slots it supplies to the MFMA
// operands of Phi(Q) and Phi(K) (K-step = channel), so the intra-chunk product and the readout take
// their feature operands straight from registers.  Only Phi(K) is written to LDS (wave-private, for the
// transposed read of the state update), with V (also wave-private).  The one cross-wave exchange is
// the reduction of the four groups' partial numerators and denominators before the normalisation.
//
// Accumulator row order.  In a 32-row accumulator tile, lane half h holds rows {4h..4h+3, 8+4h..11+4h}
// of each 16-row block, while it featurized dims 8h..8h+7; the state rows are therefore ordered
// with bits 2 and 3 of the dim swapped (swz16), and the transposed LDS read of Phi(K) for the update
// uses the same swap, so readout K-slots and state rows line up.
//
// Channel 0 of Phi is the constant 1: in the intra-chunk product its 16 features contribute exactly
// 16 to every entry, which one MFMA on two fragments of ones supplies (it costs the VALU nothing, unlike
// writing 16 accumulator registers).  The bf16 kernels for 16-, 32- and 64-token chunks and the one for
// 128-token chunks (further below) share this layout.
#include <atomic>

#include "prefill_common.h"

namespace sanatan {
namespace {

__device__ __forceinline__ int swz16(int d) { return (d & 3) | ((d >> 1) & 4) | ((d << 1) & 8); }

constexpr unsigned kOnes2 = 0x3F803F80u;  // two bf16 ones

template <int CH>
struct GeomG {
  static constexpr int TB = (CH + 31) / 32;  // 32-token blocks per chunk
  static constexpr int CT = 32 * TB;         // tile tokens
  static constexpr int KP = 104;             // Phi(K) tile pitch (bf16): 96 features + 8
  static constexpr int VP = 72;              // V tile pitch (bf16)
  static constexpr int RP = 68;              // reduction pitch (floats): 64 values, denominator at 64
  static constexpr int ks_bytes = CT * KP * 2;   // one wave's Phi(K) tile
  static constexpr int vs_bytes = CT * VP * 2;   // one V tile
  static constexpr int red_bytes = TB * 4 * 32 * RP * 4;
  // pass 3: [Phi(K) x 4 waves][V x 2 (shared, double-buffered)][reduction]; pass 1: [Phi(K) x 4][V x 4 (private)]
  static constexpr int vs_off = 4 * ks_bytes;
  static constexpr int red_off = vs_off + 2 * vs_bytes;
  static constexpr int main_bytes(bool state_only) { return state_only ? vs_off + 4 * vs_bytes : red_off + red_bytes; }
  // z per wave: fp32 [96], then (pass 3) a bf16 copy [96] for the readout's denominator
  static constexpr int lds(bool state_only) { return main_bytes(state_only) + 4 * 96 * 4 + 4 * 96 * 2; }
};

// The state slice of wave g lives in its accumulators: tile (ft, vt), register i = 8 m + j, lane (hh, n32)
// holds S[128 ft + 64 m + 16 g + 8 hh + 4 (j / 4) + j % 4][32 vt + n32] (rows are channel-major features;
// this is the accumulator layout with the dim bits 2 and 3 swapped).  For one register the 64 lanes
// cover two 128-byte row segments, so the state moves between global memory and the accumulators with
// plain coalesced loads and stores whose offsets are immediates.  z of the group is kept in LDS as
// Zg[16 c + dim], dim = 0..15.
// LOWREG keeps one tile's loads in flight at a time, for callers without registers to spare.
template <bool LOWREG = false>
__device__ __forceinline__ void gstate_add(f32x16 (&Sacc)[3][2], float* Zg, const float* __restrict__ s,
                                           const float* __restrict__ zz, int g, int l) {
  const float* base = s + (16 * g + 8 * (l >> 5)) * kDV + (l & 31);
#pragma unroll
  for (int ft = 0; ft < 3; ft++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++) {
#pragma unroll
      for (int m = 0; m < 2; m++) {
        const float* p = base + (128 * ft + 64 * m) * kDV + 32 * vt;
#pragma unroll
        for (int j = 0; j < 8; j++) Sacc[ft][vt][8 * m + j] += p[(4 * (j >> 2) + (j & 3)) * kDV];
      }
      if (LOWREG) __builtin_amdgcn_sched_barrier(0);
    }
  for (int m = l; m < 96; m += 64) Zg[m] += zz[64 * (m >> 4) + 16 * g + (m & 15)];
}
__device__ __forceinline__ void gstate_store_s(const f32x16 (&Sacc)[3][2], float* __restrict__ s, int g, int l) {
  float* base = s + (16 * g + 8 * (l >> 5)) * kDV + (l & 31);
#pragma unroll
  for (int ft = 0; ft < 3; ft++)
#pragma unroll
    for (int vt = 0; vt < 2; vt++)
#pragma unroll
      for (int m = 0; m < 2; m++) {
        float* p = base + (128 * ft + 64 * m) * kDV + 32 * vt;
#pragma unroll
        for (int j = 0; j < 8; j++) p[(4 * (j >> 2) + (j & 3)) * kDV] = Sacc[ft][vt][8 * m + j];
      }
}
__device__ __forceinline__ void gstate_store(const f32x16 (&Sacc)[3][2], const float* Zg, float* __restrict__ s,
                                             float* __restrict__ zz, int g, int l) {
  gstate_store_s(Sacc, s, g, l);
  for (int m = l; m < 96; m += 64) zz[64 * (m >> 4) + 16 * g + (m & 15)] = Zg[m];
}

// Transposed (token-consecutive) read of the Phi(K) tile for the state update: like lds_tokfrag, but
// lane row r of the 32-row tile receives column col0 + 16 (r / 16) + swz16(r % 16).
__device__ __forceinline__ bf16x8 lds_tokfrag_swz(const __bf16* buf, int pitch, int tok0, int col0, int l) {
  const int b = l >> 4, L = l & 15;
  const int tok = tok0 + 4 * (b >> 1) + (L >> 2);
  const int g4 = L & 3, sg = ((g4 & 1) << 1) | (g4 >> 1);
  const int col = col0 + 16 * (b & 1) + 4 * sg;
  const u32x2 lo =
      __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + tok * pitch + col)));
  const u32x2 hi = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + (tok + 8) * pitch + col)));
  const u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// Featurize 8 consecutive dims of one token: channels 1..5 as MFMA operand fragments (slot i = dim i),
// and the fp32 cos, sin, r.
__device__ __forceinline__ void feat8(const bf16x8& u, const float4& rh0, const float4& rh1, const float (&om4)[8],
                                      float kr, bf16x8 (&F)[5], float (&cr)[8], float (&sr)[8], float (&rr)[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float rho = i < 4 ? rh0[i] : rh1[i - 4];
    featurize1((float)u[i], rho, om4[i], kr, cr[i], sr[i], rr[i]);
  }
  u32x4 w[5];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int a = 2 * j, b = 2 * j + 1;
    w[0][j] = pack_bf16x2(cr[a], cr[b]);
    w[1][j] = pack_bf16x2(sr[a], sr[b]);
    w[2][j] = pack_bf16x2(rr[a], rr[b]);
    w[3][j] = pack_bf16x2(rr[a] * cr[a], rr[b] * cr[b]);
    w[4][j] = pack_bf16x2(rr[a] * sr[a], rr[b] * sr[b]);
  }
#pragma unroll
  for (int c = 0; c < 5; c++) F[c] = __builtin_bit_cast(bf16x8, w[c]);
}

template <int CH, bool STATE_ONLY, bool RAGGED>
__global__ __launch_bounds__(256, 1) void prefill_grp_kernel(const PrefillArgs args) {
  using G = GeomG<CH>;
  constexpr int TB = G::TB, CT = G::CT, KP = G::KP, VP = G::VP, RP = G::RP;
  // V pieces (16 bytes) per lane: pass 1 loads its private tile, pass 3 a quarter of the shared one
  constexpr int NV = STATE_ONLY ? CT / 8 : CT / 32;
  constexpr int VROW0 = STATE_ONLY ? 0 : CT / 4;  // pass 3: wave g writes rows g * CT/4 ..
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, grp = tid >> 6, l = tid & 63, h = l >> 5, n32 = l & 31;
  __bf16* KS = reinterpret_cast<__bf16*>(smem + grp * G::ks_bytes);
  __bf16* Vbase = reinterpret_cast<__bf16*>(smem + G::vs_off);
  float* red = reinterpret_cast<float*>(smem + G::red_off);
  float* Zg = reinterpret_cast<float*>(smem + G::main_bytes(STATE_ONLY)) + grp * 96;
  __bf16* Zb = reinterpret_cast<__bf16*>(smem + G::main_bytes(STATE_ONLY) + 4 * 96 * 4) + grp * 96;
  const int dbase = 16 * grp + 8 * h;
  const u32x4 ones4 = {kOnes2, kOnes2, kOnes2, kOnes2};
  const bf16x8 ONES = __builtin_bit_cast(bf16x8, ones4);
  // the V tile of chunk number j of a piece (pass 3: shared double buffer; pass 1: private)
  auto vtile = [&](int j) -> __bf16* {
    return STATE_ONLY ? Vbase + grp * CT * VP : Vbase + (j & 1) * CT * VP;
  };

  const long long total = call_chunks<RAGGED>(args);
  const int g = range_of_block(args);
  const long long hi_c = range_lo(g + 1, total, args.G);
  for (long long c = range_lo(g, total, args.G); c < hi_c;) {
    const SeqSpan sp = seq_span<RAGGED>(c, args);
    if (RAGGED && sp.bh < 0) break;
    const int bh = sp.bh;
    const long long seq_c0 = sp.c0;
    const long long seq_end = sp.c1;
    const long long pend = hi_c < seq_end ? hi_c : seq_end;
    const bool last_piece = (pend == seq_end);
    const int t_begin = (int)(c - seq_c0) * CH;
    const int t_end = min(sp.len, (int)(pend - seq_c0) * CH);
    c = pend;
    if (STATE_ONLY && last_piece) continue;
    const int hh = bh % args.H;
    const __bf16* __restrict__ kp = static_cast<const __bf16*>(args.k) + (size_t)bh * args.T * kD;
    const __bf16* __restrict__ qp = static_cast<const __bf16*>(args.q) + (size_t)bh * args.T * kD;
    const __bf16* __restrict__ vp = static_cast<const __bf16*>(args.v) + (size_t)bh * args.T * kDV;
    __bf16* __restrict__ op = static_cast<__bf16*>(args.out) + (size_t)bh * args.T * kDV;
    float* slot = args.ws_state + (size_t)(bh + g) * kStateFloats;

    float om4[8];
#pragma unroll
    for (int i = 0; i < 8; i++) om4[i] = anchor_rev(args.omega[(size_t)(hh % args.nph) * kD + dbase + i]);

    // ---- initial state of the piece
    f32x16 Sacc[3][2];
#pragma unroll
    for (int ft = 0; ft < 3; ft++)
#pragma unroll
      for (int vt = 0; vt < 2; vt++) zero16(Sacc[ft][vt]);
    for (int m = l; m < 96; m += 64) Zg[m] = 0.0f;
    if (!STATE_ONLY) {
      auto add_slot = [&](const float* s, const float* zz) { gstate_add(Sacc, Zg, s, zz, grp, l); };
      if (args.multi && args.scanned) {
        // (a ragged call's scan leaves the head piece's slot unwritten when there is no caller state)
        if (!RAGGED || args.S || g != range_of_chunk(seq_c0, total, args.G)) add_slot(slot, slot + kF * kDV);
      } else {
        if (args.S) add_slot(args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF);
        if (!RAGGED && args.multi) {  // (a uniform plan has no empty ranges: every slot gf..g-1 was written)
          const int gf = range_of_chunk(seq_c0, total, args.G);
          for (int gg = gf; gg < g; gg++) {
            const float* sj = args.ws_state + (size_t)(bh + gg) * kStateFloats;
            add_slot(sj, sj + kF * kDV);
          }
        }
      }
    }
    __syncthreads();  // the previous piece's tiles are dead (Zg is private to the wave)
    if (!STATE_ONLY)
      for (int m = l; m < 96; m += 64) Zb[m] = (__bf16)Zg[m];

    // ---- raw inputs of one chunk: this lane's rows and phases, its pieces of V
    bf16x8 uk[TB], uq[TB];
    float4 rh[TB][2];
    uint4 rv[NV];
    float4 rh2[TB][2];  // pass 3: phases of the chunk after next, while rh still serves the queries
    auto load_k = [&](int t0, float4 (&ph)[TB][2]) {
      const int nv = min(CH, t_end - t0);
#pragma unroll
      for (int b = 0; b < TB; b++) {
        const int tc = t0 + min(32 * b + n32, nv - 1);
        uk[b] = *reinterpret_cast<const bf16x8*>(kp + (size_t)tc * kD + dbase);
        const float* pr = args.rho + (size_t)tc * kD + dbase;
        ph[b][0] = *reinterpret_cast<const float4*>(pr);
        ph[b][1] = *reinterpret_cast<const float4*>(pr + 4);
      }
    };
    auto load_q = [&](int t0) {
      const int nv = min(CH, t_end - t0);
#pragma unroll
      for (int b = 0; b < TB; b++) {
        const int tc = t0 + min(32 * b + n32, nv - 1);
        uq[b] = *reinterpret_cast<const bf16x8*>(qp + (size_t)tc * kD + dbase);
      }
    };
    auto load_v = [&](int t0) {
      const int nv = min(CH, t_end - t0);
#pragma unroll
      for (int j = 0; j < NV; j++) {
        const int e = l + 64 * j, row = grp * VROW0 + (e >> 3), col = 8 * (e & 7);
        rv[j] = *reinterpret_cast<const uint4*>(vp + (size_t)(t0 + min(row, nv - 1)) * kDV + col);
      }
    };
    // Same order as the loop's own batch (V, keys and phases, queries): the compiler's wait at the loop
    // head must cover both paths, and a different order here would make it wait for everything.
    auto load_raw = [&](int t0) {
      load_v(t0);
      load_k(t0, rh);
      if (!STATE_ONLY) load_q(t0);
    };
    // this lane's pieces of V into a tile; rows past the chunk's end are zero
    auto write_v = [&](__bf16* vt_, int nvalid) {
#pragma unroll
      for (int j = 0; j < NV; j++) {
        const int e = l + 64 * j, row = grp * VROW0 + (e >> 3), col = 8 * (e & 7);
        const unsigned m = 0u - (unsigned)(row < nvalid);
        *reinterpret_cast<uint4*>(vt_ + row * VP + col) =
            make_uint4(rv[j].x & m, rv[j].y & m, rv[j].z & m, rv[j].w & m);
      }
    };
    bf16x8 KF[TB][5], QF[TB][5];
    float dz[TB];
    // Phi(K) rows to the wave's tile (channel 0 = ones); rows past the chunk's end (a ragged last chunk,
    // or the upper half of the tile for chunk 16) are zeroed so that they reach neither z nor S.
    auto write_k = [&](int nvalid) {
#pragma unroll
      for (int b = 0; b < TB; b++) {
        __bf16* row = KS + (32 * b + n32) * KP + 8 * h;
        *reinterpret_cast<u32x4*>(row) = ones4;
#pragma unroll
        for (int cc = 1; cc < 6; cc++) *reinterpret_cast<bf16x8*>(row + 16 * cc) = KF[b][cc - 1];
      }
    };
    auto zero_k_tail = [&](int nvalid) {
#pragma unroll
      for (int b = 0; b < TB; b++) {
        if (32 * b + n32 >= nvalid) {
          __bf16* row = KS + (32 * b + n32) * KP + 8 * h;
#pragma unroll
          for (int cc = 0; cc < 6; cc++) *reinterpret_cast<u32x4*>(row + 16 * cc) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto feat_q = [&]() {  // queries of the loaded chunk + their readout part of the denominator (z as it is)
#pragma unroll
      for (int b = 0; b < TB; b++) {
        float cr[8], sr[8], rr[8];
        feat8(uq[b], rh[b][0], rh[b][1], om4, args.kr, QF[b], cr, sr, rr);
      }
      // Phi(q) . z over the lane's 8 dims: channel 0 (the constant 1) in fp32, channels 1..5 as bf16
      // products like the rest of the readout
      const float4 z0a = *reinterpret_cast<const float4*>(Zg + 8 * h);
      const float4 z0b = *reinterpret_cast<const float4*>(Zg + 8 * h + 4);
      const float z0 = ((z0a.x + z0a.y) + (z0a.z + z0a.w)) + ((z0b.x + z0b.y) + (z0b.z + z0b.w));
      bf16x8 zb[5];
#pragma unroll
      for (int cc = 0; cc < 5; cc++) zb[cc] = *reinterpret_cast<const bf16x8*>(Zb + 16 * (cc + 1) + 8 * h);
#pragma unroll
      for (int b = 0; b < TB; b++) {
        float d = z0;
#pragma unroll
        for (int cc = 0; cc < 5; cc++) d = frag_dot(QF[b][cc], zb[cc], d);
        dz[b] = xor32_sum(d);
      }
    };
    auto feat_k = [&]() {
#pragma unroll
      for (int b = 0; b < TB; b++) {
        float cr[8], sr[8], rr[8];
        feat8(uk[b], rh[b][0], rh[b][1], om4, args.kr, KF[b], cr, sr, rr);
      }
    };

    // o = num / (den + c eps) for one chunk from the four groups' partials in the reduction buffer
    auto normalise = [&](int tc0, int nv) {
      constexpr int TPT = 256 / CT, NC = 64 / TPT;
      const int t = tid / TPT, c0 = NC * (tid % TPT);
      if (t < nv) {
        const float* b0 = red + ((t >> 5) * 4 * 32 + (t & 31)) * RP;
        constexpr int GS = 32 * RP;
        const float den = ((b0[64] + b0[GS + 64]) + b0[2 * GS + 64]) + b0[3 * GS + 64];
        const float inv = 1.0f / (den + args.ceps);
#pragma unroll
        for (int q4 = 0; q4 < NC / 8; q4++) {
          u32x4 w;
#pragma unroll
          for (int half = 0; half < 2; half++) {
            const int cb = c0 + 8 * q4 + 4 * half;
            const float4 a0 = *reinterpret_cast<const float4*>(b0 + cb);
            const float4 a1 = *reinterpret_cast<const float4*>(b0 + GS + cb);
            const float4 a2 = *reinterpret_cast<const float4*>(b0 + 2 * GS + cb);
            const float4 a3 = *reinterpret_cast<const float4*>(b0 + 3 * GS + cb);
            w[2 * half] = pack_bf16x2((((a0.x + a1.x) + a2.x) + a3.x) * inv, (((a0.y + a1.y) + a2.y) + a3.y) * inv);
            w[2 * half + 1] =
                pack_bf16x2((((a0.z + a1.z) + a2.z) + a3.z) * inv, (((a0.w + a1.w) + a2.w) + a3.w) * inv);
          }
          *reinterpret_cast<u32x4*>(op + (size_t)(tc0 + t) * kDV + c0 + 8 * q4) = w;
        }
      }
    };

    // ---- prologue: chunk 0 featurized, its Phi(K) and V in LDS; raw inputs of chunk 1 in registers
    {
      load_raw(t_begin);
      const int nv0 = min(CH, t_end - t_begin);
      feat_k();
      write_k(nv0);
      if (nv0 < CT) zero_k_tail(nv0);
      if (!STATE_ONLY) feat_q();
      write_v(vtile(0), nv0);
      load_raw(t_begin + CH < t_end ? t_begin + CH : t_begin);
    }

    int j = 0;
    for (int t0 = t_begin; t0 < t_end; t0 += CH, j++) {
      const int nvalid = min(CH, t_end - t0);
      const bool more = t0 + CH < t_end;
      const int nvalid1 = more ? min(CH, t_end - t0 - CH) : CT;
      const __bf16* Vs = vtile(j);
      const int t2 = t0 + 2 * CH < t_end ? t0 + 2 * CH : t0;
      if constexpr (STATE_ONLY) {
        // Pass 1: S += Phi(K)^T V for this chunk, with the next chunk's keys featurized in between the
        // update MFMAs (scheduling fences keep the two streams interleaved), LDS fragments read one
        // K-step ahead, and the raw inputs of the chunk after next loaded a full iteration ahead.
        bf16x8 uk2[TB];
        float4 rhn[TB][2];
#pragma unroll
        for (int b = 0; b < TB; b++) {
          const int nv = min(CH, t_end - t2);
          const int tc = t2 + min(32 * b + n32, nv - 1);
          uk2[b] = *reinterpret_cast<const bf16x8*>(kp + (size_t)tc * kD + dbase);
          const float* pr = args.rho + (size_t)tc * kD + dbase;
          rhn[b][0] = *reinterpret_cast<const float4*>(pr);
          rhn[b][1] = *reinterpret_cast<const float4*>(pr + 4);
        }
        float cr[TB][8], sr[TB][8], rr[TB][8];
        auto fe = [&](int e) {
          const int b = e >> 3, i = e & 7;
          const float rho = i < 4 ? rh[b][0][i] : rh[b][1][i - 4];
          featurize1((float)uk[b][i], rho, om4[i], args.kr, cr[b][i], sr[b][i], rr[b][i]);
        };
        bf16x8 Af[2][3], Bf[2][2];
        auto ldf = [&](int ks, int buf) {
          Bf[buf][0] = lds_tokfrag(Vs, VP, 16 * ks, 0, l);
          Bf[buf][1] = lds_tokfrag(Vs, VP, 16 * ks, 32, l);
#pragma unroll
          for (int ft = 0; ft < 3; ft++) Af[buf][ft] = lds_tokfrag_swz(KS, KP, 16 * ks, 32 * ft, l);
        };
        constexpr int NE = 8 * TB;  // components to featurize, spread over the 2 TB K-steps
        float zs[3] = {0.0f, 0.0f, 0.0f};
        ldf(0, 0);
#pragma unroll
        for (int ks = 0; ks < 2 * TB; ks++) {
          if (ks + 1 < 2 * TB) ldf(ks + 1, (ks + 1) & 1);
#pragma unroll
          for (int ft = 0; ft < 3; ft++) {
            mma32(Sacc[ft][0], Af[ks & 1][ft], Bf[ks & 1][0]);
            mma32(Sacc[ft][1], Af[ks & 1][ft], Bf[ks & 1][1]);
            zs[ft] = frag_sum(Af[ks & 1][ft], zs[ft]);
          }
#pragma unroll
          for (int e = ks * NE / (2 * TB); e < (ks + 1) * NE / (2 * TB); e++) fe(e);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int b = 0; b < TB; b++) {
          u32x4 w[5];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int a = 2 * q, c = 2 * q + 1;
            w[0][q] = pack_bf16x2(cr[b][a], cr[b][c]);
            w[1][q] = pack_bf16x2(sr[b][a], sr[b][c]);
            w[2][q] = pack_bf16x2(rr[b][a], rr[b][c]);
            w[3][q] = pack_bf16x2(rr[b][a] * cr[b][a], rr[b][c] * cr[b][c]);
            w[4][q] = pack_bf16x2(rr[b][a] * sr[b][a], rr[b][c] * sr[b][c]);
          }
#pragma unroll
          for (int cc = 0; cc < 5; cc++) KF[b][cc] = __builtin_bit_cast(bf16x8, w[cc]);
        }
#pragma unroll
        for (int ft = 0; ft < 3; ft++) {
          const float zf = xor32_sum(zs[ft]);
          float* zp = Zg + 32 * ft + 16 * (n32 >> 4) + swz16(n32 & 15);
          const float znew = *zp + zf;
          *zp = znew;  // both halves store the same value
        }
        write_k(nvalid1);
        write_v(vtile(j + 1), nvalid1);
        load_v(t2);
#pragma unroll
        for (int b = 0; b < TB; b++) {
          uk[b] = uk2[b];
          rh[b][0] = rhn[b][0];
          rh[b][1] = rhn[b][1];
        }
        if (nvalid1 < CT) zero_k_tail(nvalid1);
        continue;
      }
      // the previous chunk's partial numerators and this chunk's V tile are complete; the previous chunk
      // is normalised and stored here (its stores then have a whole iteration to drain), and the second
      // barrier frees the reduction buffer for this chunk
      __syncthreads();
      if (t0 > t_begin) normalise(t0 - CH, CH);
      __syncthreads();

      // keys of the next chunk (registers only; the tile is rewritten at the end of the iteration); the
      // registers consumed here are refilled at once with the chunk after next
      feat_k();
      // one batch of loads for the chunk after next, a full iteration before its use, into second
      // register sets (V and the queries of the next chunk are consumed at the end of this iteration)
      bf16x8 uq2[TB];
      uint4 rvn[NV];
#pragma unroll
      for (int jj = 0; jj < NV; jj++) {
        const int nv = min(CH, t_end - t2);
        const int e = l + 64 * jj, row = grp * VROW0 + (e >> 3), col = 8 * (e & 7);
        rvn[jj] = *reinterpret_cast<const uint4*>(vp + (size_t)(t2 + min(row, nv - 1)) * kDV + col);
      }
      load_k(t2, rh2);
#pragma unroll
      for (int b = 0; b < TB; b++) {
        const int nv = min(CH, t_end - t2);
        const int tc = t2 + min(32 * b + n32, nv - 1);
        uq2[b] = *reinterpret_cast<const bf16x8*>(qp + (size_t)tc * kD + dbase);
      }

      if (!STATE_ONLY) {
        // intra-chunk tiles A^T[s][t] = Phi(k_s) . Phi(q_t), masked to s <= t, rounded to bf16; Phi(k)
        // from this lane's own rows of the LDS tile, Phi(q) from registers
        bf16x8 P[TB][TB][2];
        float rs[TB];
#pragma unroll
        for (int tb = 0; tb < TB; tb++) {
          rs[tb] = 0.0f;
#pragma unroll
          for (int sb = 0; sb <= tb; sb++) {
            // channel 0: sixteen products 1 * 1 in every entry, from one MFMA on the ones fragment
            f32x16 at;
            zero16(at);
            mma32(at, ONES, ONES);
            const __bf16* krow = KS + (32 * sb + n32) * KP + 8 * h;
#pragma unroll
            for (int cc = 0; cc < 5; cc++)
              mma32(at, *reinterpret_cast<const bf16x8*>(krow + 16 * (cc + 1)), QF[tb][cc]);
            float lo[8], hi8[8];
#pragma unroll
            for (int i = 0; i < 16; i++) {
              const int sl = 8 * (i >> 2) + 4 * h + (i & 3);
              const float a = (sb == tb && sl > n32) ? 0.0f : at[i];
              if (i < 8) lo[i] = a;
              else hi8[i - 8] = a;
            }
            u32x4 w0, w1;
#pragma unroll
            for (int q = 0; q < 4; q++) {
              w0[q] = pack_bf16x2(lo[2 * q], lo[2 * q + 1]);
              w1[q] = pack_bf16x2(hi8[2 * q], hi8[2 * q + 1]);
            }
            P[tb][sb][0] = __builtin_bit_cast(bf16x8, w0);
            P[tb][sb][1] = __builtin_bit_cast(bf16x8, w1);
            rs[tb] = frag_sum(P[tb][sb][1], frag_sum(P[tb][sb][0], rs[tb]));
          }
        }
        // numerators: V^T P (intra) + S^T Phi(q) (readout, S from before this chunk), written straight to
        // the reduction buffer; each S^T operand is packed once and used for every token block
#pragma unroll
        for (int vt = 0; vt < 2; vt++) {
          f32x16 num[TB];
#pragma unroll
          for (int tb = 0; tb < TB; tb++) {
            zero16(num[tb]);
#pragma unroll
            for (int sb = 0; sb <= tb; sb++) {
              mma32(num[tb], lds_tokfrag(Vs, VP, 32 * sb, 32 * vt, l), P[tb][sb][0]);
              mma32(num[tb], lds_tokfrag(Vs, VP, 32 * sb + 16, 32 * vt, l), P[tb][sb][1]);
            }
          }
#pragma unroll
          for (int cc = 0; cc < 6; cc++) {
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; q++)
              w[q] = pack_bf16x2(Sacc[cc >> 1][vt][8 * (cc & 1) + 2 * q], Sacc[cc >> 1][vt][8 * (cc & 1) + 2 * q + 1]);
            const bf16x8 sa = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int tb = 0; tb < TB; tb++) mma32(num[tb], sa, cc == 0 ? ONES : QF[tb][cc - 1]);
          }
#pragma unroll
          for (int tb = 0; tb < TB; tb++) {
            float* rrow = red + ((tb * 4 + grp) * 32 + n32) * RP;
#pragma unroll
            for (int q = 0; q < 4; q++)
              *reinterpret_cast<float4*>(rrow + 32 * vt + 8 * q + 4 * h) =
                  make_float4(num[tb][4 * q], num[tb][4 * q + 1], num[tb][4 * q + 2], num[tb][4 * q + 3]);
          }
        }
#pragma unroll
        for (int tb = 0; tb < TB; tb++) {
          const float rsf = xor32_sum(rs[tb]);
          red[((tb * 4 + grp) * 32 + n32) * RP + 64] = rsf + dz[tb];  // both halves store the same value
        }
      }

      // state update S += Phi(K)^T V, z += Phi(K)^T 1 for the wave's group
      float zs[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 2 * TB; ks++) {
        const bf16x8 B0 = lds_tokfrag(Vs, VP, 16 * ks, 0, l);
        const bf16x8 B1 = lds_tokfrag(Vs, VP, 16 * ks, 32, l);
#pragma unroll
        for (int ft = 0; ft < 3; ft++) {
          const bf16x8 A = lds_tokfrag_swz(KS, KP, 16 * ks, 32 * ft, l);
          zs[ft] = frag_sum(A, zs[ft]);
          mma32(Sacc[ft][0], A, B0);
          mma32(Sacc[ft][1], A, B1);
        }
      }
#pragma unroll
      for (int ft = 0; ft < 3; ft++) {
        const float zf = xor32_sum(zs[ft]);
        float* zp = Zg + 32 * ft + 16 * (n32 >> 4) + swz16(n32 & 15);
        const float znew = *zp + zf;
        *zp = znew;  // both halves store the same value
        if (!STATE_ONLY) Zb[zp - Zg] = (__bf16)znew;
      }

      // next chunk: queries (denominator part with the updated z), Phi(K) and V tiles, raw loads
      if (!STATE_ONLY) {
        feat_q();
        write_v(vtile(j + 1), nvalid1);  // the other V buffer is no longer read by anyone
#pragma unroll
        for (int b = 0; b < TB; b++) {
          uq[b] = uq2[b];
          rh[b][0] = rh2[b][0];
          rh[b][1] = rh2[b][1];
        }
#pragma unroll
        for (int jj = 0; jj < NV; jj++) rv[jj] = rvn[jj];
      }
      write_k(nvalid1);
      if (nvalid1 < CT) zero_k_tail(nvalid1);
    }
    if (!STATE_ONLY) {
      __syncthreads();  // the last chunk's partial numerators and denominators are in
      const int t_last = t_end - 1 - (t_end - 1 - t_begin) % CH;
      normalise(t_last, t_end - t_last);
    }

    float* dst_s = STATE_ONLY ? slot : (last_piece && args.S ? args.S + (size_t)bh * kF * kDV : nullptr);
    float* dst_z = STATE_ONLY ? slot + kF * kDV : (last_piece && args.S ? args.z + (size_t)bh * kF : nullptr);
    if (dst_s) gstate_store(Sacc, Zg, dst_s, dst_z, grp, l);
  }
}

// Pass 1 for chunk 64 with the two 32-token halves of every chunk on different waves: wave 4 s + g
// accumulates the feature-group-g increment of S and z over tokens 32 s .. 32 s + 31 of each chunk of
// the piece, so that two waves share each SIMD.  Every wave's Phi(K) and V tiles are private, so the
// chunk loop has no barrier; the two halves of a group meet at the end of the piece (the sum is over
// tokens, so splitting it changes nothing but the rounding order).
//
// Per chunk j a wave reads all of its tile's MFMA operands into registers first, then overwrites the
// tile with chunk j + 1 (featurized during the previous chunk), then runs the update MFMAs with the keys
// of chunk j + 2 featurized in between.  A tile write and the next read of that tile are a whole chunk
// apart, so neither waits on the other.
struct GeomS8 {
  static constexpr int CT = 32, KP = 104, VP = 72;
  static constexpr int ks_bytes = CT * KP * 2;
  static constexpr int vs_bytes = CT * VP * 2;
  static constexpr int vs_off = 8 * ks_bytes;
  // at the end of a piece the second-half waves pass their state slices to the first-half waves through
  // a staging area that aliases the tiles: [group][register / 4][lane][4] floats, then z as [group][96]
  static constexpr int stage_bytes = 4 * 96 * 64 * 4 + 4 * 96 * 4;
  static constexpr int tiles_bytes = vs_off + 8 * vs_bytes;
  static constexpr int lds = tiles_bytes > stage_bytes ? tiles_bytes : stage_bytes;
};

// PCH is the chunk of the call (64 or 128), which fixes the pieces; the increment over a piece does
// not depend on the chunking, so the loop always steps 64 tokens.
template <int PCH, bool RAGGED>
__global__ __launch_bounds__(512, 1) void prefill_state8_kernel(const PrefillArgs args) {
  constexpr int CH = 64, KP = GeomS8::KP, VP = GeomS8::VP;
  static_assert(PCH % CH == 0, "pieces are whole 64-token steps");
  constexpr int NV = GeomS8::CT / 8;  // 16-byte pieces of the wave's V rows per lane
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, w = tid >> 6, grp = w & 3, half = w >> 2, l = tid & 63, h = l >> 5, n32 = l & 31;
  __bf16* KS = reinterpret_cast<__bf16*>(smem + w * GeomS8::ks_bytes);
  __bf16* Vs = reinterpret_cast<__bf16*>(smem + GeomS8::vs_off + w * GeomS8::vs_bytes);
  const int dbase = 16 * grp + 8 * h;
  const int toff = 32 * half;  // this wave's token offset inside a chunk
  const u32x4 ones4 = {kOnes2, kOnes2, kOnes2, kOnes2};

  const long long total = call_chunks<RAGGED>(args);
  const int g = range_of_block(args);
  const long long hi_c = range_lo(g + 1, total, args.G);
  for (long long c = range_lo(g, total, args.G); c < hi_c;) {
    const SeqSpan sp = seq_span<RAGGED>(c, args);
    if (RAGGED && sp.bh < 0) break;
    const int bh = sp.bh;
    const long long seq_c0 = sp.c0;
    const long long seq_end = sp.c1;
    const long long pend = hi_c < seq_end ? hi_c : seq_end;
    const bool last_piece = (pend == seq_end);
    const int t_begin = (int)(c - seq_c0) * PCH;
    const int t_end = min(sp.len, (int)(pend - seq_c0) * PCH);
    c = pend;
    if (last_piece) continue;  // the final piece's state comes out of pass 3
    const int hh = bh % args.H;
    const __bf16* __restrict__ kp = static_cast<const __bf16*>(args.k) + (size_t)bh * args.T * kD;
    const __bf16* __restrict__ vp = static_cast<const __bf16*>(args.v) + (size_t)bh * args.T * kDV;
    float* slot = args.ws_state + (size_t)(bh + g) * kStateFloats;

    float om4[8];
#pragma unroll
    for (int i = 0; i < 8; i++) om4[i] = anchor_rev(args.omega[(size_t)(hh % args.nph) * kD + dbase + i]);

    f32x16 Sacc[3][2];
#pragma unroll
    for (int ft = 0; ft < 3; ft++)
#pragma unroll
      for (int vt = 0; vt < 2; vt++) zero16(Sacc[ft][vt]);
    // z of feature 32 ft + n32 of the group's tile order (both lane halves hold the same value)
    float zacc[3] = {0.0f, 0.0f, 0.0f};

    // Raw inputs of one 64-token step (start t0; a step past the piece's end re-reads the last one): this
    // lane's key row and phases (token toff + n32), its pieces of the wave's V rows.  A piece handled here
    // is not its sequence's last, so it starts and ends on chunk boundaries strictly inside the sequence:
    // every step is whole.  The loads are buffer loads over the sequence (and the phase table), with the
    // lane's offset inside a step fixed and the step's start as the scalar offset, so a step costs no
    // address arithmetic; the descriptors' range check would return zeros past the sequence's end.
    auto next_t = [&](int t0) { return t0 + CH < t_end ? t0 + CH : t0; };
    constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw-buffer format
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, args.T * kD * 2, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, args.T * kDV * 2, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc((void*)args.rho, (short)0, args.T * kD * 4, kRawBufferWord3);
    const unsigned koff = (unsigned)(((toff + n32) * kD + dbase) * 2);
    const unsigned poff = (unsigned)(((toff + n32) * kD + dbase) * 4);
    auto load_k = [&](int t0, bf16x8& u, float4 (&ph)[2]) {
      u = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, koff, t0 * kD * 2, 0));
      ph[0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prs, poff, t0 * kD * 4, 0));
      ph[1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prs, poff + 16, t0 * kD * 4, 0));
    };
    auto load_v = [&](int t0, uint4 (&r)[NV]) {
#pragma unroll
      for (int j = 0; j < NV; j++) {
        const int e = l + 64 * j, row = e >> 3, col = 8 * (e & 7);
        r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             vrs, (unsigned)(((toff + row) * kDV + col) * 2), t0 * kDV * 2, 0));
      }
    };
    auto half_valid = [&](int t0) { return max(0, min(CH, t_end - t0) - toff); };
    // the wave's rows of V and Phi(K) into its tiles; rows past the chunk's end are zero
    // (a full half, the common case, takes the unmasked branch; nvh is the same on every lane)
    auto write_v = [&](const uint4 (&r)[NV], int nvh) {
#pragma unroll
      for (int j = 0; j < NV; j++) {
        const int e = l + 64 * j, row = e >> 3, col = 8 * (e & 7);
        const unsigned m = 0u - (unsigned)(row < nvh);
        *reinterpret_cast<uint4*>(Vs + row * VP + col) = make_uint4(r[j].x & m, r[j].y & m, r[j].z & m, r[j].w & m);
      }
    };
    // (channel 0, the constant 1, is written with the piece's first chunk only: the loop writes whole
    // chunks, so nothing overwrites it before the staging at the piece's end)
    auto write_k = [&](const bf16x8 (&F)[5], int nvh, bool ones) {
      __bf16* row = KS + n32 * KP + 8 * h;
      if (n32 < nvh) {
        if (ones) *reinterpret_cast<u32x4*>(row) = ones4;
#pragma unroll
        for (int cc = 1; cc < 6; cc++) *reinterpret_cast<bf16x8*>(row + 16 * cc) = F[cc - 1];
      } else {
#pragma unroll
        for (int cc = 0; cc < 6; cc++) *reinterpret_cast<u32x4*>(row + 16 * cc) = u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto pack = [&](const float (&cr)[8], const float (&sr)[8], const float (&rr)[8], bf16x8 (&F)[5]) {
      u32x4 wv[5];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int a = 2 * q, b = 2 * q + 1;
        wv[0][q] = pack_bf16x2(cr[a], cr[b]);
        wv[1][q] = pack_bf16x2(sr[a], sr[b]);
        wv[2][q] = pack_bf16x2(rr[a], rr[b]);
        wv[3][q] = pack_bf16x2(rr[a] * cr[a], rr[b] * cr[b]);
        wv[4][q] = pack_bf16x2(rr[a] * sr[a], rr[b] * sr[b]);
      }
#pragma unroll
      for (int cc = 0; cc < 5; cc++) F[cc] = __builtin_bit_cast(bf16x8, wv[cc]);
    };

    // prologue: chunk 0 in the tiles; V rows and raw keys of chunk 1 in flight (set A)
    bf16x8 uk;
    float4 rh[2];
    uint4 rv[NV];
    {
      load_v(t_begin, rv);
      load_k(t_begin, uk, rh);
      bf16x8 F[5];
      float cr[8], sr[8], rr[8];
      feat8(uk, rh[0], rh[1], om4, args.kr, F, cr, sr, rr);
      const int nvh = half_valid(t_begin);
      write_k(F, nvh, true);
      write_v(rv, nvh);
      // V before keys, as in the loop, so that the loop's first wait for V does not also wait for the keys
      const int t1 = next_t(t_begin);
      load_v(t1, rv);
      __builtin_amdgcn_sched_barrier(0);
      load_k(t1, uk, rh);
    }

    // The loop over chunks j: rv and (uk, rh) hold chunk j + 1's V rows and raw keys, loaded during chunk
    // j - 1.  After the MFMA operands of chunk j are read out of the tiles, chunk j + 1's V rows overwrite the
    // V tile and its keys, featurized between the update MFMAs, overwrite the Phi(K) tile (LDS serves the
    // wave in order, so the reads see chunk j).  Each register set is reloaded with chunk j + 2 as soon as it
    // has been consumed, so no copy closes the loop (a copy would wait for loads issued in the same chunk),
    // and the V rows are waited for only in the next chunk's step 2, the keys in its step 4.
    for (int t0 = t_begin; t0 < t_end; t0 += CH) {
      const int ta = next_t(t0), tb = next_t(ta);  // chunks j + 1, j + 2
      const int nvh1 = ta != t0 ? half_valid(ta) : 0;  // 0: no next chunk, the tiles are not written again
      // 1. every MFMA operand of chunk j out of the tiles
      bf16x8 Af[2][3], Bf[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        Bf[ks][0] = lds_tokfrag(Vs, VP, 16 * ks, 0, l);
        Bf[ks][1] = lds_tokfrag(Vs, VP, 16 * ks, 32, l);
#pragma unroll
        for (int ft = 0; ft < 3; ft++) Af[ks][ft] = lds_tokfrag_swz(KS, KP, 16 * ks, 32 * ft, l);
      }
      // 2. chunk j + 1's V rows into the V tile, 3. and chunk j + 2's into their registers
      if (nvh1 > 0) write_v(rv, nvh1);
      load_v(tb, rv);
      // 4. the update MFMAs of chunk j with the keys of chunk j + 1 featurized in between, then into the tile
      float cr[8], sr[8], rr[8];
      float zs[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
#pragma unroll
        for (int ft = 0; ft < 3; ft++) {
          mma32(Sacc[ft][0], Af[ks][ft], Bf[ks][0]);
          mma32(Sacc[ft][1], Af[ks][ft], Bf[ks][1]);
          zs[ft] = frag_sum(Af[ks][ft], zs[ft]);
        }
#pragma unroll
        for (int i = 4 * ks; i < 4 * ks + 4; i++) {
          const float rho = i < 4 ? rh[0][i] : rh[1][i - 4];
          featurize1((float)uk[i], rho, om4[i], args.kr, cr[i], sr[i], rr[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 F[5];
      pack(cr, sr, rr, F);
      if (nvh1 > 0) write_k(F, nvh1, false);
#pragma unroll
      for (int ft = 0; ft < 3; ft++) zacc[ft] += xor32_sum(zs[ft]);
      // 5. chunk j + 2's keys into the registers just read
      __builtin_amdgcn_sched_barrier(0);
      load_k(tb, uk, rh);
    }

    // the two halves of each group meet: the second-half waves hand their slices over through LDS, the
    // first-half waves add them to their own and store the sum in the slot
    float4* stage = reinterpret_cast<float4*>(smem) + grp * 24 * 64 + l;
    float* zstage = reinterpret_cast<float*>(smem + 4 * 96 * 64 * 4) + grp * 96;
    __syncthreads();  // every wave is done with its tiles
    if (half == 1) {
#pragma unroll
      for (int r4 = 0; r4 < 24; r4++) {
        const int r = 4 * r4, ft = r >> 5, vt = (r >> 4) & 1, i = r & 15;
        stage[64 * r4] = make_float4(Sacc[ft][vt][i], Sacc[ft][vt][i + 1], Sacc[ft][vt][i + 2], Sacc[ft][vt][i + 3]);
      }
      if (h == 0) {
#pragma unroll
        for (int ft = 0; ft < 3; ft++) zstage[32 * ft + n32] = zacc[ft];
      }
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int r4 = 0; r4 < 24; r4++) {
        const int r = 4 * r4, ft = r >> 5, vt = (r >> 4) & 1, i = r & 15;
        const float4 o = stage[64 * r4];
        Sacc[ft][vt][i] += o.x;
        Sacc[ft][vt][i + 1] += o.y;
        Sacc[ft][vt][i + 2] += o.z;
        Sacc[ft][vt][i + 3] += o.w;
      }
      gstate_store_s(Sacc, slot, grp, l);
      // feature 32 ft + n32 of the tile order is channel 2 ft + n32 / 16, dim 16 g + swz16(n32 % 16)
      if (h == 0) {
        float* zz = slot + kF * kDV;
#pragma unroll
        for (int ft = 0; ft < 3; ft++)
          zz[64 * (2 * ft + (n32 >> 4)) + 16 * grp + swz16(n32 & 15)] = zacc[ft] + zstage[32 * ft + n32];
      }
    }
    __syncthreads();  // the staging area is free again before the next piece's tiles are written
  }
}

// ------------------------------------------------------------------------------- chunk 128 (bf16)
// Pass 3 for 128-token chunks with the layout of the kernel above (wave g = feature group g; lane
// (n32, h) featurizes dims 16g + 8h + 0..7 of token n32 of a 32-token block straight into MFMA
// K-slots).  A chunk runs as four 32-token blocks in order.  Block b featurizes its keys (kept in
// registers for the diagonal score tile, and written to the wave's Phi(K) tile for the later blocks and
// the state update) and its queries, then reads out against S as it was at the chunk's start (packed to
// bf16 once per chunk) plus the masked scores of key blocks 0..b.  The four groups' partial numerators
// of a block meet in one reduction buffer.  Raw key, query and phase rows are loaded one block ahead
// and V rows two blocks ahead; the V rows of block b + 1 go to the shared tile while block b runs, so
// block b's barriers publish them.
struct Geom128 {
  static constexpr int CH = 128, TB = 4, KP = 104, VP = 72, RP = 68;
  static constexpr int ks_bytes = CH * KP * 2;  // one wave's Phi(K) tile
  static constexpr int vs_off = 4 * ks_bytes;
  static constexpr int vs_bytes = CH * VP * 2;
  static constexpr int red_off = vs_off + vs_bytes;
  static constexpr int red_bytes = 4 * 32 * RP * 4;  // one query block: [group][32][RP]
  static constexpr int z_off = red_off + red_bytes;
  static constexpr int lds = z_off + 4 * 96 * 4 + 4 * 96 * 2;  // z fp32 and its bf16 copy per wave
};

// one lane's raw key, query and phase values of a token (8 dims)
struct RawKQ {
  bf16x8 k, q;
  float4 r0, r1;
};

template <bool RAGGED>
__global__ __launch_bounds__(256, 1) void prefill_grp128_kernel(const PrefillArgs args) {
  using G = Geom128;
  constexpr int CH = G::CH, TB = G::TB, KP = G::KP, VP = G::VP, RP = G::RP;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, grp = tid >> 6, l = tid & 63, h = l >> 5, n32 = l & 31;
  __bf16* KS = reinterpret_cast<__bf16*>(smem + grp * G::ks_bytes);
  __bf16* Vs = reinterpret_cast<__bf16*>(smem + G::vs_off);
  float* red = reinterpret_cast<float*>(smem + G::red_off);
  float* Zg = reinterpret_cast<float*>(smem + G::z_off) + grp * 96;
  __bf16* Zb = reinterpret_cast<__bf16*>(smem + G::z_off + 4 * 96 * 4) + grp * 96;
  const int dbase = 16 * grp + 8 * h;
  const int vrow = tid >> 3, vcol = 8 * (tid & 7);  // this thread's 16 bytes of a block's V rows
  const u32x4 ones4 = {kOnes2, kOnes2, kOnes2, kOnes2};
  const bf16x8 ONES = __builtin_bit_cast(bf16x8, ones4);

  const long long total = call_chunks<RAGGED>(args);
  const int g = range_of_block(args);
  const long long hi_c = range_lo(g + 1, total, args.G);
  for (long long c = range_lo(g, total, args.G); c < hi_c;) {
    const SeqSpan sp = seq_span<RAGGED>(c, args);
    if (RAGGED && sp.bh < 0) break;
    const int bh = sp.bh;
    const long long seq_c0 = sp.c0;
    const long long seq_end = sp.c1;
    const long long pend = hi_c < seq_end ? hi_c : seq_end;
    const bool last_piece = (pend == seq_end);
    const int t_begin = (int)(c - seq_c0) * CH;
    const int t_end = min(sp.len, (int)(pend - seq_c0) * CH);
    c = pend;
    const int hh = bh % args.H;
    const __bf16* __restrict__ kp = static_cast<const __bf16*>(args.k) + (size_t)bh * args.T * kD;
    const __bf16* __restrict__ qp = static_cast<const __bf16*>(args.q) + (size_t)bh * args.T * kD;
    const __bf16* __restrict__ vp = static_cast<const __bf16*>(args.v) + (size_t)bh * args.T * kDV;
    __bf16* __restrict__ op = static_cast<__bf16*>(args.out) + (size_t)bh * args.T * kDV;
    const float* slot = args.ws_state + (size_t)(bh + g) * kStateFloats;

    float om4[8];
#pragma unroll
    for (int i = 0; i < 8; i++) om4[i] = anchor_rev(args.omega[(size_t)(hh % args.nph) * kD + dbase + i]);

    // ---- state before the piece: the caller's state and the earlier pieces' increments (or their scan)
    f32x16 Sacc[3][2];
#pragma unroll
    for (int ft = 0; ft < 3; ft++)
#pragma unroll
      for (int vt = 0; vt < 2; vt++) zero16(Sacc[ft][vt]);
    for (int m = l; m < 96; m += 64) Zg[m] = 0.0f;
    if (args.multi && args.scanned) {
      // (a ragged call's scan leaves the head piece's slot unwritten when there is no caller state)
      if (!RAGGED || args.S || g != range_of_chunk(seq_c0, total, args.G))
        gstate_add(Sacc, Zg, slot, slot + kF * kDV, grp, l);
    } else {
      if (args.S) gstate_add(Sacc, Zg, args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF, grp, l);
      if (!RAGGED && args.multi) {  // (a uniform plan has no empty ranges: every slot gf..g-1 was written)
        const int gf = range_of_chunk(seq_c0, total, args.G);
        for (int gg = gf; gg < g; gg++) {
          const float* sj = args.ws_state + (size_t)(bh + gg) * kStateFloats;
          gstate_add(Sacc, Zg, sj, sj + kF * kDV, grp, l);
        }
      }
    }
    __syncthreads();  // the previous piece's tiles are dead
    for (int m = l; m < 96; m += 64) Zb[m] = (__bf16)Zg[m];

    // raw rows of block i of the piece (chunk t_begin + 128 (i / 4), tokens 32 (i % 4) ..); indexes past
    // the piece's last block re-read that block, rows past a chunk's end re-read the chunk's last row
    const int nblk = TB * ((t_end - t_begin + CH - 1) / CH);
    auto src_row = [&](int i, int r) {
      const int ib = min(i, nblk - 1);
      const int t0 = t_begin + CH * (ib / TB);
      return t0 + min(32 * (ib % TB) + r, min(CH, t_end - t0) - 1);
    };
    auto load_kq = [&](int i) {
      RawKQ x;
      const int tc = src_row(i, n32);
      x.k = *reinterpret_cast<const bf16x8*>(kp + (size_t)tc * kD + dbase);
      x.q = *reinterpret_cast<const bf16x8*>(qp + (size_t)tc * kD + dbase);
      const float* pr = args.rho + (size_t)tc * kD + dbase;
      x.r0 = *reinterpret_cast<const float4*>(pr);
      x.r1 = *reinterpret_cast<const float4*>(pr + 4);
      return x;
    };
    auto load_v = [&](int i) { return *reinterpret_cast<const uint4*>(vp + (size_t)src_row(i, vrow) * kDV + vcol); };
    // this thread's piece of the V rows of block b of a chunk with nvalid tokens (rows past the end zero)
    auto write_v = [&](int b, int nvalid, const uint4& x) {
      const int row = 32 * b + vrow;
      *reinterpret_cast<uint4*>(Vs + row * VP + vcol) = row < nvalid ? x : make_uint4(0u, 0u, 0u, 0u);
    };

    RawKQ kq = load_kq(0);
    uint4 va = load_v(0), vb = load_v(1);  // V of the next block to publish, and of the one after
    for (int t0 = t_begin, i0 = 0; t0 < t_end; t0 += CH, i0 += TB) {
      const int nvalid = min(CH, t_end - t0);
      write_v(0, nvalid, va);
      __syncthreads();  // V rows of block 0 are in

      // S^T operands of the readout, from the state before this chunk
      bf16x8 SA[2][6];
#pragma unroll
      for (int vt = 0; vt < 2; vt++)
#pragma unroll
        for (int cc = 0; cc < 6; cc++) {
          u32x4 w;
#pragma unroll
          for (int q = 0; q < 4; q++)
            w[q] = pack_bf16x2(Sacc[cc >> 1][vt][8 * (cc & 1) + 2 * q], Sacc[cc >> 1][vt][8 * (cc & 1) + 2 * q + 1]);
          SA[vt][cc] = __builtin_bit_cast(bf16x8, w);
        }

#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        const RawKQ kqn = load_kq(i0 + tb + 1);
        const uint4 vn = load_v(i0 + tb + 2);
        // keys of this block: features in registers, and rows of the wave's Phi(K) tile (ones, then
        // channels 1..5; zero rows past the chunk's end, so they reach neither S nor z)
        bf16x8 KF[5], QF[5];
        float dz;
        {
          float cr[8], sr[8], rr[8];
          feat8(kq.k, kq.r0, kq.r1, om4, args.kr, KF, cr, sr, rr);
          __bf16* row = KS + (32 * tb + n32) * KP + 8 * h;
          if (32 * tb + n32 < nvalid) {
            *reinterpret_cast<u32x4*>(row) = ones4;
#pragma unroll
            for (int cc = 1; cc < 6; cc++) *reinterpret_cast<bf16x8*>(row + 16 * cc) = KF[cc - 1];
          } else {
#pragma unroll
            for (int cc = 0; cc < 6; cc++) *reinterpret_cast<u32x4*>(row + 16 * cc) = u32x4{0u, 0u, 0u, 0u};
          }
          feat8(kq.q, kq.r0, kq.r1, om4, args.kr, QF, cr, sr, rr);
          // Phi(q) . z: channel 0 in fp32, channels 1..5 as bf16 products like the rest of the readout
          const float4 z0a = *reinterpret_cast<const float4*>(Zg + 8 * h);
          const float4 z0b = *reinterpret_cast<const float4*>(Zg + 8 * h + 4);
          float d = ((z0a.x + z0a.y) + (z0a.z + z0a.w)) + ((z0b.x + z0b.y) + (z0b.z + z0b.w));
#pragma unroll
          for (int cc = 0; cc < 5; cc++) d = frag_dot(QF[cc], *reinterpret_cast<const bf16x8*>(Zb + 16 * (cc + 1) + 8 * h), d);
          dz = xor32_sum(d);
        }
        if (tb + 1 < TB) write_v(tb + 1, nvalid, vb);  // published by this block's barriers

        // numerators S^T Phi(q) (readout) + V^T P, P = the intra-chunk tiles A^T[s][t] of key blocks
        // sb <= tb, masked on the diagonal, as bf16 B operands, each folded in as soon as it is packed
        f32x16 num[2];
#pragma unroll
        for (int vt = 0; vt < 2; vt++) {
          zero16(num[vt]);
#pragma unroll
          for (int cc = 0; cc < 6; cc++) mma32(num[vt], SA[vt][cc], cc == 0 ? ONES : QF[cc - 1]);
        }
        float rs = 0.0f;
#pragma unroll
        for (int sb = 0; sb <= tb; sb++) {
          f32x16 at;
          zero16(at);
          mma32(at, ONES, ONES);  // channel 0: sixteen products 1 * 1
          const __bf16* krow = KS + (32 * sb + n32) * KP + 8 * h;
#pragma unroll
          for (int cc = 0; cc < 5; cc++)
            mma32(at, sb == tb ? KF[cc] : *reinterpret_cast<const bf16x8*>(krow + 16 * (cc + 1)), QF[cc]);
          float lo[8], hi8[8];
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int sl = 8 * (i >> 2) + 4 * h + (i & 3);
            const float a = (sb == tb && sl > n32) ? 0.0f : at[i];
            if (i < 8) lo[i] = a;
            else hi8[i - 8] = a;
          }
          u32x4 w0, w1;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            w0[q] = pack_bf16x2(lo[2 * q], lo[2 * q + 1]);
            w1[q] = pack_bf16x2(hi8[2 * q], hi8[2 * q + 1]);
          }
          const bf16x8 P0 = __builtin_bit_cast(bf16x8, w0), P1 = __builtin_bit_cast(bf16x8, w1);
          rs = frag_sum(P1, frag_sum(P0, rs));
#pragma unroll
          for (int vt = 0; vt < 2; vt++) {
            mma32(num[vt], lds_tokfrag(Vs, VP, 32 * sb, 32 * vt, l), P0);
            mma32(num[vt], lds_tokfrag(Vs, VP, 32 * sb + 16, 32 * vt, l), P1);
          }
        }
        const float den = xor32_sum(rs) + dz;
        // the previous block's normalisation (same scheduling region as this block's work, so the two
        // overlap) must be done everywhere before the buffer is overwritten
        if (tb > 0) __syncthreads();
        float* rrow = red + (grp * 32 + n32) * RP;
#pragma unroll
        for (int vt = 0; vt < 2; vt++)
#pragma unroll
          for (int q = 0; q < 4; q++)
            *reinterpret_cast<float4*>(rrow + 32 * vt + 8 * q + 4 * h) =
                make_float4(num[vt][4 * q], num[vt][4 * q + 1], num[vt][4 * q + 2], num[vt][4 * q + 3]);
        rrow[64] = den;  // both halves store the same value
        __syncthreads();
        // o = num / (den + c eps) for the block's rows: thread -> row tid / 8, values 8 (tid % 8) .. + 7
        {
          const int t = tid >> 3, c0 = 8 * (tid & 7);
          if (32 * tb + t < nvalid) {
            const float* b0 = red + t * RP;
            constexpr int GS = 32 * RP;
            const float dsum = ((b0[64] + b0[GS + 64]) + b0[2 * GS + 64]) + b0[3 * GS + 64];
            const float inv = 1.0f / (dsum + args.ceps);
            u32x4 w;
#pragma unroll
            for (int half = 0; half < 2; half++) {
              const int cb = c0 + 4 * half;
              const float4 a0 = *reinterpret_cast<const float4*>(b0 + cb);
              const float4 a1 = *reinterpret_cast<const float4*>(b0 + GS + cb);
              const float4 a2 = *reinterpret_cast<const float4*>(b0 + 2 * GS + cb);
              const float4 a3 = *reinterpret_cast<const float4*>(b0 + 3 * GS + cb);
              w[2 * half] = pack_bf16x2((((a0.x + a1.x) + a2.x) + a3.x) * inv, (((a0.y + a1.y) + a2.y) + a3.y) * inv);
              w[2 * half + 1] =
                  pack_bf16x2((((a0.z + a1.z) + a2.z) + a3.z) * inv, (((a0.w + a1.w) + a2.w) + a3.w) * inv);
            }
            *reinterpret_cast<u32x4*>(op + (size_t)(t0 + 32 * tb + t) * kDV + c0) = w;
          }
        }
        kq = kqn;
        va = vb;
        vb = vn;
      }

      // state update S += Phi(K)^T V, z += Phi(K)^T 1 over the chunk's 128 tokens
      float zs[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 2 * TB; ks++) {
        const bf16x8 B0 = lds_tokfrag(Vs, VP, 16 * ks, 0, l);
        const bf16x8 B1 = lds_tokfrag(Vs, VP, 16 * ks, 32, l);
#pragma unroll
        for (int ft = 0; ft < 3; ft++) {
          const bf16x8 A = lds_tokfrag_swz(KS, KP, 16 * ks, 32 * ft, l);
          zs[ft] = frag_sum(A, zs[ft]);
          mma32(Sacc[ft][0], A, B0);
          mma32(Sacc[ft][1], A, B1);
        }
      }
#pragma unroll
      for (int ft = 0; ft < 3; ft++) {
        const int m = 32 * ft + 16 * (n32 >> 4) + swz16(n32 & 15);
        const float znew = Zg[m] + xor32_sum(zs[ft]);
        Zg[m] = znew;  // both halves store the same value
        Zb[m] = (__bf16)znew;
      }
      __syncthreads();  // everyone is done with this chunk's tiles
    }
    if (last_piece && args.S) gstate_store(Sacc, Zg, args.S + (size_t)bh * kF * kDV, args.z + (size_t)bh * kF, grp, l);
  }
}

template <bool RAGGED>
hipError_t launch_prefill_grp128(const PrefillArgs& a, hipStream_t stream) {
  static_assert(Geom128::lds <= 160 * 1024, "LDS budget");
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute((const void*)prefill_grp128_kernel<RAGGED>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, Geom128::lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(prefill_grp128_kernel<RAGGED>, dim3(a.G), dim3(256), Geom128::lds, stream, a);
  return hipGetLastError();
}

template <int CH, bool RAGGED>
hipError_t launch_grp_t(const PrefillArgs& a, int BH, hipStream_t stream) {
  using G = GeomG<CH>;
  static_assert(G::lds(false) <= 160 * 1024, "LDS budget");
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)prefill_grp_kernel<CH, true, RAGGED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G::lds(true));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)prefill_grp_kernel<CH, false, RAGGED>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, G::lds(false));
    if (e != hipSuccess) return e;
    if constexpr (CH == 64) {
      e = hipFuncSetAttribute((const void*)prefill_state8_kernel<64, RAGGED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, GeomS8::lds);
      if (e != hipSuccess) return e;
    }
    attr_set[dev].store(true, std::memory_order_release);
  }
  if (a.multi) {
    if constexpr (CH == 64)
      hipLaunchKernelGGL((prefill_state8_kernel<64, RAGGED>), dim3(a.G), dim3(512), GeomS8::lds, stream, a);
    else
      hipLaunchKernelGGL((prefill_grp_kernel<CH, true, RAGGED>), dim3(a.G), dim3(256), G::lds(true), stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.scanned) {
      e = launch_prefill_scan(a, BH, stream);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((prefill_grp_kernel<CH, false, RAGGED>), dim3(a.G), dim3(256), G::lds(false), stream, a);
  return hipGetLastError();
}

// pass 1 for 128-token chunks: the 8-wave state kernel walks each chunk as two 64-token halves
template <bool RAGGED>
hipError_t launch_prefill_state8_128(const PrefillArgs& a, hipStream_t stream) {
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute((const void*)prefill_state8_kernel<128, RAGGED>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, GeomS8::lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((prefill_state8_kernel<128, RAGGED>), dim3(a.G), dim3(512), GeomS8::lds, stream, a);
  return hipGetLastError();
}

template <bool RAGGED>
hipError_t launch_prefill_grp_r(const PrefillArgs& a, int chunk, int BH, hipStream_t stream) {
  switch (chunk) {
    case 16: return launch_grp_t<16, RAGGED>(a, BH, stream);
    case 32: return launch_grp_t<32, RAGGED>(a, BH, stream);
    case 64: return launch_grp_t<64, RAGGED>(a, BH, stream);
    case 128: {
      if (a.multi) {
        hipError_t e = launch_prefill_state8_128<RAGGED>(a, stream);
        if (e != hipSuccess) return e;
        if (a.scanned) {
          e = launch_prefill_scan(a, BH, stream);
          if (e != hipSuccess) return e;
        }
      }
      return launch_prefill_grp128<RAGGED>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_grp(const PrefillArgs& a, int chunk, int BH, hipStream_t stream) {
  return a.lens ? launch_prefill_grp_r<true>(a, chunk, BH, stream) : launch_prefill_grp_r<false>(a, chunk, BH, stream);
}

}  // namespace sanatan
