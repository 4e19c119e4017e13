// prefill_common.h -- pieces shared by the chunked-prefill kernels (prefill.hip, prefill_grp.hip).
//
// Feature ownership used by every variant: feature group g (0..3) = content dims 16g..16g+15,
// i.e. 96 features (6 channels x 16 dims); wave feature index m = 16 c + dim.  Within a group the
// state rows are tiled as 3 "f-tiles" of 32 features (ft = m / 32).  In a 32x32 accumulator tile
// lane (n32 = l % 32, h = l / 32) holds rows 8 j + 4 h + i4 (j < 4, i4 < 4; register 4 j + i4) of
// column n32 -- so K-step c (16 features) of an MFMA operand is channel c, and lane (row, h) holds
// dims {4h..4h+3, 8+4h..11+4h} of it.
#pragma once

#include <type_traits>

#include "launchers.h"
#include "sanatan_device.h"

namespace sanatan {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> one word of two bf16 (round to nearest even), low half = a.
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// x[l] + x[l ^ 32] in every lane, with the gfx950 half-swap instead of an LDS permute.  The swapped
// words are read back through plain unsigned copies: a bit_cast applied directly to an element of
// the returned pair was miscompiled into element 0.
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a0 = r[0], a1 = r[1];
  return __uint_as_float(a0) + __uint_as_float(a1);
}

__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; i++) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
}
// acc = a b + c (the accumulator starts from c instead of its own value)
__device__ __forceinline__ void mma32c(f32x16& acc, const bf16x8& a, const bf16x8& b, const f32x16& c) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32c(f32x16& acc, const f32x8& a, const f32x8& b, const f32x16& c) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
#pragma unroll
  for (int i = 1; i < 8; i++) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
}
__device__ __forceinline__ void zero16(f32x16& a) {
#pragma unroll
  for (int i = 0; i < 16; i++) a[i] = 0.0f;
}

// Work partition (see prefill_plan): the flattened (sequence, chunk) list split into G ranges, one per
// workgroup.  Piece (bh, g) owns boundary-state slot bh + g (disjoint and increasing in (bh, g)).
// A ragged call (lens != null) gives batch element b the length lens[b] (clamped to [0, T]); its H
// sequences then hold ceil(len / chunk) chunks each, in the same flattened order.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* omega;
  float* S;          // user state [BH][6d][dv] or null
  float* z;          // user state [BH][6d] or null
  float* ws_state;   // [BH + G - 1][kStateFloats]
  const float* rho;  // [T][64] position phases in revolutions
  long long total;   // BH * ncs chunks (uniform calls)
  int G, ncs, nph, H, T;
  int multi;         // some sequence spans several pieces: pass 1 ran
  int scanned;       // the scan kernel ran: each slot holds its piece's prefix (else pass 3 sums slots)
  float kr, ceps;
  const int* lens;   // [B] per-batch-element lengths (device), or null: every sequence has T tokens
  int B, chunk;
  int chunk_log2;    // chunk = 1 << chunk_log2 (16, 32, 64 or 128)
};

__device__ __forceinline__ int ragged_len(const PrefillArgs& a, int b) {
  const int L = a.lens[b];
  return L < 0 ? 0 : (L > a.T ? a.T : L);
}
// chunks of a sequence of L tokens (the chunk is a power of two: a shift, not a division)
__device__ __forceinline__ long long ragged_chunks(const PrefillArgs& a, int L) {
  return (long long)((L + a.chunk - 1) >> a.chunk_log2);
}
// Chunks of the whole call.  A ragged call's count is summed from the lengths by every workgroup (B scalar
// loads and a few scalar operations each), so that the partition needs no host copy of them.  RAGGED is a template flag of the kernels, so
// that the uniform kernels carry none of this code.
template <bool RAGGED>
__device__ __forceinline__ long long call_chunks(const PrefillArgs& a) {
  if (!RAGGED) return a.total;
  long long n = 0;
  for (int b = 0; b < a.B; b++) n += (long long)a.H * ragged_chunks(a, ragged_len(a, b));
  return n;
}
// The sequence holding flattened chunk c: its index bh, its chunks [c0, c1) and its length in tokens.
// bh = -1 if no sequence holds c (cannot happen for c < call_chunks(a) with unchanged lengths).
struct SeqSpan {
  long long c0, c1;
  int bh, len;
};
template <bool RAGGED>
__device__ __forceinline__ SeqSpan seq_span(long long c, const PrefillArgs& a) {
  SeqSpan s;
  if (!RAGGED) {
    s.bh = (int)(c / a.ncs);
    s.c0 = (long long)s.bh * a.ncs;
    s.c1 = s.c0 + a.ncs;
    s.len = a.T;
    return s;
  }
  long long acc = 0;
  for (int b = 0; b < a.B; b++) {
    const int L = ragged_len(a, b);
    const long long n = ragged_chunks(a, L);
    if (c < acc + a.H * n) {
      const int h = (int)((c - acc) / n);
      s.bh = b * a.H + h;
      s.c0 = acc + h * n;
      s.c1 = s.c0 + n;
      s.len = L;
      return s;
    }
    acc += a.H * n;
  }
  s.bh = -1; s.c0 = s.c1 = c; s.len = 0;
  return s;
}
// The chunks [c0, c1) of sequence bh (empty for a ragged length of 0).
__device__ __forceinline__ SeqSpan seq_span_of(int bh, const PrefillArgs& a) {
  SeqSpan s;
  s.bh = bh;
  if (!a.lens) {
    s.c0 = (long long)bh * a.ncs;
    s.c1 = s.c0 + a.ncs;
    s.len = a.T;
    return s;
  }
  const int bb = bh / a.H, h = bh % a.H;
  long long acc = 0;
  for (int b = 0; b < bb; b++) acc += (long long)a.H * ragged_chunks(a, ragged_len(a, b));
  s.len = ragged_len(a, bb);
  const long long n = ragged_chunks(a, s.len);
  s.c0 = acc + h * n;
  s.c1 = s.c0 + n;
  return s;
}

__device__ __forceinline__ long long range_lo(long long g, long long total, int G) { return g * total / G; }
// Range (logical workgroup) of this workgroup.  Workgroups are dealt round-robin to the 8 XCDs, each
// with its own L2; consecutive ranges -- the pieces of one sequence -- are given to workgroups on the
// same XCD, so that pass 3 reads its predecessors' boundary states from the L2 that pass 1 wrote
// them through.  A bijection on [0, G); the last G % 8 workgroups keep their own index.
__device__ __forceinline__ int range_of_block(const PrefillArgs& a) {
  const int b = (int)blockIdx.x, per = a.G / 8;
  return b < 8 * per ? (b % 8) * per + b / 8 : b;
}
// The range holding chunk c (ranges may be empty when G exceeds the chunk count; c's range is still unique)
__device__ __forceinline__ int range_of_chunk(long long c, long long total, int G) {
  return (int)(((c + 1) * G - 1) / total);
}

hipError_t launch_prefill_grp(const PrefillArgs& a, int chunk, int BH, hipStream_t stream);
hipError_t launch_prefill_scan(const PrefillArgs& a, int BH, hipStream_t stream);

template <typename T> __device__ __forceinline__ typename FragT<T>::type pack8f(const float (&x)[8]) {
  typename FragT<T>::type f;
#pragma unroll
  for (int i = 0; i < 8; i++) f[i] = (T)x[i];
  return f;
}

// Token-consecutive operand from a token-major LDS tile [token][pitch]: lane (row = l % 32, h)
// gets column col0 + (l % 32) at tokens tok0 + 8*(i/4) + 4h + (i % 4), i = 0..7.
// bf16: two transposing loads; each 16-lane block addresses 4 tokens x 4 column groups, and lane j
// of the block receives column j of those 4 tokens.  Whole-vector bit casts only: per-element casts
// of the loaded halves were miscompiled into duplicated words.
__device__ __forceinline__ bf16x8 lds_tokfrag(const __bf16* buf, int pitch, int tok0, int col0, int l) {
  const int b = l >> 4, L = l & 15;
  const int tok = tok0 + 4 * (b >> 1) + (L >> 2);
  const int col = col0 + 16 * (b & 1) + 4 * (L & 3);
  const u32x2 lo =
      __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + tok * pitch + col)));
  const u32x2 hi = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + (tok + 8) * pitch + col)));
  const u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ f32x8 lds_tokfrag(const float* buf, int pitch, int tok0, int col0, int l) {
  const int col = col0 + (l & 31), tb = tok0 + 4 * (l >> 5);
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[i] = buf[(tb + i) * pitch + col];
    f[4 + i] = buf[(tb + 8 + i) * pitch + col];
  }
  return f;
}

// Row operand (channel c = K-step, 8 dims of one token) from a token-major feature tile [token][pitch]
// whose columns are wave features 16c + dim.
template <typename T>
__device__ __forceinline__ typename FragT<T>::type lds_rowfrag(const T* ks, int pitch, int s, int c, int h) {
  typename FragT<T>::type f;
  const T* p = ks + s * pitch + 16 * c + 4 * h;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[i] = p[i];
    f[4 + i] = p[8 + i];
  }
  return f;
}

// This lane's 8 values (dims dbase + {0..3, 8..11}) of one row.
__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 8);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const __bf16* p, float (&o)[8]) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p), b = *reinterpret_cast<const bf16x4*>(p + 8);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o[i] = (float)a[i];
    o[4 + i] = (float)b[i];
  }
}

// The same 8 values kept raw (two 4-element pieces) so that they can be loaded a chunk ahead.
template <typename T> struct Raw8 {
  typedef typename std::conditional<sizeof(T) == 2, uint2, uint4>::type Half;
  Half a, b;
};
template <typename T> __device__ __forceinline__ void load_raw8(const T* p, Raw8<T>& r) {
  r.a = *reinterpret_cast<const typename Raw8<T>::Half*>(p);
  r.b = *reinterpret_cast<const typename Raw8<T>::Half*>(p + 8);
}
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float (&o)[8]) {
  o[0] = __uint_as_float(r.a.x); o[1] = __uint_as_float(r.a.y); o[2] = __uint_as_float(r.a.z);
  o[3] = __uint_as_float(r.a.w); o[4] = __uint_as_float(r.b.x); o[5] = __uint_as_float(r.b.y);
  o[6] = __uint_as_float(r.b.z); o[7] = __uint_as_float(r.b.w);
}
__device__ __forceinline__ void unpack8(const Raw8<__bf16>& r, float (&o)[8]) {
  const bf16x4 a = __builtin_bit_cast(bf16x4, r.a), b = __builtin_bit_cast(bf16x4, r.b);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o[i] = (float)a[i];
    o[4 + i] = (float)b[i];
  }
}

// Featurize this lane's 8 dims of one token given the position phases rho (revolutions):
// ch[c][i] = channel c (1, cos, sin, r, r cos, r sin) of dim i.
__device__ __forceinline__ void featurize8(const float (&u)[8], const float (&rho)[8], const float (&om4)[8], float kr,
                                           float (&ch)[6][8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float cr, sr, rr;
    featurize1(u[i], rho[i], om4[i], kr, cr, sr, rr);
    ch[0][i] = 1.0f;
    ch[1][i] = cr;
    ch[2][i] = sr;
    ch[3][i] = rr;
    ch[4][i] = rr * cr;
    ch[5][i] = rr * sr;
  }
}

// Sum of the 8 bf16 values of a fragment (v_dot2 with ones).  Pairs are taken with shufflevector:
// extracting words from a bit-cast of the bf16 vector was miscompiled into reusing the first word.
__device__ __forceinline__ float frag_sum(const bf16x8& f, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), one, acc, false);
  return acc;
}
// acc + sum of the 8 products f[i] g[i] of two bf16 fragments (four v_dot2)
__device__ __forceinline__ float frag_dot(const bf16x8& f, const bf16x8& g, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), __builtin_shufflevector(g, g, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), __builtin_shufflevector(g, g, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), __builtin_shufflevector(g, g, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), __builtin_shufflevector(g, g, 6, 7), acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sum(const f32x8& f, float acc) {
#pragma unroll
  for (int i = 0; i < 8; i++) acc += f[i];
  return acc;
}

// ------------------------------------------------------------------ state staging through LDS
// State I/O goes through LDS so global traffic stays coalesced and each lane moves its accumulator
// slice with constant LDS offsets.  Staging layout (floats): S at [g][vt][ft][i][lane] (lane fastest,
// i = accumulator register), then z at [g][96] (wave feature m).
constexpr int kStageS = 4 * 2 * 3 * 16 * 64;  // = 6d * d_v

__device__ __forceinline__ int stage_index(int row, int col) {
  const int c = row >> 6, a = row & 63, g = a >> 4, dim = a & 15;
  const int m = 16 * c + dim, ft = m >> 5, mm = m & 31;
  const int j = mm >> 3, h = (mm >> 2) & 1, i4 = mm & 3;
  const int vt = col >> 5, n32 = col & 31;
  return (((g * 2 + vt) * 3 + ft) * 16 + 4 * j + i4) * 64 + 32 * h + n32;
}

// global state (ABI layout: S [6d][d_v] then z [6d]) <-> staging; NT threads cooperate.
template <int NT>
__device__ __forceinline__ void stage_in(float* st, const float* __restrict__ s, const float* __restrict__ zz) {
  for (int e4 = threadIdx.x; e4 < kF * kDV / 4; e4 += NT) {
    const float4 v = reinterpret_cast<const float4*>(s)[e4];
    const int row = (4 * e4) / kDV, col = (4 * e4) % kDV;
    *reinterpret_cast<float4*>(st + stage_index(row, col)) = v;  // 4 columns = 4 consecutive lanes
  }
  for (int r = threadIdx.x; r < kF; r += NT) {
    const int c = r >> 6, a = r & 63;
    st[kStageS + (a >> 4) * 96 + 16 * c + (a & 15)] = zz[r];
  }
}
template <int NT>
__device__ __forceinline__ void stage_out(const float* st, float* __restrict__ s, float* __restrict__ zz) {
  for (int e4 = threadIdx.x; e4 < kF * kDV / 4; e4 += NT) {
    const int row = (4 * e4) / kDV, col = (4 * e4) % kDV;
    reinterpret_cast<float4*>(s)[e4] = *reinterpret_cast<const float4*>(st + stage_index(row, col));
  }
  for (int r = threadIdx.x; r < kF; r += NT) {
    const int c = r >> 6, a = r & 63;
    zz[r] = st[kStageS + (a >> 4) * 96 + 16 * c + (a & 15)];
  }
}
// One value tile (vt) of group g: staging -> accumulators (added) / accumulators -> staging.
__device__ __forceinline__ void stage_add_tile(f32x16 (&acc)[3], const float* st, int g, int vt, int l) {
  const float* p = st + (g * 2 + vt) * (3 * 16 * 64) + l;
#pragma unroll
  for (int ft = 0; ft < 3; ft++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[ft][i] += p[(ft * 16 + i) * 64];
}
__device__ __forceinline__ void stage_put_tile(const f32x16 (&acc)[3], float* st, int g, int vt, int l) {
  float* p = st + (g * 2 + vt) * (3 * 16 * 64) + l;
#pragma unroll
  for (int ft = 0; ft < 3; ft++)
#pragma unroll
    for (int i = 0; i < 16; i++) p[(ft * 16 + i) * 64] = acc[ft][i];
}

}  // namespace sanatan
