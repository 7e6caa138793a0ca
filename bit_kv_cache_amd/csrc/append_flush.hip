// Append + flush kernels of the WUSH-KV cache on gfx950.
//
// Append writes new tokens' fp16 values into the sink window or the ring of the
// recent window.  Flush quantizes tokens leaving the recent window (WUSH-KV digest,
// "takeaways" / "method key points": FP16 sink and recent windows, chunked flush;
// the key transform after RoPE, one d x d product per token).
//
// Flush: per token, x = T_K k16 (keys) on MFMA, the token's quantizer parameters
// (RMS step or percentile-clipped scale / zero), codes, then K rows and V set words
// packed and stored.  The kernel's own layout of work is described at flush_kernel.
#include <type_traits>

#include "wushkv_internal.h"

namespace wushkv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// ------------------------------------------------------------------ append

// The new tokens of a sequence that land in a window: t in [0, ns) go to the sink, t in
// [tr, n_new) to the ring; the ones between are quantized straight from the input by the
// flush kernel.  Returns ns + (n_new - tr).
__host__ __device__ inline int64_t window_tokens(int64_t n_before, int64_t n_new, int64_t q_after, int S,
                                                 int64_t &ns, int64_t &tr) {
  ns = S - n_before;
  ns = ns < 0 ? 0 : (ns > n_new ? n_new : ns);
  tr = S + q_after - n_before;
  tr = tr < ns ? ns : (tr > n_new ? n_new : tr);
  return ns + (n_new - tr);
}

// Element (window token i, 8-channel group) idx of KV head bg: its fp16 copy into the
// sink or its ring slot.
template <class A>
__device__ __forceinline__ void append_group(const A &a, _Float16 *sink_k, _Float16 *sink_v, _Float16 *ring_k,
                                             _Float16 *ring_v, size_t sink_bytes, int bg, int64_t n_before,
                                             int64_t q_after, int64_t idx) {
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int groups = a.d / 8;
  const int64_t i = idx / groups;
  const int j0 = (int)(idx % groups) * 8;
  int64_t ns, tr;
  if (i >= window_tokens(n_before, a.n_new, q_after, a.S, ns, tr)) return;
  const int64_t t = i < ns ? i : tr + (i - ns);
  const int64_t p = n_before + t;
  _Float16 *dk, *dv;
  if (p < a.S) {
    dk = (_Float16 *)((char *)sink_k + bg * sink_bytes) + p * a.d;
    dv = (_Float16 *)((char *)sink_v + bg * sink_bytes) + p * a.d;
  } else {
    const int64_t slot = (p - a.S) % (a.R + a.C);
    dk = (_Float16 *)((char *)ring_k + bg * a.ring_bytes) + slot * a.d;
    dv = (_Float16 *)((char *)ring_v + bg * a.ring_bytes) + slot * a.d;
  }
  const size_t src = (((size_t)b * a.Hkv + g) * a.n_new + t) * a.d + j0;
  half8 hk, hv;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hk[e] = (_Float16)load_in(a.k_new, a.in_dtype, src + e);
    hv[e] = (_Float16)load_in(a.v_new, a.in_dtype, src + e);
  }
  *(half8 *)(dk + j0) = hk;
  *(half8 *)(dv + j0) = hv;
}

__global__ void __launch_bounds__(kThreads) append_kernel(AppendArgs a) {
  // one thread per (window token, 8-channel group); blockIdx.y = b * Hkv + g.  The grid
  // covers the most window tokens any sequence has, not all n_new tokens.
  const int bg = blockIdx.y;
  const int64_t n_before = seq_before(a, bg / a.Hkv);
  if (n_before < 0) return;
  const int64_t q_after = a.ragged ? n_quantized(n_before + a.n_new, a.S, a.R, a.C) : a.q_after;
  append_group(a, a.sink_k, a.sink_v, a.ring_k, a.ring_v, a.sink_bytes, bg, n_before, q_after,
               (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// ------------------------------------------------------------------ flush
//
// Workgroup of 4 waves; it stages T_K of its KV head in LDS once and then walks
// steps of 128 body tokens (two 64-token V sets).  In a step, wave w holds 32
// tokens as two 16-token tiles.  Lane (q, tok) = (lane / 16, lane % 16) owns
// CPL = D / 4 channels of token tok of each tile (eight-channel chunks q, q + 4, ...
// of the row), so a token's row sits in the 4 lanes tok, tok+16, tok+32, tok+48 and
// every per-token reduction is two cross-row exchanges.
//   keys:   x = T_K k16 on v_mfma_f32_16x16x32_f16 with A = T_K rows (LDS) and
//           B = the lane's own fp16 channels, so the result D[out channel][token]
//           lands with lane (q, tok) holding out channels 16*ct + 4*q + i of tok;
//   values: used as loaded (their fp16 value).
// Codes go to LDS (keys token-major, values channel-major), then the whole
// workgroup packs K rows and V set words and writes them with 16-byte stores.

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStepTok = 128;      // body tokens per workgroup step (two V sets)
// An element whose scaled value lies within these distances (in bins) of a
// decision boundary is decided again from its exact value in fp64.  Keys carry
// the fp32 accumulation error of the MFMA contraction (at most 6.2e-6 bins at 4
// bits, 1.5e-6 at 2 bits, over 1.3e8 transformed keys of the bulk-flush
// workload).  In bins that error grows with the number of levels L (a bin is 1/L of
// the clip range, resp. 1/(L-1) of the percentile range), so the key distance is
// kEdgeK * L / 16: the same eightfold margin at every width.  Values carry only the
// rounding of the scale's reciprocal and of one product.
constexpr float kEdgeK = 5e-5f;
constexpr float kEdgeV = 1e-5f;

// fp16 parameters are re-decided in fp64 when their fp32 value lies within these
// relative distances of an fp16 rounding midpoint (measured on gfx950 over 2.6e5 keys of
// the bulk-flush workload: the contraction's fp32 error moves a key row's sum of squares
// by at most 1.2e-7 and an extreme element by at most 4.9e-7 of itself; a row's fp32
// sum of squares, a chain of 12 roundings, by at most 7.2e-7).
//   kParV:    values (their x is exact): the fp32 arithmetic alone.
//   kParKA:   QuEST keys, first stage: all of the fp32 error; the step is then taken
//             from the fp64 sum of squares of the fp32 x.
//   kParKB:   QuEST keys, second stage: the contraction's error alone (3x); such rows get
//             the exact sum of squares from fp64 dot products.
//   kParKAff: affine keys: the extreme elements' error and the fp32 interpolation (3x);
//             such rows get their order
//             statistics from exact fp64 dot products.
constexpr float kParV = 1.2e-6f;
constexpr float kParKA = 1.5e-6f;
constexpr float kParKB = 2e-7f;
constexpr float kParKAff = 2.5e-6f;
constexpr float kParKAff2 = 1.5e-6f;   // affine keys after the fp64 interpolation: the elements' error (3x)
constexpr int kDefer = 32;     // key rows per wave and step queued for exact parameters (all of them)
constexpr int kStaged = 2;     // of those, per wave, the first ones whose fp16 key row is kept in LDS
constexpr int kMaxCand = 16;   // affine: order-statistic candidates resolved exactly per row

// A queued key row: its row in the step; affine: each of its four lanes' candidate
// elements (bit 4 ct + i = out channel 16 ct + 4 q + i) with the cuts, and the first
// stage's parameters.
struct DeferRow {
  unsigned cm[4];
  float clo, chi, mg, sc, zp;
  int row;
};

template <int D>
struct __align__(16) FlushSmem {
  static constexpr int TP = D + 8;      // T_K row pitch (halves)
  static constexpr int KP = D + 16;     // key-code row pitch (bytes; rows stay 16-byte aligned)
  static constexpr int VP = kSet + 4;   // value-code row pitch (bytes), one row per channel
  _Float16 t[D][TP];
  union {
    struct {   // codes as bytes (3- and 4-bit widths)
      uint8_t kc[kStepTok][KP];
      uint8_t vc[2][D][VP];
    };
    struct {   // 2-bit K and V: packed key rows and, per set and 16-token quarter, set words
      unsigned kp[kStepTok][D / 16];
      unsigned vw[2][4][4 * D];
    };
  };
  unsigned krow[D / 2];                 // one key row's fp16 pairs (exact re-decisions)
  double red[4][2 * kMaxOrderStats];    // per wave: partial sums / order statistics of that row
  double cand[kMaxCand];                // affine: exact values of the row's candidates
  int dqn[4];                           // per wave: rows queued in this step
  DeferRow dq[4][kDefer];               // per wave: the step's queued key rows
  unsigned kq[4][kStaged][D / 2];       // per wave: the first queued rows' fp16 keys (as krow)
};

// Raw bytes of one lane's CPL channels of one token row, in the input's element size.
// Channel of position k of lane group q's list.
__device__ __forceinline__ int seg_chan(int q, int k) { return 32 * (k >> 3) + 8 * q + (k & 7); }

template <int ES, int CPL>
struct RawSeg {
  u32x4 r[CPL * ES / 16];
};

template <int ES, int CPL>
__device__ __forceinline__ unsigned raw_word(const RawSeg<ES, CPL> &s, int i) {
  return s.r[i >> 2][i & 3];
}

// Load the segment of body token u (valid) from the ring if it was appended by an
// earlier call (an fp16 row), else from the new input; an invalid token reads zeros (2-byte
// input: the head's first input row), values that are never used.
// Lane group q holds channels 32 i + 8 q .. 32 i + 8 q + 7 (i = 0 .. D/32 - 1), at
// position 8 i + e of its list: one load instruction then covers 32 contiguous
// channels of each of its 16 rows.
template <int D, int ES>
__device__ __forceinline__ void load_seg(const FlushArgs &a, int64_t n_before, const char *ring_h, const char *in_h,
                                         int64_t u, bool valid, int q, RawSeg<ES, D / 4> &s) {
  constexpr int CPL = D / 4;
  if constexpr (ES == 2) {
    // 2-byte input rows have the ring's layout: every lane issues the same loads from a
    // selected row (an invalid token reads the head's first input row, which exists
    // whenever there is a body row to flush, and its values are never used), so no
    // branch surrounds the loads and the wave's load counter stays exact
    const bool ring = valid && a.S + u < n_before;
    const char *row = in_h + (size_t)((valid && !ring) ? a.S + u - n_before : 0) * (D * 2);
    if (__builtin_expect(__any(ring), 0)) {
      const unsigned slot = (unsigned)u % (unsigned)(a.R + a.C);
      if (ring) row = ring_h + (size_t)slot * (D * 2);
    }
    const u32x4 *src = (const u32x4 *)row + q;
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) s.r[i] = __builtin_nontemporal_load(src + 4 * i);
    return;
  }
#pragma unroll
  for (int i = 0; i < CPL * ES / 16; ++i) s.r[i] = (u32x4){0u, 0u, 0u, 0u};
  if (!valid) return;
  if (a.S + u < n_before) {
    const unsigned slot = (unsigned)u % (unsigned)(a.R + a.C);
    const u32x4 *src = (const u32x4 *)(ring_h + (size_t)slot * (D * 2)) + q;
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) s.r[i] = src[4 * i];
    return;
  }
  const u32x4 *src = (const u32x4 *)(in_h + (size_t)(a.S + u - n_before) * (D * ES)) + (ES / 2) * q;
#pragma unroll
  for (int i = 0; i < CPL / 8; ++i)
#pragma unroll
    for (int h = 0; h < ES / 2; ++h) s.r[(ES / 2) * i + h] = __builtin_nontemporal_load(src + 2 * ES * i + h);
}

// The same row segment with lane group q holding channels 16 ct + 4 q .. 16 ct + 4 q + 3
// (ct = 0 .. D/16 - 1), at positions 4 ct + i: the channels the key contraction's output
// puts in a lane, so that the in-register Hadamard transform needs no transpose.
template <int D, int ES>
__device__ __forceinline__ void load_seg_ct(const FlushArgs &a, int64_t n_before, const char *ring_h, const char *in_h,
                                            int64_t u, bool valid, int q, RawSeg<ES, D / 4> &s) {
  constexpr int NCT = D / 16;
#pragma unroll
  for (int i = 0; i < D * ES / 64; ++i) s.r[i] = (u32x4){0u, 0u, 0u, 0u};
  if (!valid) return;
  const bool ring = a.S + u < n_before;
  const char *row = ring ? ring_h + (size_t)((unsigned)u % (unsigned)(a.R + a.C)) * (D * 2)
                         : in_h + (size_t)(a.S + u - n_before) * (D * ES);
  if (ring || ES == 2) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const u32x2 w = ring ? *(const u32x2 *)(row + 32 * ct + 8 * q)
                           : __builtin_nontemporal_load((const u32x2 *)(row + 32 * ct + 8 * q));
      s.r[ct >> 1][2 * (ct & 1)] = w[0];
      s.r[ct >> 1][2 * (ct & 1) + 1] = w[1];
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s.r[ct] = __builtin_nontemporal_load((const u32x4 *)(row + 64 * ct + 16 * q));
  }
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(unsigned w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16_hi(unsigned w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
__device__ __forceinline__ float f16_round(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ unsigned pack_f16(float x, float y) {
  f16x2 v = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(unsigned, v);
}

// The segment as fp16 pairs (the key's fp16 value, round-to-nearest-even).
template <int ES, int CPL>
__device__ __forceinline__ void seg_half2(const RawSeg<ES, CPL> &s, bool ring, int dt, unsigned (&h)[CPL / 2]) {
  if (ring || (ES == 2 && dt == WUSHKV_DT_F16)) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) h[i] = raw_word(s, i);
  } else if (ES == 2) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
      const unsigned w = raw_word(s, i);
      h[i] = pack_f16(bf16_lo(w), bf16_hi(w));
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i)
      h[i] = pack_f16(__uint_as_float(raw_word(s, 2 * i)), __uint_as_float(raw_word(s, 2 * i + 1)));
  }
}

// The segment as floats holding the fp16 values.
template <int ES, int CPL>
__device__ __forceinline__ void seg_float(const RawSeg<ES, CPL> &s, bool ring, int dt, float (&x)[CPL]) {
  if (ring || (ES == 2 && dt == WUSHKV_DT_F16)) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
      const unsigned w = raw_word(s, i);
      x[2 * i] = f16_lo(w);
      x[2 * i + 1] = f16_hi(w);
    }
  } else {
    // one round-to-nearest-even conversion per pair, then the fp16 values as floats
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
      unsigned h = ES == 2 ? pack_f16(bf16_lo(raw_word(s, i)), bf16_hi(raw_word(s, i)))
                           : pack_f16(__uint_as_float(raw_word(s, 2 * i)), __uint_as_float(raw_word(s, 2 * i + 1)));
      asm("" : "+v"(h));   // keep the paired conversion (not one per element)
      x[2 * i] = f16_lo(h);
      x[2 * i + 1] = f16_hi(h);
    }
  }
}

// ---- per-token parameters; the 4 lanes of a token exchange through lanes ^16, ^32

// x + x of lane ^ M (M = 16 or 32) through gfx950's permlane swaps, which give both lanes
// of the pair (x of the lower lane, x of the upper lane): the same sum, bit for bit, in
// both, with no LDS round trip
template <int M>
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int NL>
struct OrderStats {
  float lo[NL > 0 ? NL : 1], hi[NL > 0 ? NL : 1];  // lo ascending, hi descending
};

template <int NL>
__device__ __forceinline__ void os_init(OrderStats<NL> &o) {
#pragma unroll
  for (int k = 0; k < NL; ++k) { o.lo[k] = INFINITY; o.hi[k] = -INFINITY; }
}

template <int NL>
__device__ __forceinline__ void os_insert(OrderStats<NL> &o, float v) {
#pragma unroll
  for (int k = NL - 1; k > 0; --k) o.lo[k] = __builtin_amdgcn_fmed3f(o.lo[k - 1], o.lo[k], v);
  o.lo[0] = fminf(o.lo[0], v);
#pragma unroll
  for (int k = NL - 1; k > 0; --k) o.hi[k] = __builtin_amdgcn_fmed3f(o.hi[k - 1], o.hi[k], v);
  o.hi[0] = fmaxf(o.hi[0], v);
}

// Keep the NL smallest / largest of this lane's lists and those of lane ^ mask:
// pairing a[k] with b[NL-1-k] leaves a bitonic sequence of the NL extremes, which
// a bitonic merge sorts.
template <int NL>
__device__ __forceinline__ void os_merge(OrderStats<NL> &o, int mask) {
  float bl[NL], bh[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) { bl[k] = __shfl_xor(o.lo[k], mask); bh[k] = __shfl_xor(o.hi[k], mask); }
#pragma unroll
  for (int k = 0; k < NL; ++k) { o.lo[k] = fminf(o.lo[k], bl[NL - 1 - k]); o.hi[k] = fmaxf(o.hi[k], bh[NL - 1 - k]); }
  constexpr int LOG = NL >= 8 ? 3 : (NL >= 4 ? 2 : (NL >= 2 ? 1 : 0));
#pragma unroll
  for (int ls = LOG - 1; ls >= 0; --ls)
#pragma unroll
    for (int k = 0; k < NL; ++k)
      if ((k & (1 << ls)) == 0) {
        const int st = 1 << ls;
        const float x = o.lo[k], y = o.lo[k + st];
        o.lo[k] = fminf(x, y); o.lo[k + st] = fmaxf(x, y);
        const float u = o.hi[k], v = o.hi[k + st];
        o.hi[k] = fmaxf(u, v); o.hi[k + st] = fminf(u, v);
      }
}

template <int NL>
__device__ __forceinline__ float pick(const float (&x)[NL > 0 ? NL : 1], int i) {
  // a select chain kept in registers (the empty asm stops it being turned into an
  // indexed scratch load)
  float r = x[0];
#pragma unroll
  for (int k = 1; k < NL; ++k) {
    float c = x[k];
    asm("" : "+v"(c));
    r = (i == k) ? c : r;
  }
  return r;
}

// (scale, zero) of a row before their fp16 rounding, from its merged order statistics:
// linear interpolation at virtual index (D-1)*pct/100 between sorted values.  Also the
// order statistics used: x0 <= x1 at the bottom, y0 >= y1 at the top.
struct AffPre {
  float vs, vz, x0, x1, y0, y1;
};

template <int D, int NL>
__device__ __forceinline__ AffPre affine_pre(const FlushArgs &a, const OrderStats<NL> &o, float ilm1) {
  AffPre p;
  p.x0 = pick<NL>(o.lo, a.lo_i);
  p.x1 = (a.lo_i + 1 < D) ? pick<NL>(o.lo, a.lo_i + 1) : p.x0;
  const float vlo = (a.lo_i + 1 < D) ? p.x0 + a.lo_t * (p.x1 - p.x0) : p.x0;
  const int hk = D - 1 - a.hi_i;
  p.y0 = pick<NL>(o.hi, hk);
  p.y1 = (hk >= 1) ? pick<NL>(o.hi, hk - 1) : p.y0;
  const float vhi = (a.hi_i + 1 < D) ? p.y0 + a.hi_t * (p.y1 - p.y0) : p.y0;
  p.vs = (vhi - vlo) * ilm1;   // ilm1 = 1 / (L - 1)
  p.vz = vlo;
  return p;
}

// The RMS step before its fp16 rounding, sqrt(ss) * fac with fac = 2 c / (sqrt(d) L)
// (rounded once, from fp64).  v_sqrt_f32 (1 ulp) and the product keep it within 3e-7 of
// the exact step, inside the parameter bands below.
__device__ __forceinline__ float quest_pre(float ss, float fac) { return __builtin_amdgcn_sqrtf(ss) * fac; }
__device__ __forceinline__ float quest_fac(float clip, int L, int D) {
  return (float)(2.0 * (double)clip / (sqrt((double)D) * (double)L));
}

// fp64 -> fp16, correctly rounded (to nearest, ties to even), returned as a float: round
// to fp32 toward zero and make it odd when inexact, then round to fp16.  fp32 carries 13
// more significand bits than fp16, so the two roundings give the single one.
__device__ __forceinline__ float f16_of_f64(double v) {
  float f = __double2float_rz(v);
  if ((double)f != v) f = __uint_as_float(__float_as_uint(f) | 1u);
  return (float)(_Float16)f;
}

// Whether an fp16 rounding boundary lies within eps (>= 0) of v: then the rounding of
// the exact value, which lies within eps of v, may differ from v's.
__device__ __forceinline__ bool near_mid(float v, float eps) {
  return (float)(_Float16)(v - eps) != (float)(_Float16)(v + eps);
}

__device__ __forceinline__ double quest_pre64(double ss, float clip, int L, int D) {
  return 2.0 * (double)clip * sqrt(ss / (double)D) / (double)L;
}

// The affine interpolation in fp64 from given order statistics (fp64 weights t of the
// percentiles' virtual indices): exactly the definition's arithmetic; the fp16
// parameters, and optionally their values before rounding.
template <int D>
__device__ __forceinline__ void affine_exact(const FlushArgs &a, double x0, double x1, double y0, double y1, int L,
                                             float &sc, float &zp, double *s64 = nullptr, double *z64 = nullptr) {
  const double lo = (a.lo_i + 1 < D) ? x0 + a.lo_t64 * (x1 - x0) : x0;
  const double hi = (a.hi_i + 1 < D) ? y0 + a.hi_t64 * (y1 - y0) : y0;
  const double s = (hi - lo) / (double)(L - 1);
  sc = f16_of_f64(s);
  zp = f16_of_f64(lo);
  if (s64) *s64 = s;
  if (z64) *z64 = lo;
}

// Exact code of a value known in fp64 (a zero step or scale gives the degenerate code).
__device__ __forceinline__ int exact_code(double x, float sc, float zp, int quant, int L) {
  if (sc == 0.f) return quant == WUSHKV_Q_QUEST ? L / 2 : 0;
  double t;
  if (quant == WUSHKV_Q_QUEST) t = floor(x / (double)sc + (double)(L / 2));
  else t = rint((x - (double)zp) / (double)sc);
  return (int)fmin(fmax(t, 0.0), (double)(L - 1));
}

// Quantizer of one row.  QuEST: code floor(x/step + L/2).  Affine: code
// rint((x - z)/s), half to even.  Codes are clamped to [0, L-1].  Both are taken as
// floor(v) of v = x/step + L/2 + tol, resp. (x - z)/s + 1/2 + tol: that equals the
// code unless the unshifted value lies within tol (bins) of a decision boundary,
// which is exactly when frac(v) < 2 tol.  The smallest frac(v) of each group of four
// elements is kept; the elements of groups that reach the band are decided again in fp64.  A zero step / scale gives the
// degenerate code (L/2, resp. 0) and no boundary.
template <bool QU>
struct Quant {
  float inv, add, z, top, band;
};

template <bool QU>
__device__ __forceinline__ Quant<QU> make_quant(float sc, float zp, int L, float tol) {
  Quant<QU> q;
  q.inv = sc != 0.f ? __builtin_amdgcn_rcpf(sc) : 0.f;   // 1 ulp: far inside the edge bands
  q.add = (QU ? (float)(L / 2) : 0.5f) + tol;
  q.z = zp;
  q.top = (float)(L - 1);
  q.band = 2.0f * tol;
  return q;
}

template <bool QU>
__device__ __forceinline__ float scaled(const Quant<QU> &q, float x) {
  return QU ? fmaf(x, q.inv, q.add) : fmaf(x - q.z, q.inv, q.add);
}

// Codes of two values; their fractions enter the row's minimum in one min3.
template <bool QU>
__device__ __forceinline__ void code2(const Quant<QU> &q, float x0, float x1, float &e, float &c0, float &c1) {
  const float v0 = scaled(q, x0), v1 = scaled(q, x1);
  const float f0 = floorf(v0), f1 = floorf(v1);
  e = fminf(fminf(e, v0 - f0), v1 - f1);
  c0 = __builtin_amdgcn_fmed3f(f0, 0.f, q.top);
  c1 = __builtin_amdgcn_fmed3f(f1, 0.f, q.top);
}

template <bool QU>
__device__ __forceinline__ bool edge_near(const Quant<QU> &q, float e) {
  return q.inv != 0.f && e < q.band;
}

// The same test for one value.
template <bool QU>
__device__ __forceinline__ bool value_near(const Quant<QU> &q, float x) {
  const float v = scaled(q, x);
  return v - floorf(v) < q.band;
}

// ---- exact key parameters for the rare rows near an fp16 rounding midpoint.  The whole
// workgroup works on one row at a time, after the step's tiles.

// The LDS copy of one fp16 key row (sm.krow, sm.kq): word c / 2 holds channels c and c + 1.
// Exact x_j = sum_i T[j][i] k[i] over 8-channel block blk of that row, in fp64 (fp16 x
// fp16 products are exact in fp32).
template <int D>
__device__ __forceinline__ double block_dot(const FlushSmem<D> &sm, int j, int blk) {
  const half8 tv = *(const half8 *)&sm.t[j][8 * blk];
  const u32x4 kw = *(const u32x4 *)&sm.krow[4 * blk];
  double x = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned w = kw[i >> 1];
    const float kv = (i & 1) ? (float)__builtin_bit_cast(f16x2, w)[1] : (float)__builtin_bit_cast(f16x2, w)[0];
    x += (double)((float)tv[i] * kv);
  }
  return x;
}

// Keep the NL smallest (ascending) or largest (descending) values seen.
template <int NL>
__device__ __forceinline__ void keep_low(double (&l)[NL], double v) {
#pragma unroll
  for (int k = NL - 1; k > 0; --k) l[k] = fmax(l[k - 1], fmin(l[k], v));
  l[0] = fmin(l[0], v);
}
template <int NL>
__device__ __forceinline__ void keep_high(double (&h)[NL], double v) {
#pragma unroll
  for (int k = NL - 1; k > 0; --k) h[k] = fmin(h[k - 1], fmax(h[k], v));
  h[0] = fmax(h[0], v);
}
template <int NL>
__device__ __forceinline__ double pick64(const double (&x)[NL], int i) {
  double r = x[0];
#pragma unroll
  for (int k = 1; k < NL; ++k) r = (i == k) ? x[k] : r;
  return r;
}

// Workgroup barrier that orders LDS only.  The flush's waves share nothing through
// global memory within a call (every code row, set word and parameter has one writer),
// so its barriers need not wait for the wave's global loads and stores: the next step's
// rows stay in flight across them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// DPP quad permutations (gfx9 quad_perm): lane i of a quad reads lane i^2 / i^1.
__device__ __forceinline__ unsigned quad_xor2(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);
}
__device__ __forceinline__ unsigned quad_xor1(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
}

// 4 x 4 byte transpose across a quad: lane e holds bytes [x_e0..x_e3] in, lane r
// holds [x_0r..x_3r] out (two exchanges: 16-bit halves with lane ^2, bytes with ^1).
__device__ __forceinline__ unsigned quad_transpose(unsigned x, unsigned selA, unsigned selB) {
  x = __builtin_amdgcn_perm(quad_xor2(x), x, selA);
  return __builtin_amdgcn_perm(quad_xor1(x), x, selB);
}

// 4 x 4 byte transpose across the lane groups q = lane / 16 of a token: lane q holds
// byte q of each of four dwords X_0..X_3 (its bytes 0..3 from X_0..X_3 of its own row
// position) in, and X_q's byte q' from lane q' out.  Two exchanges through gfx950's
// permlane swaps (16-bit halves with lane ^32, bytes with lane ^16), each of which hands
// a lane both values of its pair: (lower lane's x, upper lane's x).
__device__ __forceinline__ unsigned qgroup_transpose(unsigned x, int q) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const unsigned z = __builtin_amdgcn_perm(r[1], r[0], q < 2 ? 0x05040100u : 0x07060302u);
  const auto t = __builtin_amdgcn_permlane16_swap(z, z, false, false);
  return __builtin_amdgcn_perm(t[1], t[0], (q & 1) ? 0x07030501u : 0x06020400u);
}

// A 2-bit V set word's fields from one 16-token quarter, unshifted: a dword of 4 tokens'
// codes (bytes e = 0..3 of one channel, each 0..3) -> e0 at bits 0-1, e2 at 2-3, e1 at
// 16-17, e3 at 18-19 (the quarter's place in the word is a shift by 4 per quarter).
__device__ __forceinline__ unsigned vquarter2(unsigned x) {
  const unsigned hi = __builtin_amdgcn_perm(x, x, 0x0C030C02u);   // [e2, 0, e3, 0]
  const unsigned lo = __builtin_amdgcn_perm(x, x, 0x0C010C00u);   // [e0, 0, e1, 0]
  return (hi << 2) + lo;
}

// V set word fields from a dword of 4 tokens' codes (bytes e = 0..3 of one channel):
// low 2 bits of e at bit 4*(e>>1)... i.e. e0 -> 0, e2 -> 2, e1 -> 16, e3 -> 18.
__device__ __forceinline__ unsigned vfield2(unsigned x) {
  const unsigned m = x & 0x03030303u;
  const unsigned p = __builtin_amdgcn_perm(m, m, 0x03010200u);  // bytes [e0, e2, e1, e3]
  return (p | (p >> 6)) & 0x000F000Fu;
}
// Third bit (bit 2 of the code) of e at e0 -> 0, e2 -> 1, e1 -> 8, e3 -> 9.
__device__ __forceinline__ unsigned vfield1(unsigned x) {
  const unsigned n = (x >> 2) & 0x01010101u;
  const unsigned p = __builtin_amdgcn_perm(n, n, 0x03010200u);
  const unsigned y = (p | (p >> 7)) & 0x00030003u;
  return (y | (y >> 8)) & 0x0303u;
}
// K row packing: 4 consecutive channels' codes (bytes) -> 8 bits (2 bits each).
__device__ __forceinline__ unsigned kpack2(unsigned x) {
  const unsigned m = x & 0x03030303u;
  const unsigned y = (m | (m >> 6)) & 0x000F000Fu;
  return (y | (y >> 12)) & 0xFFu;
}
// ... bit 2 of each of 4 codes (channels 4e .. 4e + 3 of a 32-channel group) -> bits
// 0, 1, 4, 5: a 3-bit row's third-bit word holds channel f of its 32 at bit
// 4 ((f >> 1) & 7) + (f & 1) + 2 (f >> 4), so these land at 8 (e & 3) + 2 (e >> 2)
__device__ __forceinline__ unsigned kpack1(unsigned x) {
  const unsigned n = (x >> 2) & 0x01010101u;
  const unsigned y = (n | (n >> 7)) & 0x00030003u;
  return (y | (y >> 12)) & 0x33u;
}

// HAD: the key transform is T_K = a.had * H (Sylvester-Hadamard, H[j][i] = (-1)^popcount(i & j)),
// formed by butterflies in registers instead of the contraction; T_K itself is generated
// in LDS for the exact re-decisions.
// B2: 2-bit keys and values.  A lane packs its key codes in registers (four to a byte)
// and the token's four lanes exchange bytes into row order; value codes go to LDS as
// set-word fields of their 16-token quarter.  Otherwise codes go to LDS as bytes and
// the step's packing reads them back.
template <int D, int ES, int NL, bool PAGED, bool HAD, bool B2>
__global__ void __launch_bounds__(kThreads, 2) flush_kernel(FlushArgs a, int steps_per_wg) {
  constexpr int CPL = D / 4, KS = D / 32, NCT = D / 16;
  // word of the LDS key row (channel order) holding this lane's key word w
  auto kh_word = [](int q, int w) { return HAD ? 8 * (w >> 1) + 2 * q + (w & 1) : 16 * (w >> 2) + 4 * q + (w & 3); };
  // parameter bands of the key rows: the butterflies' seven fp32 roundings per element
  // get wider bands than the contraction's measured error
  constexpr float parKA = HAD ? 4e-6f : kParKA, parKB = HAD ? 1.5e-6f : kParKB;
  constexpr float parKAff = HAD ? 6e-6f : kParKAff, parKAff2 = HAD ? 4e-6f : kParKAff2;
  using QuestTag = std::integral_constant<bool, true>;
  using AffineTag = std::integral_constant<bool, false>;
  __shared__ FlushSmem<D> sm;
  if (a.append_x > 0 && (int)blockIdx.x >= (int)gridDim.x - a.append_x) {
    // fused window append (uniform counts; no flushed row comes from the ring)
    append_group(a, a.sink_k, a.sink_v, (_Float16 *)a.ring_k, (_Float16 *)a.ring_v, a.sink_bytes, blockIdx.y,
                 a.n_before, a.u1, (int64_t)(blockIdx.x - (gridDim.x - a.append_x)) * kThreads + threadIdx.x);
    return;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, tok = lane & 15;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int Lk = 1 << a.bits_k, Lv = 1 << a.bits_v;
  const float qfac_k = quest_fac(a.clip, Lk, D), qfac_v = quest_fac(a.clip, Lv, D);
  const float ilm1_k = (float)(1.0 / (double)(Lk - 1)), ilm1_v = (float)(1.0 / (double)(Lv - 1));
  // this sequence's rows before the call and its flushed body rows [u0, u1)
  const int64_t n_before = seq_before(a, b);
  if (n_before < 0) return;   // (device counts) out of range: the sequence is left alone
  const int64_t u0 = a.ragged ? n_quantized(n_before, a.S, a.R, a.C) : a.u0;
  const int64_t u1 = a.ragged ? n_quantized(n_before + a.n_new, a.S, a.R, a.C) : a.u1;
  const int64_t s_first = u0 / kSet, s_end = (u1 + kSet - 1) / kSet;
  const int64_t nsteps = u1 > u0 ? (s_end - s_first + 1) / 2 : 0;
  const int64_t st0 = (int64_t)blockIdx.x * steps_per_wg;
  const int64_t st1 = st0 + steps_per_wg < nsteps ? st0 + steps_per_wg : nsteps;
  if (st0 >= st1) return;   // (ragged batch) this sequence needs fewer steps, or none

  // Each tile's raw rows are refilled with the next step's as soon as they have been
  // converted, so every load has about a step of work to hide behind.
  RawSeg<ES, CPL> rk[2], rv[2];
  auto tok_of = [&](int64_t st, int tt) { return (s_first + 2 * st) * kSet + 32 * wave + 16 * tt + tok; };
  auto tok_valid = [&](int64_t u) { return u >= u0 && u < u1; };
  // rows of earlier calls come from the ring (fp16); invalid rows are converted as fp16
  auto tok_ring = [&](int64_t u) { return !tok_valid(u) || a.S + u < n_before; };
  // this KV head's ring and input rows
  const char *ring_kh = (const char *)a.ring_k + (size_t)bg * a.ring_bytes;
  const char *ring_vh = (const char *)a.ring_v + (size_t)bg * a.ring_bytes;
  const size_t in_off = (size_t)bg * (size_t)a.n_new * (D * ES);
  const char *in_kh = (const char *)a.k_new + in_off;
  const char *in_vh = (const char *)a.v_new + in_off;
  // Refill of a tile with step st's rows.  After the run's last step (st == st1) the
  // refill loads rows that are never used: as for invalid tokens, every lane then reads
  // the head's first input row (one cached row, no HBM traffic to speak of) with the
  // same load instructions, so the wave's load count stays uniform.
  auto load_k = [&](int64_t st, int tt) {
    const int64_t u = tok_of(st, tt);
    const bool valid = st < st1 && tok_valid(u);
    if constexpr (HAD) load_seg_ct<D, ES>(a, n_before, ring_kh, in_kh, u, valid, q, rk[tt]);
    else load_seg<D, ES>(a, n_before, ring_kh, in_kh, u, valid, q, rk[tt]);
  };
  auto load_v = [&](int64_t st, int tt) {
    const int64_t u = tok_of(st, tt);
    load_seg<D, ES>(a, n_before, ring_vh, in_vh, u, st < st1 && tok_valid(u), q, rv[tt]);
  };
  // the first step's rows, in flight while T_K is staged
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) { load_k(st0, tt); load_v(st0, tt); }
  if constexpr (HAD) {
    const _Float16 hp = (_Float16)a.had, hn = (_Float16)(-a.had);
    for (int i = tid; i < D * D; i += kThreads) {
      const int r = i / D, c = i % D;
      sm.t[r][c] = (__builtin_popcount(r & c) & 1) ? hn : hp;
    }
  } else {
    const _Float16 *T = a.tk + (size_t)g * D * D;
    for (int i = tid; i < D * D / 8; i += kThreads) {
      const int r = i / (D / 8), c8 = i % (D / 8);
      *(u32x4 *)&sm.t[r][8 * c8] = *(const u32x4 *)(T + (size_t)r * D + 8 * c8);
    }
  }
  // quad-transpose selectors of this lane (position e = tok & 3 in its quad)
  const unsigned selA = (tok & 2) ? 0x03020706u : 0x05040100u;
  const unsigned selB = (tok & 1) ? 0x03070105u : 0x06020400u;
  lds_barrier();

  for (int64_t st = st0; st < st1; ++st) {
    const int64_t set0 = s_first + 2 * st;
    const int64_t ubase = set0 * kSet + 32 * wave;   // this wave's first token
    // Key rows whose parameters need the exact x go to this wave's queue (want is the
    // same in a token's four lanes); the workgroup resolves them after the step's tiles.
    int ndq = 0;
    auto defer = [&](bool want, int row, const unsigned (&kh)[D / 8], unsigned cmask, float clo, float chi, float mg,
                     float sca, float zpa) {
      const unsigned tm = (unsigned)(__ballot(want) & 0xFFFFull);
      if (tm == 0) return;
      const int pos = ndq + __builtin_popcount(tm & ((1u << tok) - 1u));
      if (want) {
        DeferRow &d = sm.dq[wave][pos];
        d.cm[q] = cmask;
        if (q == 0) { d.row = row; d.clo = clo; d.chi = chi; d.mg = mg; d.sc = sca; d.zp = zpa; }
        if (pos < kStaged) {
#pragma unroll
          for (int w = 0; w < D / 8; ++w) sm.kq[wave][pos][kh_word(q, w)] = kh[w];
        }
      }
      ndq += __builtin_popcount(tm);
    };

    // ---- keys, one tile at a time: x = T_K k16 on MFMA, parameters, codes
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t u = ubase + 16 * tt + tok;
      const bool vt = tok_valid(u);
      if (!__any(vt)) {   // no row of this call's flush in the tile (a decode step's chunk, a call's edges)
        load_k(st + 1, tt);
        continue;
      }
      unsigned kh[CPL / 2];
      // rows of earlier calls (fp16, from the ring) in the tile: rare outside decode steps
      if (__builtin_expect(__any(vt && a.S + u < n_before), 0)) seg_half2<ES, CPL>(rk[tt], tok_ring(u), a.in_dtype, kh);
      else seg_half2<ES, CPL>(rk[tt], false, a.in_dtype, kh);   // (an invalid row's values are never used)
      load_k(st + 1, tt);
      f32x4 acc[NCT];
      if constexpr (HAD) {
        // x = a H k16 by butterflies: element (ct, i) of lane (q, tok) is channel 16 ct + 4 q
        // + i, so channel bits 0-1 pair elements of a chunk, bits 2-3 pair the token's lanes
        // (lane ^ 16, ^ 32), bits 4 and up pair chunks
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float k0 = f16_lo(kh[2 * ct]), k1 = f16_hi(kh[2 * ct]);
          const float k2 = f16_lo(kh[2 * ct + 1]), k3 = f16_hi(kh[2 * ct + 1]);
          const float a0 = k0 + k1, a1 = k0 - k1, a2 = k2 + k3, a3 = k2 - k3;
          acc[ct] = (f32x4){a0 + a2, a1 + a3, a0 - a2, a1 - a3};
        }
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
          const bool upper = (lane & m) != 0;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float o = __shfl_xor(acc[ct][i], m);
              acc[ct][i] = upper ? o - acc[ct][i] : acc[ct][i] + o;
            }
        }
#pragma unroll
        for (int m = 1; m < NCT; m <<= 1)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
            if (!(ct & m)) {
              const f32x4 x0 = acc[ct], x1 = acc[ct | m];
              acc[ct] = x0 + x1;
              acc[ct | m] = x0 - x1;
            }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] *= a.had;
      } else {
        // K-steps outer, tiles inner: NCT independent accumulation chains
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 bw = {kh[4 * s], kh[4 * s + 1], kh[4 * s + 2], kh[4 * s + 3]};
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const half8 A = *(const half8 *)&sm.t[16 * ct + tok][32 * s + 8 * q];
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8, bw), acc[ct], 0, 0, 0);
          }
        }
      }
      const int row = 32 * wave + 16 * tt + tok;
      auto key_tile = [&](auto tag) {
        constexpr bool QU = decltype(tag)::value;
        float sc, zp = 0.f;
        bool kdef = false;   // queued for exact parameters: the queue stores them
        if constexpr (QU) {
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = fmaf(acc[ct][i], acc[ct][i], s4[i]);
          float ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          ss = pair_sum<32>(pair_sum<16>(ss));
          const float v32 = quest_pre(ss, qfac_k);
          sc = f16_round(v32);
          // a step near an fp16 rounding midpoint is decided again: from the fp64 sum of
          // squares of the fp32 x, then, if still near one, from the exact x
          const bool pn = vt && near_mid(v32, parKA * v32);
          if (__builtin_expect(__any(pn), 0)) {
            double s64 = 0.0;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
              for (int i = 0; i < 4; ++i) s64 = fma((double)acc[ct][i], (double)acc[ct][i], s64);
            s64 += __shfl_xor(s64, 16);
            s64 += __shfl_xor(s64, 32);
            const double d64 = quest_pre64(s64, a.clip, Lk, D);
            if (pn) sc = f16_of_f64(d64);
            // still near one: the exact x after the step's tiles
            kdef = pn && near_mid((float)d64, parKB * (float)d64);
            defer(kdef, row, kh, 0u, 0.f, 0.f, 0.f, sc, 0.f);
          }
        } else if constexpr (NL > 0) {
          OrderStats<NL> o;
          os_init(o);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) os_insert(o, acc[ct][i]);
          os_merge(o, 16);
          os_merge(o, 32);
          const AffPre ap = affine_pre<D, NL>(a, o, ilm1_k);
          sc = f16_round(ap.vs);
          zp = f16_round(ap.vz);
          // scale or zero near an fp16 rounding midpoint: decided again from the fp64
          // interpolation of the order statistics, and if still near one, from the exact x
          // after the step's tiles
          const float sx = fabsf(ap.x0) + fabsf(ap.x1), sxy = sx + fabsf(ap.y0) + fabsf(ap.y1);
          const bool pn = vt && (near_mid(ap.vz, parKAff * sx) || near_mid(ap.vs, parKAff * sxy * ilm1_k));
          if (__builtin_expect(__any(pn), 0)) {
            double s64, z64;
            float sc1, zp1;
            affine_exact<D>(a, ap.x0, ap.x1, ap.y0, ap.y1, Lk, sc1, zp1, &s64, &z64);
            if (pn) { sc = sc1; zp = zp1; }
            const bool pn2 = pn && (near_mid((float)z64, parKAff2 * sx) ||
                                    near_mid((float)s64, parKAff2 * sxy * ilm1_k));
            // candidates for the exact order statistics: this lane's elements within mg of the
            // cuts (the contraction's error is far below mg)
            const float cut_lo = fmaxf(ap.x0, ap.x1), cut_hi = fminf(ap.y0, ap.y1);
            const float mg = 8e-6f * fmaxf(fabsf(cut_lo), fabsf(cut_hi));
            unsigned cmask = 0;
            if (pn2) {
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (acc[ct][i] <= cut_lo + mg || acc[ct][i] >= cut_hi - mg) cmask |= 1u << (4 * ct + i);
            }
            kdef = pn2;
            defer(pn2, row, kh, cmask, cut_lo, cut_hi, mg, sc, zp);
          }
        } else {
          sc = 0.f;
        }
        if (q == 0 && vt && !kdef) {
          const int64_t off = body_offset<PAGED>(a.pg, a.Hkv, a.body_cap, b, g, u, 2 * a.kpar_n);
          _Float16 *pk = (_Float16 *)((char *)a.par_k + off);
          if (PAGED && off < 0) {
          } else if constexpr (QU) {
            pk[0] = (_Float16)sc;
          } else {
            *(unsigned *)pk = pack_f16(sc, zp);
          }
        }
        const Quant<QU> qk = make_quant<QU>(sc, zp, Lk, kEdgeK * (float)Lk * (1.0f / 16.0f));
        float e[NCT];   // per group of 4 elements, so a recheck visits only the near groups
        // B2: byte ct % 4 of word ct / 4 packs out channels 16 ct + 4 q .. 16 ct + 4 q + 3
        unsigned kpk[B2 ? NCT / 4 : 1];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float c0, c1, c2, c3;
          e[ct] = 1.0f;
          code2(qk, acc[ct][0], acc[ct][1], e[ct], c0, c1);
          code2(qk, acc[ct][2], acc[ct][3], e[ct], c2, c3);
          if constexpr (B2) {
            // four 2-bit codes as one byte, exact in fp32
            const float byte = fmaf(fmaf(fmaf(c3, 4.f, c2), 4.f, c1), 4.f, c0);
            kpk[ct >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(byte, ct & 3, (ct & 3) ? kpk[ct >> 2] : 0u);
          } else {
            unsigned w = __builtin_amdgcn_cvt_pk_u8_f32(c0, 0, 0u);
            w = __builtin_amdgcn_cvt_pk_u8_f32(c1, 1, w);
            w = __builtin_amdgcn_cvt_pk_u8_f32(c2, 2, w);
            w = __builtin_amdgcn_cvt_pk_u8_f32(c3, 3, w);
            *(unsigned *)&sm.kc[row][16 * ct + 4 * q] = w;
          }
        }
        // elements near a boundary: the 4 lanes of a token take one candidate at a
        // time, each summing its CPL channels' exact products in fp64
        float emin = e[0];
#pragma unroll
        for (int ct = 1; ct < NCT; ++ct) emin = fminf(emin, e[ct]);
        const bool kn = vt && edge_near(qk, emin);
        if (__builtin_expect(__any(kn), 0)) {
          unsigned m = 0;
          if (kn) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
              if (e[ct] < qk.band) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (value_near(qk, acc[ct][i])) m |= 1u << (4 * ct + i);
              }
          }
          while (__any(m != 0)) {
            const unsigned m0 = __shfl(m, tok), m1 = __shfl(m, 16 + tok), m2 = __shfl(m, 32 + tok), m3 = __shfl(m, 48 + tok);
            const int qs = m0 ? 0 : (m1 ? 1 : (m2 ? 2 : (m3 ? 3 : -1)));
            const unsigned mm = qs == 0 ? m0 : (qs == 1 ? m1 : (qs == 2 ? m2 : m3));
            const int bit = qs >= 0 ? __builtin_ctz(mm) : 0;
            const int j = 16 * (bit >> 2) + 4 * (qs >= 0 ? qs : 0) + (bit & 3);
            double part = 0.0;
#pragma unroll
            for (int w = 0; w < CPL / 2; ++w) {   // the lane's channels, two per key word
              const int c0 = 2 * kh_word(q, w);
              const f16x2 tv = *(const f16x2 *)&sm.t[j][c0];
              part += (double)((float)tv[0] * f16_lo(kh[w]));   // fp16 x fp16 is exact in fp32
              part += (double)((float)tv[1] * f16_hi(kh[w]));
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            if (qs == q) {
              const int code = exact_code(part, sc, zp, QU ? WUSHKV_Q_QUEST : WUSHKV_Q_AFFINE_PCT, Lk);
              if constexpr (B2) {
                const int sh = 8 * ((bit >> 2) & 3) + 2 * (bit & 3);
#pragma unroll
                for (int kk = 0; kk < NCT / 4; ++kk)
                  if (kk == bit >> 4) kpk[kk] = (kpk[kk] & ~(3u << sh)) | ((unsigned)code << sh);
              } else {
                sm.kc[row][j] = (uint8_t)code;
              }
              m &= ~(1u << bit);
            }
          }
        }
        if constexpr (B2) {
          // lane q now writes words q, q + 4, ... of the token's packed row
#pragma unroll
          for (int kk = 0; kk < NCT / 4; ++kk) sm.kp[row][4 * kk + q] = qgroup_transpose(kpk[kk], q);
        }
      };
      if (a.quant_k == WUSHKV_Q_QUEST) key_tile(QuestTag{});
      else key_tile(AffineTag{});
    }

    // ---- values
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t u = ubase + 16 * tt + tok;
      const bool vt = tok_valid(u);
      const int s2 = wave >> 1;                       // set of this wave within the step
      const int col = 32 * (wave & 1) + 16 * tt;      // first token of the tile in its set
      if (!__any(vt)) {
        load_v(st + 1, tt);
        if constexpr (B2) {
          // the quarter's words are OR-ed into whole set words, so they must hold fields
          // only: zero codes (the set's merge keeps the stored fields of these tokens)
#pragma unroll
          for (int g4 = 0; g4 < CPL / 4; ++g4) {
            const int j = seg_chan(q, 4 * g4 + (tok & 3));
            sm.vw[s2][col >> 4][(16 * (tok >> 2) + (j & 15)) * (D / 16) + (j >> 4)] = 0u;
          }
        }
        continue;
      }
      float xv[CPL];
      if (__builtin_expect(__any(vt && a.S + u < n_before), 0)) seg_float<ES, CPL>(rv[tt], tok_ring(u), a.in_dtype, xv);
      else seg_float<ES, CPL>(rv[tt], false, a.in_dtype, xv);
      load_v(st + 1, tt);
      auto value_tile = [&](auto tag) {
        constexpr bool QU = decltype(tag)::value;
        float sc, zp = 0.f;
        if constexpr (QU) {
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < CPL; ++k) s4[k & 3] = fmaf(xv[k], xv[k], s4[k & 3]);
          float ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          ss = pair_sum<32>(pair_sum<16>(ss));
          const float v32 = quest_pre(ss, qfac_v);
          sc = f16_round(v32);
          // near an fp16 rounding midpoint: the step from the exact (fp64) sum of squares
          const bool pn = vt && near_mid(v32, kParV * v32);
          if (__builtin_expect(__any(pn), 0)) {
            double s64 = 0.0;
#pragma unroll
            for (int k = 0; k < CPL; ++k) s64 = fma((double)xv[k], (double)xv[k], s64);
            s64 += __shfl_xor(s64, 16);
            s64 += __shfl_xor(s64, 32);
            if (pn) sc = f16_of_f64(quest_pre64(s64, a.clip, Lv, D));
          }
        } else if constexpr (NL > 0) {
          OrderStats<NL> o;
          os_init(o);
#pragma unroll
          for (int k = 0; k < CPL; ++k) os_insert(o, xv[k]);
          os_merge(o, 16);
          os_merge(o, 32);
          const AffPre ap = affine_pre<D, NL>(a, o, ilm1_v);
          sc = f16_round(ap.vs);
          zp = f16_round(ap.vz);
          // near an fp16 rounding midpoint: the interpolation in fp64 (the order statistics
          // of values are exact)
          const float ez = kParV * (fabsf(ap.x0) + fabsf(ap.x1));
          const float es = kParV * (fabsf(ap.x0) + fabsf(ap.x1) + fabsf(ap.y0) + fabsf(ap.y1)) * ilm1_v;
          if (__builtin_expect(vt && (near_mid(ap.vz, ez) || near_mid(ap.vs, es)), 0))
            affine_exact<D>(a, ap.x0, ap.x1, ap.y0, ap.y1, Lv, sc, zp);
        } else {
          sc = 0.f;
        }
        if (q == 0 && vt) {
          const int64_t off = body_offset<PAGED>(a.pg, a.Hkv, a.body_cap, b, g, u, 2 * a.vpar_n);
          _Float16 *pv = (_Float16 *)((char *)a.par_v + off);
          if (PAGED && off < 0) {
          } else if constexpr (QU) {
            pv[0] = (_Float16)sc;
          } else {
            *(unsigned *)pv = pack_f16(sc, zp);
          }
        }
        const Quant<QU> qv = make_quant<QU>(sc, zp, Lv, kEdgeV);
        float e[CPL / 4];   // per group of 4 elements, as for the keys
#pragma unroll
        for (int g4 = 0; g4 < CPL / 4; ++g4) {
          float c0, c1, c2, c3;
          e[g4] = 1.0f;
          code2(qv, xv[4 * g4], xv[4 * g4 + 1], e[g4], c0, c1);
          code2(qv, xv[4 * g4 + 2], xv[4 * g4 + 3], e[g4], c2, c3);
          unsigned w = __builtin_amdgcn_cvt_pk_u8_f32(c0, 0, 0u);
          w = __builtin_amdgcn_cvt_pk_u8_f32(c1, 1, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(c2, 2, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(c3, 3, w);
          // lane tok = 4c + e now gets channel 4*g4 + e of tokens 4c .. 4c+3
          w = quad_transpose(w, selA, selB);
          if constexpr (B2) {
            // the fields of set word (16 c + j % 16, j / 16) from this quarter
            const int j = seg_chan(q, 4 * g4 + (tok & 3));
            sm.vw[s2][col >> 4][(16 * (tok >> 2) + (j & 15)) * (D / 16) + (j >> 4)] = vquarter2(w);
          } else {
            *(unsigned *)&sm.vc[s2][seg_chan(q, 4 * g4 + (tok & 3))][col + 4 * (tok >> 2)] = w;
          }
        }
        float emin = e[0];
#pragma unroll
        for (int g4 = 1; g4 < CPL / 4; ++g4) emin = fminf(emin, e[g4]);
        const bool vn = vt && edge_near(qv, emin);
        if (__builtin_expect(__any(vn), 0)) {
          unsigned m = 0;
          if (vn) {
#pragma unroll
            for (int g4 = 0; g4 < CPL / 4; ++g4)
              if (e[g4] < qv.band) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (value_near(qv, xv[4 * g4 + i])) m |= 1u << (4 * g4 + i);
              }
          }
          // one near element per pass (a rolled loop keeps this rare path small)
          while (m != 0) {
            const int k = __builtin_ctz(m);
            m &= m - 1;
            const int code =
                exact_code((double)pick<CPL>(xv, k), sc, zp, QU ? WUSHKV_Q_QUEST : WUSHKV_Q_AFFINE_PCT, Lv);
            if constexpr (B2) {
              // this token's field of its set word (other lanes may patch the same word)
              const int j = seg_chan(q, k);
              const int sh = ((tok & 1) ? 16 : 0) + ((tok & 2) ? 2 : 0);
              unsigned *wp = &sm.vw[s2][col >> 4][(16 * (tok >> 2) + (j & 15)) * (D / 16) + (j >> 4)];
              atomicAnd(wp, ~(3u << sh));
              atomicOr(wp, (unsigned)code << sh);
            } else {
              sm.vc[s2][seg_chan(q, k)][col + tok] = (uint8_t)code;
            }
          }
        }
      };
      if (a.quant_v == WUSHKV_Q_QUEST) value_tile(QuestTag{});
      else value_tile(AffineTag{});
    }
    // ---- the queued key rows, resolved by the whole workgroup after the step's tiles.  A
    // row's fp16 key is in LDS (staged when it was queued, else read again from the ring or
    // the input).  Affine rows first get the exact values of their candidate elements (16
    // lanes per candidate, one pass); a row whose parameters change, and every QuEST row,
    // gets the exact x of all channels (thread group of channel j: x_j in fp64), its exact
    // parameters and the codes of its exact x.
    if (lane == 0) sm.dqn[wave] = ndq;
    lds_barrier();
    const int nq0 = sm.dqn[0], nq1 = sm.dqn[1], nq2 = sm.dqn[2], nq3 = sm.dqn[3];
    if (__builtin_expect(nq0 + nq1 + nq2 + nq3 > 0, 0)) {
      auto key_row8 = [&](int64_t u, int m) -> u32x4 {
        if (a.S + u < n_before) {
          const unsigned slot = (unsigned)u % (unsigned)(a.R + a.C);
          return *(const u32x4 *)(ring_kh + (size_t)slot * (D * 2) + 16 * m);
        }
        const char *src = in_kh + (size_t)(a.S + u - n_before) * (D * ES) + (size_t)8 * ES * m;
        if constexpr (ES == 2) {
          const u32x4 w = *(const u32x4 *)src;
          if (a.in_dtype == WUSHKV_DT_F16) return w;
          return (u32x4){pack_f16(bf16_lo(w[0]), bf16_hi(w[0])), pack_f16(bf16_lo(w[1]), bf16_hi(w[1])),
                         pack_f16(bf16_lo(w[2]), bf16_hi(w[2])), pack_f16(bf16_lo(w[3]), bf16_hi(w[3]))};
        } else {
          const u32x4 w0 = *(const u32x4 *)src, w1 = *(const u32x4 *)(src + 16);
          return (u32x4){pack_f16(__uint_as_float(w0[0]), __uint_as_float(w0[1])),
                         pack_f16(__uint_as_float(w0[2]), __uint_as_float(w0[3])),
                         pack_f16(__uint_as_float(w1[0]), __uint_as_float(w1[1])),
                         pack_f16(__uint_as_float(w1[2]), __uint_as_float(w1[3]))};
        }
      };
      constexpr int TPC = kThreads / D;         // threads per channel: 2 (D = 128) or 4 (D = 64)
      constexpr int BPT = D / 8 / TPC;          // 8-channel blocks per thread
      const int j = tid / TPC, h = tid % TPC;
#pragma unroll 1
      for (int wv = 0; wv < 4; ++wv) {
        const int nqw = wv == 0 ? nq0 : (wv == 1 ? nq1 : (wv == 2 ? nq2 : nq3));
#pragma unroll 1
        for (int e = 0; e < nqw; ++e) {
          const DeferRow &d = sm.dq[wv][e];
          const int row = d.row;
          const int64_t u = set0 * kSet + row;
          if (e < kStaged) {
            if (tid < D / 2) sm.krow[tid] = sm.kq[wv][e][tid];
          } else if (tid < D / 8) {
            *(u32x4 *)&sm.krow[4 * tid] = key_row8(u, tid);
          }
          lds_barrier();
          float scx = d.sc, zpx = d.zp;
          bool full = a.quant_k == WUSHKV_Q_QUEST;
          int total = 0;
          if constexpr (NL > 0) {
            if (!full) {
              const unsigned cm[4] = {d.cm[0], d.cm[1], d.cm[2], d.cm[3]};
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) total += __builtin_popcount(cm[qq]);
              if (total > kMaxCand) {
                full = true;
              } else {
                // candidate c = tid / 16, its 16 lanes one 8-channel block each
                const int c = tid >> 4, m = tid & 15;
                int left = c, jc = 0;
                bool found = false;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                  const int cnt = __builtin_popcount(cm[qq]);
                  if (!found && left < cnt) {
                    unsigned mm = cm[qq];
                    for (int s2 = 0; s2 < left; ++s2) mm &= mm - 1;
                    const int bit = __builtin_ctz(mm);
                    jc = 16 * (bit >> 2) + 4 * qq + (bit & 3);
                    found = true;
                  } else if (!found) {
                    left -= cnt;
                  }
                }
                double part = (found && m < D / 8) ? block_dot<D>(sm, jc, m) : 0.0;
#pragma unroll
                for (int sh = 1; sh < 16; sh <<= 1) part += __shfl_xor(part, sh);
                if (m == 0 && found) sm.cand[c] = part;
                lds_barrier();
                double lo_s[NL], hi_s[NL];
#pragma unroll
                for (int k = 0; k < NL; ++k) { lo_s[k] = INFINITY; hi_s[k] = -INFINITY; }
#pragma unroll 1
                for (int cc = 0; cc < total; ++cc) {
                  const double v = sm.cand[cc];
                  if (v <= (double)(d.clo + d.mg)) keep_low<NL>(lo_s, v);
                  if (v >= (double)(d.chi - d.mg)) keep_high<NL>(hi_s, v);
                }
                const double x0 = pick64<NL>(lo_s, a.lo_i);
                const double x1 = (a.lo_i + 1 < D) ? pick64<NL>(lo_s, a.lo_i + 1) : x0;
                const int hk = D - 1 - a.hi_i;
                const double y0 = pick64<NL>(hi_s, hk);
                const double y1 = (hk >= 1) ? pick64<NL>(hi_s, hk - 1) : y0;
                affine_exact<D>(a, x0, x1, y0, y1, Lk, scx, zpx);
                full = scx != d.sc || zpx != d.zp;   // the codes follow the new parameters
              }
            }
          }
          if (full) {
            double xa = 0.0, xb = 0.0;   // two independent chains
#pragma unroll 2
            for (int k2 = 0; k2 < BPT; k2 += 2) {
              xa += block_dot<D>(sm, j, h * BPT + k2);
              xb += block_dot<D>(sm, j, h * BPT + k2 + 1);
            }
            double x = xa + xb;
#pragma unroll
            for (int sh = 1; sh < TPC; sh <<= 1) x += __shfl_xor(x, sh);   // every thread of channel j: x_j
            if (a.quant_k == WUSHKV_Q_QUEST) {
              // sum of squares: each channel counted TPC times (an exact scaling), waves in order
              double ss = x * x;
#pragma unroll
              for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m);
              if (lane == 0) sm.red[wave][0] = ss;
              lds_barrier();
              ss = ((sm.red[0][0] + sm.red[1][0]) + (sm.red[2][0] + sm.red[3][0])) / (double)TPC;
              scx = f16_of_f64(quest_pre64(ss, a.clip, Lk, D));
            } else if constexpr (NL > 0) {
              if (total > kMaxCand) {
                // the NL smallest and largest exact values of all channels: per wave (one
                // thread per channel), then over the four waves' lists
                double lo_s[NL], hi_s[NL];
#pragma unroll
                for (int k = 0; k < NL; ++k) { lo_s[k] = INFINITY; hi_s[k] = -INFINITY; }
                if (h == 0) { lo_s[0] = x; hi_s[0] = x; }
#pragma unroll 1
                for (int m = 1; m < 64; m <<= 1) {
                  double ol[NL], oh[NL];
#pragma unroll
                  for (int k = 0; k < NL; ++k) { ol[k] = __shfl_xor(lo_s[k], m); oh[k] = __shfl_xor(hi_s[k], m); }
#pragma unroll
                  for (int k = 0; k < NL; ++k) { keep_low<NL>(lo_s, ol[k]); keep_high<NL>(hi_s, oh[k]); }
                }
                if (lane == 0) {
#pragma unroll
                  for (int k = 0; k < NL; ++k) { sm.red[wave][k] = lo_s[k]; sm.red[wave][NL + k] = hi_s[k]; }
                }
                lds_barrier();
#pragma unroll
                for (int k = 0; k < NL; ++k) { lo_s[k] = INFINITY; hi_s[k] = -INFINITY; }
#pragma unroll
                for (int wv2 = 0; wv2 < 4; ++wv2)
#pragma unroll
                  for (int k = 0; k < NL; ++k) {
                    keep_low<NL>(lo_s, sm.red[wv2][k]);
                    keep_high<NL>(hi_s, sm.red[wv2][NL + k]);
                  }
                const double x0 = pick64<NL>(lo_s, a.lo_i);
                const double x1 = (a.lo_i + 1 < D) ? pick64<NL>(lo_s, a.lo_i + 1) : x0;
                const int hk = D - 1 - a.hi_i;
                const double y0 = pick64<NL>(hi_s, hk);
                const double y1 = (hk >= 1) ? pick64<NL>(hi_s, hk - 1) : y0;
                affine_exact<D>(a, x0, x1, y0, y1, Lk, scx, zpx);
              }
            }
            if (h == 0) {
              const int code = exact_code(x, scx, zpx, a.quant_k, Lk);
              if constexpr (B2) {
                const int sh = 2 * (j & 15);
                atomicAnd(&sm.kp[row][j >> 4], ~(3u << sh));
                atomicOr(&sm.kp[row][j >> 4], (unsigned)code << sh);
              } else {
                sm.kc[row][j] = (uint8_t)code;
              }
            }
          }
          const int64_t off = body_offset<PAGED>(a.pg, a.Hkv, a.body_cap, b, g, u, 2 * a.kpar_n);
          if (tid == 0 && !(PAGED && off < 0)) {
            _Float16 *pk = (_Float16 *)((char *)a.par_k + off);
            if (a.quant_k == WUSHKV_Q_QUEST) pk[0] = (_Float16)scx;
            else *(unsigned *)pk = pack_f16(scx, zpx);
          }
          lds_barrier();
        }
      }
    }
    // ---- K rows: two threads per token, D/2 channels each (the bit width is a
    // template argument so only its own packing is issued)
    auto pack_k_rows = [&](auto bits_tag) {
      constexpr int BK = decltype(bits_tag)::value;
      const int r = tid >> 1, h = tid & 1;
      const int64_t u = set0 * kSet + r;
      if (u < u0 || u >= u1) return;
      constexpr int HC = D / 2;
      const int64_t koff = body_offset<PAGED>(a.pg, a.Hkv, a.body_cap, b, g, u, (int64_t)a.kcode_row);
      if (PAGED && koff < 0) return;   // the row's page is outside the table or the pool
      uint8_t *rowp = a.codes_k + koff;
      u32x4 cw[HC / 16];
#pragma unroll
      for (int i = 0; i < HC / 16; ++i) cw[i] = *(const u32x4 *)&sm.kc[r][HC * h + 16 * i];
      unsigned p0[HC / 16];
#pragma unroll
      for (int k = 0; k < HC / 16; ++k)
        p0[k] = kpack2(cw[k][0]) | (kpack2(cw[k][1]) << 8) | (kpack2(cw[k][2]) << 16) | (kpack2(cw[k][3]) << 24);
      if constexpr (HC / 16 == 4) *(u32x4 *)(rowp + 16 * h) = (u32x4){p0[0], p0[1], p0[2], p0[3]};
      else *(u32x2 *)(rowp + 8 * h) = (u32x2){p0[0], p0[1]};
      if constexpr (BK == 3) {
        unsigned p1[HC / 32];
#pragma unroll
        for (int k = 0; k < HC / 32; ++k) {
          unsigned w = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) w |= kpack1(cw[2 * k + e / 4][e % 4]) << (8 * (e & 3) + 2 * (e >> 2));
          p1[k] = w;
        }
        if constexpr (HC / 32 == 2) *(u32x2 *)(rowp + D / 4 + 8 * h) = (u32x2){p1[0], p1[1]};
        else *(unsigned *)(rowp + D / 4 + 4 * h) = p1[0];
      } else if constexpr (BK == 4) {
#pragma unroll
        for (int k = 0; k < HC / 16; ++k)
          p0[k] = kpack2(cw[k][0] >> 2) | (kpack2(cw[k][1] >> 2) << 8) | (kpack2(cw[k][2] >> 2) << 16) |
                  (kpack2(cw[k][3] >> 2) << 24);
        if constexpr (HC / 16 == 4) *(u32x4 *)(rowp + D / 4 + 16 * h) = (u32x4){p0[0], p0[1], p0[2], p0[3]};
        else *(u32x2 *)(rowp + D / 4 + 8 * h) = (u32x2){p0[0], p0[1]};
      }
    };
    using Bits2 = std::integral_constant<int, 2>;
    using Bits3 = std::integral_constant<int, 3>;
    using Bits4 = std::integral_constant<int, 4>;
    if constexpr (B2) {
      // packed rows: a copy, two threads per row
      const int r = tid >> 1, h = tid & 1;
      const int64_t u = set0 * kSet + r;
      const int64_t koff = (u >= u0 && u < u1) ? body_offset<PAGED>(a.pg, a.Hkv, a.body_cap, b, g, u, (int64_t)a.kcode_row)
                                               : -1;
      if (koff >= 0) {
        uint8_t *rowp = a.codes_k + koff;
        if constexpr (D == 128) *(u32x4 *)(rowp + 16 * h) = *(const u32x4 *)&sm.kp[r][4 * h];
        else *(u32x2 *)(rowp + 8 * h) = *(const u32x2 *)&sm.kp[r][2 * h];
      }
    } else {
      if (a.bits_k == 2) pack_k_rows(Bits2{});
      else if (a.bits_k == 3) pack_k_rows(Bits3{});
      else pack_k_rows(Bits4{});
    }

    // ---- V set words: 128 threads per set, 4 consecutive words each.  A set only
    // partly covered by this call keeps its other tokens' fields.
    constexpr int NT = D / 16, NW = 64 * NT;
    const int s2 = tid >> 7, t128 = tid & 127;
    const int64_t sidx = set0 + s2;
    const int64_t vbase = sidx * kSet;
    const int64_t vlo = u0 > vbase ? u0 : vbase;
    const int64_t vhi = u1 < vbase + kSet ? u1 : vbase + kSet;
    auto pack_v_words = [&](auto bits_tag, auto full_tag) {
      constexpr int BVV = decltype(bits_tag)::value;
      constexpr bool FULL = decltype(full_tag)::value;
      const int r0 = (int)(vlo - vbase), r1 = (int)(vhi - vbase);
      const int64_t voff = body_offset<PAGED>(a.pg, a.Hkv, a.body_cap, b, g, vbase, (int64_t)(a.vset_bytes / kSet));
      if (PAGED && voff < 0) return;   // the set's page is outside the table or the pool
      uint8_t *vb = a.codes_v + voff;
      unsigned w0[4], w1[4], k0[4], k1[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int wi = 4 * t128 + jj;
        const int ln = wi / NT, t = wi % NT;
        const int c = ln >> 4, j = 16 * t + (ln & 15);
        w0[jj] = w1[jj] = k0[jj] = k1[jj] = 0u;
        if constexpr (B2)   // the four quarters' fields, each shifted to its place
          w0[jj] = sm.vw[s2][0][wi] | (sm.vw[s2][1][wi] << 4) | (sm.vw[s2][2][wi] << 8) | (sm.vw[s2][3][wi] << 12);
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          if constexpr (!B2) {
            const unsigned x = *(const unsigned *)&sm.vc[s2][j][16 * aa + 4 * c];
            w0[jj] |= vfield2(x) << (4 * aa);
            if constexpr (BVV == 3) w1[jj] |= vfield1(x) << (2 * aa);
            if constexpr (BVV == 4) w1[jj] |= vfield2(x >> 2) << (4 * aa);
          }
          if constexpr (!FULL) {
            unsigned vm = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rr = 16 * aa + 4 * c + e;
              if (rr >= r0 && rr < r1) vm |= 0x0Fu << (8 * e);
            }
            k0[jj] |= vfield2(vm) << (4 * aa);
            if constexpr (BVV == 3) k1[jj] |= vfield1(vm) << (2 * aa);
            if constexpr (BVV == 4) k1[jj] |= vfield2(vm >> 2) << (4 * aa);
          }
        }
      }
      u32x4 *p0 = (u32x4 *)(vb + 16 * t128);
      if constexpr (FULL) {
        *p0 = (u32x4){w0[0], w0[1], w0[2], w0[3]};
      } else {
        u32x4 old = *p0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) old[jj] = (old[jj] & ~k0[jj]) | (w0[jj] & k0[jj]);
        *p0 = old;
      }
      if constexpr (BVV == 3) {
        u32x2 *p1 = (u32x2 *)(vb + 4 * NW + 8 * t128);
        u32x2 nw = {w1[0] | (w1[1] << 16), w1[2] | (w1[3] << 16)};
        if constexpr (!FULL) {
          const u32x2 mk = {k1[0] | (k1[1] << 16), k1[2] | (k1[3] << 16)};
          const u32x2 old = *p1;
          nw = (old & ~mk) | (nw & mk);
        }
        *p1 = nw;
      } else if constexpr (BVV == 4) {
        u32x4 *p1 = (u32x4 *)(vb + 4 * NW + 16 * t128);
        u32x4 nw = {w1[0], w1[1], w1[2], w1[3]};
        if constexpr (!FULL) {
          const u32x4 old = *p1;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) nw[jj] = (old[jj] & ~k1[jj]) | (nw[jj] & k1[jj]);
        }
        *p1 = nw;
      }
    };
    if (vlo < vhi && 4 * t128 < NW) {
      using Full = std::integral_constant<bool, true>;
      using Part = std::integral_constant<bool, false>;
      const bool full = vlo == vbase && vhi == vbase + kSet;
      if constexpr (B2) {
        if (full) pack_v_words(Bits2{}, Full{});
        else pack_v_words(Bits2{}, Part{});
      } else if (full) {
        if (a.bits_v == 2) pack_v_words(Bits2{}, Full{});
        else if (a.bits_v == 3) pack_v_words(Bits3{}, Full{});
        else pack_v_words(Bits4{}, Full{});
      } else {
        if (a.bits_v == 2) pack_v_words(Bits2{}, Part{});
        else if (a.bits_v == 3) pack_v_words(Bits3{}, Part{});
        else pack_v_words(Bits4{}, Part{});
      }
    }
    lds_barrier();
  }
}

}  // namespace

// Workgroups of the window append for a uniform call (0 if it writes no window row).
int append_workgroups(int64_t n_before, int64_t n_new, int64_t q_after, int S, int d) {
  int64_t ns, tr;
  const int64_t most = window_tokens(n_before, n_new, q_after, S, ns, tr);
  return (int)((most * (d / 8) + kThreads - 1) / kThreads);
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  // window tokens of the sequence with the most: exact for host counts; device counts
  // are unknown here, and a sequence never has more than S + R + C - 1 (the sink, and
  // a ring that holds fewer than R + C after its flush)
  int64_t most = 0, ns, tr;
  if (a.ragged == kRaggedDevice) {
    most = a.n_new < (int64_t)a.S + a.R + a.C ? a.n_new : (int64_t)a.S + a.R + a.C;
  } else if (a.ragged == kRaggedHost) {
    for (int b = 0; b < a.B; ++b) {
      const int64_t nb = a.seq_nb[b];
      const int64_t w = window_tokens(nb, a.n_new, n_quantized(nb + a.n_new, a.S, a.R, a.C), a.S, ns, tr);
      most = w > most ? w : most;
    }
  } else {
    most = window_tokens(a.n_before, a.n_new, a.q_after, a.S, ns, tr);
  }
  if (most == 0) return hipSuccess;
  const int64_t work = most * (a.d / 8);
  dim3 grid((unsigned)((work + kThreads - 1) / kThreads), a.B * a.Hkv);
  hipLaunchKernelGGL(append_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// Device token counts: after a call's flush and append, each in-range count grows by
// n_new (the same range test as seq_before, so a skipped sequence keeps its count).
__global__ void advance_kernel(int32_t *dev_n, int B, int n_new, int64_t cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int64_t n = dev_n[b];
  if (n >= 0 && n + n_new <= cap) dev_n[b] = (int32_t)(n + n_new);
}

hipError_t launch_advance(int32_t *dev_n, int B, int n_new, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0, s, dev_n, B, n_new, cap);
  return hipGetLastError();
}

// Steps (128 body rows) of a flush of body rows [u0, u1).
// The flush instance for (d, input element size, order statistics): Hadamard butterflies,
// the 2-bit packing (d = 128 only), or the byte-code path; paged or contiguous body.
template <int D, int ES, int NL>
static void launch_flush_inst(const FlushArgs &a, bool b2, dim3 grid, hipStream_t s, int sp) {
  if (a.had != 0.f) {
    hipLaunchKernelGGL((flush_kernel<D, ES, NL, false, true, false>), grid, dim3(kThreads), 0, s, a, sp);
    return;
  }
  if constexpr (D == 128) {
    if (b2) {
      if (a.pg.table) hipLaunchKernelGGL((flush_kernel<D, ES, NL, true, false, true>), grid, dim3(kThreads), 0, s, a, sp);
      else hipLaunchKernelGGL((flush_kernel<D, ES, NL, false, false, true>), grid, dim3(kThreads), 0, s, a, sp);
      return;
    }
  }
  if (a.pg.table) hipLaunchKernelGGL((flush_kernel<D, ES, NL, true, false, false>), grid, dim3(kThreads), 0, s, a, sp);
  else hipLaunchKernelGGL((flush_kernel<D, ES, NL, false, false, false>), grid, dim3(kThreads), 0, s, a, sp);
}

static int64_t flush_steps(int64_t u0, int64_t u1) {
  if (u1 <= u0) return 0;
  const int64_t s0 = u0 / kSet, s1 = (u1 + kSet - 1) / kSet;
  return (s1 - s0 + 1) / 2;
}

hipError_t launch_flush(const FlushArgs &a, hipStream_t s) {
  int64_t steps = 0;   // the most any sequence needs; workgroups past a sequence's own return
  if (a.ragged == kRaggedDevice) {
    // counts unknown here: the most n_new tokens can make due, n_new + C - 1 body rows
    // starting anywhere in a 64-row set
    const int64_t sets = (a.n_new + a.C - 1 + kSet - 1) / kSet + 1;
    steps = (sets + 1) / 2;
  } else if (a.ragged) {
    for (int b = 0; b < a.B; ++b) {
      const int64_t nb = a.seq_nb[b];
      const int64_t st = flush_steps(n_quantized(nb, a.S, a.R, a.C), n_quantized(nb + a.n_new, a.S, a.R, a.C));
      if (st > steps) steps = st;
    }
  } else {
    steps = flush_steps(a.u0, a.u1);
  }
  if (steps == 0) return hipSuccess;
  const int64_t heads = (int64_t)a.B * a.Hkv;
  // about 512 workgroups (one round of the two that fit per CU); each walks a
  // contiguous run of at least two steps of one KV head, so T_K is staged once per
  // run and a step's loads overlap the previous step's stores (two rounds of shorter
  // runs measured ~4% slower on the bulk flush)
  int64_t spw = (steps * heads + 511) / 512;
  if (spw < 2) spw = 2;
  dim3 grid((unsigned)((steps + spw - 1) / spw + a.append_x), (unsigned)heads);
  int need = 0;
  if (a.quant_k == WUSHKV_Q_AFFINE_PCT || a.quant_v == WUSHKV_Q_AFFINE_PCT)
    need = a.need_lo > a.need_hi ? a.need_lo : a.need_hi;
  const int nl = need == 0 ? 0 : (need <= 2 ? 2 : (need <= 4 ? 4 : 8));
  const bool f32 = a.in_dtype == WUSHKV_DT_F32;
  const int sp = (int)spw;
  const bool b2 = a.d == 128 && a.bits_k == 2 && a.bits_v == 2 && a.had == 0.f;
#define WUSHKV_FLUSH_NL(D, ES)                                 \
  switch (nl) {                                                 \
    case 0: launch_flush_inst<D, ES, 0>(a, b2, grid, s, sp); break; \
    case 2: launch_flush_inst<D, ES, 2>(a, b2, grid, s, sp); break; \
    case 4: launch_flush_inst<D, ES, 4>(a, b2, grid, s, sp); break; \
    default: launch_flush_inst<D, ES, 8>(a, b2, grid, s, sp); break; \
  }
  if (a.d == 128) {
    if (f32) { WUSHKV_FLUSH_NL(128, 4) } else { WUSHKV_FLUSH_NL(128, 2) }
  } else {
    if (f32) { WUSHKV_FLUSH_NL(64, 4) } else { WUSHKV_FLUSH_NL(64, 2) }
  }
#undef WUSHKV_FLUSH_NL
  return hipGetLastError();
}

}  // namespace wushkv
