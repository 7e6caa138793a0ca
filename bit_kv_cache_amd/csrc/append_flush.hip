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

__global__ void __launch_bounds__(kThreads) append_kernel(AppendArgs a) {
  // one thread per (token, 8-channel group); blockIdx.y = b * Hkv + g
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int groups = a.d / 8;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_new * groups) return;
  const int64_t t = idx / groups;
  const int j0 = (int)(idx % groups) * 8;
  const int64_t n_before = seq_before(a, b);
  if (n_before < 0) return;
  const int64_t q_after = a.ragged ? n_quantized(n_before + a.n_new, a.S, a.R, a.C) : a.q_after;
  const int64_t p = n_before + t;
  _Float16 *dk, *dv;
  if (p < a.S) {
    dk = (_Float16 *)((char *)a.sink_k + bg * a.sink_bytes) + p * a.d;
    dv = (_Float16 *)((char *)a.sink_v + bg * a.sink_bytes) + p * a.d;
  } else if (p >= a.S + q_after) {
    const int64_t slot = (p - a.S) % (a.R + a.C);
    dk = (_Float16 *)((char *)a.ring_k + bg * a.ring_bytes) + slot * a.d;
    dv = (_Float16 *)((char *)a.ring_v + bg * a.ring_bytes) + slot * a.d;
  } else {
    return;  // flushed straight from the input by the flush kernel
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

template <int D>
struct FlushSmem {
  static constexpr int TP = D + 8;      // T_K row pitch (halves)
  static constexpr int KP = D + 16;     // key-code row pitch (bytes; rows stay 16-byte aligned)
  static constexpr int VP = kSet + 4;   // value-code row pitch (bytes), one row per channel
  _Float16 t[D][TP];
  uint8_t kc[kStepTok][KP];
  uint8_t vc[2][D][VP];
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
// earlier call (an fp16 row), else from the new input; an invalid token reads zeros.
// Lane group q holds channels 32 i + 8 q .. 32 i + 8 q + 7 (i = 0 .. D/32 - 1), at
// position 8 i + e of its list: one load instruction then covers 32 contiguous
// channels of each of its 16 rows.
template <int D, int ES>
__device__ __forceinline__ void load_seg(const FlushArgs &a, int64_t n_before, const char *ring_h, const char *in_h,
                                         int64_t u, bool valid, int q, RawSeg<ES, D / 4> &s) {
  constexpr int CPL = D / 4;
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
  } else if (ES == 2) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
      const unsigned w = raw_word(s, i);
      x[2 * i] = f16_round(bf16_lo(w));
      x[2 * i + 1] = f16_round(bf16_hi(w));
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPL; ++i) x[i] = f16_round(__uint_as_float(raw_word(s, i)));
  }
}

// ---- per-token parameters; the 4 lanes of a token exchange through lanes ^16, ^32

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

// (scale, zero) of a row from its merged order statistics: linear interpolation at
// virtual index (D-1)*pct/100 between sorted values, both rounded to fp16.
template <int D, int NL>
__device__ __forceinline__ void affine_from_stats(const FlushArgs &a, const OrderStats<NL> &o, int L, float &sc, float &zp) {
  const float x0 = pick<NL>(o.lo, a.lo_i);
  const float x1 = (a.lo_i + 1 < D) ? pick<NL>(o.lo, a.lo_i + 1) : x0;
  const float vlo = (a.lo_i + 1 < D) ? x0 + a.lo_t * (x1 - x0) : x0;
  const int hk = D - 1 - a.hi_i;
  const float y0 = pick<NL>(o.hi, hk);
  const float y1 = (hk >= 1) ? pick<NL>(o.hi, hk - 1) : y0;
  const float vhi = (a.hi_i + 1 < D) ? y0 + a.hi_t * (y1 - y0) : y0;
  sc = f16_round((vhi - vlo) / (float)(L - 1));
  zp = f16_round(vlo);
}

__device__ __forceinline__ float quest_step(float ss, float clip, int L, int D) {
  return f16_round(2.0f * clip * sqrtf(ss / (float)D) / (float)L);
}

// Exact code of a value known in fp64.
__device__ __forceinline__ int exact_code(double x, float sc, float zp, int quant, int L) {
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
  q.inv = sc != 0.f ? 1.0f / sc : 0.f;
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
// ... bit 2 of each of 4 codes -> 4 bits.
__device__ __forceinline__ unsigned kpack1(unsigned x) {
  const unsigned n = (x >> 2) & 0x01010101u;
  const unsigned y = (n | (n >> 7)) & 0x00030003u;
  return (y | (y >> 14)) & 0xFu;
}

template <int D, int ES, int NL, bool PAGED>
__global__ void __launch_bounds__(kThreads, 2) flush_kernel(FlushArgs a, int steps_per_wg) {
  constexpr int CPL = D / 4, KS = D / 32, NCT = D / 16;
  using QuestTag = std::integral_constant<bool, true>;
  using AffineTag = std::integral_constant<bool, false>;
  __shared__ FlushSmem<D> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, tok = lane & 15;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int Lk = 1 << a.bits_k, Lv = 1 << a.bits_v;
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
  // rows of earlier calls come from the ring (fp16); invalid rows read as fp16 zeros
  auto tok_ring = [&](int64_t u) { return !tok_valid(u) || a.S + u < n_before; };
  // this KV head's ring and input rows
  const char *ring_kh = (const char *)a.ring_k + (size_t)bg * a.ring_bytes;
  const char *ring_vh = (const char *)a.ring_v + (size_t)bg * a.ring_bytes;
  const size_t in_off = (size_t)bg * (size_t)a.n_new * (D * ES);
  const char *in_kh = (const char *)a.k_new + in_off;
  const char *in_vh = (const char *)a.v_new + in_off;
  auto load_k = [&](int64_t st, int tt) {
    const int64_t u = tok_of(st, tt);
    load_seg<D, ES>(a, n_before, ring_kh, in_kh, u, tok_valid(u), q, rk[tt]);
  };
  auto load_v = [&](int64_t st, int tt) {
    const int64_t u = tok_of(st, tt);
    load_seg<D, ES>(a, n_before, ring_vh, in_vh, u, tok_valid(u), q, rv[tt]);
  };
  if (st0 < st1) {   // in flight while T_K is staged
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) { load_k(st0, tt); load_v(st0, tt); }
  }
  {
    const _Float16 *T = a.tk + (size_t)g * D * D;
    for (int i = tid; i < D * D / 8; i += kThreads) {
      const int r = i / (D / 8), c8 = i % (D / 8);
      *(u32x4 *)&sm.t[r][8 * c8] = *(const u32x4 *)(T + (size_t)r * D + 8 * c8);
    }
  }
  // quad-transpose selectors of this lane (position e = tok & 3 in its quad)
  const unsigned selA = (tok & 2) ? 0x03020706u : 0x05040100u;
  const unsigned selB = (tok & 1) ? 0x03070105u : 0x06020400u;
  __syncthreads();

  for (int64_t st = st0; st < st1; ++st) {
    const int64_t set0 = s_first + 2 * st;
    const int64_t ubase = set0 * kSet + 32 * wave;   // this wave's first token

    // ---- keys, one tile at a time: x = T_K k16 on MFMA, parameters, codes
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int64_t u = ubase + 16 * tt + tok;
      const bool vt = tok_valid(u);
      unsigned kh[CPL / 2];
      seg_half2<ES, CPL>(rk[tt], tok_ring(u), a.in_dtype, kh);
      if (st + 1 < st1) load_k(st + 1, tt);
      // K-steps outer, tiles inner: NCT independent accumulation chains
      f32x4 acc[NCT];
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
      const int row = 32 * wave + 16 * tt + tok;
      auto key_tile = [&](auto tag) {
        constexpr bool QU = decltype(tag)::value;
        float sc, zp = 0.f;
        if constexpr (QU) {
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = fmaf(acc[ct][i], acc[ct][i], s4[i]);
          float ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          ss += __shfl_xor(ss, 16);
          ss += __shfl_xor(ss, 32);
          sc = quest_step(ss, a.clip, Lk, D);
        } else if constexpr (NL > 0) {
          OrderStats<NL> o;
          os_init(o);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) os_insert(o, acc[ct][i]);
          os_merge(o, 16);
          os_merge(o, 32);
          affine_from_stats<D, NL>(a, o, Lk, sc, zp);
        } else {
          sc = 0.f;
        }
        if (q == 0 && vt) {
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
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float c0, c1, c2, c3;
          e[ct] = 1.0f;
          code2(qk, acc[ct][0], acc[ct][1], e[ct], c0, c1);
          code2(qk, acc[ct][2], acc[ct][3], e[ct], c2, c3);
          unsigned w = __builtin_amdgcn_cvt_pk_u8_f32(c0, 0, 0u);
          w = __builtin_amdgcn_cvt_pk_u8_f32(c1, 1, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(c2, 2, w);
          w = __builtin_amdgcn_cvt_pk_u8_f32(c3, 3, w);
          *(unsigned *)&sm.kc[row][16 * ct + 4 * q] = w;
        }
        // elements near a boundary: the 4 lanes of a token take one candidate at a
        // time, each summing its CPL channels' exact products in fp64
        float emin = e[0];
#pragma unroll
        for (int ct = 1; ct < NCT; ++ct) emin = fminf(emin, e[ct]);
        const bool kn = vt && edge_near(qk, emin);
        if (__any(kn)) {
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
            for (int s = 0; s < CPL / 8; ++s) {
              const half8 tv = *(const half8 *)&sm.t[j][32 * s + 8 * q];
#pragma unroll
              for (int e8 = 0; e8 < 8; ++e8) {
                const unsigned w = kh[4 * s + e8 / 2];
                const float kv = (e8 & 1) ? f16_hi(w) : f16_lo(w);
                part += (double)((float)tv[e8] * kv);   // fp16 x fp16 is exact in fp32
              }
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            if (qs == q) {
              sm.kc[row][j] = (uint8_t)exact_code(part, sc, zp, QU ? WUSHKV_Q_QUEST : WUSHKV_Q_AFFINE_PCT, Lk);
              m &= ~(1u << bit);
            }
          }
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
      float xv[CPL];
      seg_float<ES, CPL>(rv[tt], tok_ring(u), a.in_dtype, xv);
      if (st + 1 < st1) load_v(st + 1, tt);
      const int s2 = wave >> 1;                       // set of this wave within the step
      const int col = 32 * (wave & 1) + 16 * tt;      // first token of the tile in its set
      auto value_tile = [&](auto tag) {
        constexpr bool QU = decltype(tag)::value;
        float sc, zp = 0.f;
        if constexpr (QU) {
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < CPL; ++k) s4[k & 3] = fmaf(xv[k], xv[k], s4[k & 3]);
          float ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          ss += __shfl_xor(ss, 16);
          ss += __shfl_xor(ss, 32);
          sc = quest_step(ss, a.clip, Lv, D);
        } else if constexpr (NL > 0) {
          OrderStats<NL> o;
          os_init(o);
#pragma unroll
          for (int k = 0; k < CPL; ++k) os_insert(o, xv[k]);
          os_merge(o, 16);
          os_merge(o, 32);
          affine_from_stats<D, NL>(a, o, Lv, sc, zp);
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
          *(unsigned *)&sm.vc[s2][seg_chan(q, 4 * g4 + (tok & 3))][col + 4 * (tok >> 2)] = w;
        }
        float emin = e[0];
#pragma unroll
        for (int g4 = 1; g4 < CPL / 4; ++g4) emin = fminf(emin, e[g4]);
        const bool vn = vt && edge_near(qv, emin);
        if (__any(vn)) {
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
            sm.vc[s2][seg_chan(q, k)][col + tok] =
                (uint8_t)exact_code((double)pick<CPL>(xv, k), sc, zp, QU ? WUSHKV_Q_QUEST : WUSHKV_Q_AFFINE_PCT, Lv);
          }
        }
      };
      if (a.quant_v == WUSHKV_Q_QUEST) value_tile(QuestTag{});
      else value_tile(AffineTag{});
    }
    __syncthreads();
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
          for (int e = 0; e < 8; ++e) w |= kpack1(cw[2 * k + e / 4][e % 4]) << (4 * e);
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
    using B2 = std::integral_constant<int, 2>;
    using B3 = std::integral_constant<int, 3>;
    using B4 = std::integral_constant<int, 4>;
    if (a.bits_k == 2) pack_k_rows(B2{});
    else if (a.bits_k == 3) pack_k_rows(B3{});
    else pack_k_rows(B4{});

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
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          const unsigned x = *(const unsigned *)&sm.vc[s2][j][16 * aa + 4 * c];
          w0[jj] |= vfield2(x) << (4 * aa);
          if constexpr (BVV == 3) w1[jj] |= vfield1(x) << (2 * aa);
          if constexpr (BVV == 4) w1[jj] |= vfield2(x >> 2) << (4 * aa);
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
      if (vlo == vbase && vhi == vbase + kSet) {
        if (a.bits_v == 2) pack_v_words(B2{}, Full{});
        else if (a.bits_v == 3) pack_v_words(B3{}, Full{});
        else pack_v_words(B4{}, Full{});
      } else {
        if (a.bits_v == 2) pack_v_words(B2{}, Part{});
        else if (a.bits_v == 3) pack_v_words(B3{}, Part{});
        else pack_v_words(B4{}, Part{});
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  const int64_t work = a.n_new * (a.d / 8);
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
  dim3 grid((unsigned)((steps + spw - 1) / spw), (unsigned)heads);
  int need = 0;
  if (a.quant_k == WUSHKV_Q_AFFINE_PCT || a.quant_v == WUSHKV_Q_AFFINE_PCT)
    need = a.need_lo > a.need_hi ? a.need_lo : a.need_hi;
  const int nl = need == 0 ? 0 : (need <= 2 ? 2 : (need <= 4 ? 4 : 8));
  const bool f32 = a.in_dtype == WUSHKV_DT_F32;
  const int sp = (int)spw;
#define WUSHKV_FLUSH(D, ES, NL)                                                                          \
  if (a.pg.table) hipLaunchKernelGGL((flush_kernel<D, ES, NL, true>), grid, dim3(kThreads), 0, s, a, sp); \
  else hipLaunchKernelGGL((flush_kernel<D, ES, NL, false>), grid, dim3(kThreads), 0, s, a, sp)
#define WUSHKV_FLUSH_NL(D, ES)            \
  switch (nl) {                            \
    case 0: WUSHKV_FLUSH(D, ES, 0); break; \
    case 2: WUSHKV_FLUSH(D, ES, 2); break; \
    case 4: WUSHKV_FLUSH(D, ES, 4); break; \
    default: WUSHKV_FLUSH(D, ES, 8); break; \
  }
  if (a.d == 128) {
    if (f32) { WUSHKV_FLUSH_NL(128, 4) } else { WUSHKV_FLUSH_NL(128, 2) }
  } else {
    if (f32) { WUSHKV_FLUSH_NL(64, 4) } else { WUSHKV_FLUSH_NL(64, 2) }
  }
#undef WUSHKV_FLUSH_NL
#undef WUSHKV_FLUSH
  return hipGetLastError();
}

}  // namespace wushkv
