// GQA decode attention over the 2-bit key cache on MFMA (gfx950), head_dim 128,
// G = 4 or 8 query heads per KV head, 2- or 3-bit values.
//
// What it computes is the plain softmax attention of the pages' method: scores
// (q . k)/sqrt(d) on the FP16 sink and recent tokens and (q~ . x^)/sqrt(d) on the
// quantized body, q~ = T^{-T} q (WUSH-KV digest, "method key points"); every KV
// head's codes are read once for its G query heads (review blog, Key Terms: GQA).
//
// Per body token the key reconstruction is x^ = s*c + z (affine) or (c - (L-1)/2)*s
// (QuEST), so q~ . x^ = s*(q~ . c) + z*sum(q~): the per-token parameters come out of
// the dot product and q~ . c is an integer-code contraction.
//
// Grid (ceil(P/4), B * Hkv), 256 threads.  Each wave streams the 64-token sets of one
// KV partition:
//   QK: v_mfma_i32_16x16x64_i8.  A = one 16-token tile of 2-bit codes spread to
//       bytes, B = q~ split into three signed 8-bit digits (q~ ~ alpha*(65536 d0 +
//       256 d1 + d2)), one digit per group of G columns, so the integer dot products
//       are exact and q~ keeps ~23 bits.  The digit columns are recombined in fp32
//       with DPP row shifts and the tiles are packed into full 64-lane registers
//       (lane column = G * tile + head) with bank-masked DPP moves.
//   softmax: online, base 2, per head; W = p * s_V as an fp16 hi + lo pair.
//   PV: v_mfma_f32_16x16x32_f16.  A = W (row = tile * G + head, zero outside the
//       row's own tile), B = value codes read straight from the set layout: a
//       field pair is one and/or with an fp16 exponent pattern, giving BASE + c
//       (BASE = 4, 16 or 64 by the pair's position); BASE * W is removed exactly
//       through the per-head zero term.  W enters as two MFMAs (hi and lo fp16
//       parts), so its rounding does not show in the output.
// Each partition wave first takes its share of the FP16 sink + recent tokens on
// plain fp32 VALU, which seeds its softmax state, then streams its body sets.
// Each workgroup merges its 4 waves in LDS and writes one partial (m, l, o); the
// merge kernel that follows on the stream combines the partials.
#include <type_traits>

#include "wushkv_internal.h"

namespace wushkv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

// DPP encodings (gfx9): row_shl:n = 0x100+n (lane i reads i+n), row_shr:n = 0x110+n
// (lane i reads i-n), row_ror:n = 0x120+n; bank b = lanes 4b..4b+3 of each row.
// acc += src[lane + 4 or 8 in the row] * k as one v_fmac_f32_dpp; a lane whose source
// lies outside its row keeps acc.  The s_nop 1 gives the two wait states a DPP read
// needs after a VALU write of its source (the compiler does not see into asm).
__device__ __forceinline__ void fmac_shl4(float &acc, float src, float k) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_shl:4 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(src), "v"(k));
}
__device__ __forceinline__ void fmac_shl8(float &acc, float src, float k) {
  asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_shl:8 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(src), "v"(k));
}

template <int CTRL, int BANK = 0xF>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, BANK, false));
}

// Byte layout of one ring slot.  A body set: key codes (2 KB), value codes (2 KB),
// the 3-bit plane (1 KB), key then value parameters (up to 256 B each), all copied
// verbatim.  A window stage: 8 FP16 key rows (2 KB) then 8 FP16 value rows (2 KB).
// Both kinds are filled by exactly DMAS load-to-LDS instructions, so one vmcnt per
// pending slot covers either.
template <int BV>
struct Stage {
  static constexpr int K = 0, V = 2048, VH = 4096;
  static constexpr int KP = BV == 3 ? 5120 : 4096, VP = KP + 256, SIZE = VP + 256;
  static constexpr int WK = 0, WV = 2048;
  static constexpr int DMAS = BV == 3 ? 6 : 5;
};

constexpr int kStages = 2;   // body sets staged per wave: the one computed and the next

template <int G, int BV>
struct __align__(16) FastSmem {
  float qt[G][kD];
  float q[G][kD];
  float wp[kWaves][G][8];         // window stage: probabilities [head][token]
  float wmx[kWaves][16], wls[kWaves][16];  // window partial: max and sum per head
  union {
    uint8_t ring[kWaves][kStages][Stage<BV>::SIZE];
    struct {
      float o[kWaves][16][kD];    // per wave: rows (tile-phase, head), columns channels
      float wo[kWaves][G][kD];    // window partial: weighted FP16 values [head][channel]
    };
  } u;
  float alpha[16], sq[16];
  float m[kWaves][16], l[kWaves][16], z[kWaves][16];
};

__device__ __forceinline__ int digit_of(float qt, float inv_alpha, int dg) {
  int Q = (int)rintf(qt * inv_alpha);
  int d2 = ((Q + 128) & 255) - 128;
  int Q1 = (Q - d2) >> 8;
  int d1 = ((Q1 + 128) & 255) - 128;
  int d0 = (Q1 - d1) >> 8;
  return dg == 0 ? d0 : (dg == 1 ? d1 : d2);
}

__device__ __forceinline__ unsigned pack_h2(float x, float y) {
  f16x2 v = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ float h_lo(unsigned w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float h_hi(unsigned w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }

// A 32-bit constant held in a VGPR the compiler cannot fold, so masks and exponent
// patterns feed three-operand VALU forms (gfx9 VOP3 has no literal operand).
__device__ __forceinline__ unsigned vconst(unsigned c) {
  unsigned r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// Value-code pair k of a word sits at bits (2k, 2k+16).  With the code at mantissa
// bits 4-5, 6-7 or 8-9 of an fp16 whose exponent makes that field's unit 1, the
// fp16 is exactly BASE + c with BASE = 64, 16 or 4.  Pairs 2, 3, 4 are read in place,
// pairs 5, 6, 7 from w >> 6 and pairs 0, 1 from w << 4, so a word costs two shifts
// and one and/or per pair.
struct VConst {
  unsigned m2, m3, m4, e2, e3, e4;  // masks and exponent patterns of positions 2, 3, 4
  unsigned m3b, mhi, e3b;           // 3-bit codes: low bits at 6-7, third bit at 8, base 16
};

__device__ __forceinline__ VConst make_vconst() {
  VConst c;
  c.m2 = vconst(0x00300030u); c.e2 = vconst(0x54005400u);
  c.m3 = vconst(0x00C000C0u); c.e3 = vconst(0x4C004C00u);
  c.m4 = vconst(0x03000300u); c.e4 = vconst(0x44004400u);
  c.m3b = c.m3; c.mhi = vconst(0x01000100u); c.e3b = c.e3;
  return c;
}

__device__ __forceinline__ unsigned and_or(unsigned x, unsigned m, unsigned o) { return (x & m) | o; }

// BASE of value pair k for 2-bit codes (see above): k = 0,2,5 -> 64; 1,3,6 -> 16; 4,7 -> 4.
__device__ __forceinline__ float vbase2(int k) {
  return (k == 4 || k == 7) ? 4.0f : ((k == 1 || k == 3 || k == 6) ? 16.0f : 64.0f);
}

template <int K>
__device__ __forceinline__ unsigned shift_to3(unsigned w) {
  if constexpr (K == 3) return w;
  else if constexpr (K < 3) return w << (2 * (3 - K));
  else return w >> (2 * (K - 3));
}

// 3-bit: low 2 bits at mantissa 6..7, the third bit at mantissa 8, exponent 2^4 -> 16 + c.
template <int K>
__device__ __forceinline__ unsigned v_pair3(unsigned w, unsigned hi, const VConst &c) {
  return (shift_to3<K>(w) & c.m3b) | ((hi >> K) & c.mhi) | c.e3b;
}

// B operand of PV instruction iota (pairs 4*iota .. 4*iota+3) from one value word.
template <int BV>
__device__ __forceinline__ f16x8 v_operand(unsigned w, unsigned hi, int iota, const VConst &c) {
  u32x4 r;
  if constexpr (BV == 2) {
    if (iota == 0) {
      const unsigned w4 = w << 4;
      r[0] = and_or(w4, c.m2, c.e2);   // pair 0
      r[1] = and_or(w4, c.m3, c.e3);   // pair 1
      r[2] = and_or(w, c.m2, c.e2);    // pair 2
      r[3] = and_or(w, c.m3, c.e3);    // pair 3
    } else {
      const unsigned w6 = w >> 6;
      r[0] = and_or(w, c.m4, c.e4);    // pair 4
      r[1] = and_or(w6, c.m2, c.e2);   // pair 5
      r[2] = and_or(w6, c.m3, c.e3);   // pair 6
      r[3] = and_or(w6, c.m4, c.e4);   // pair 7
    }
  } else {
    if (iota == 0) {
      r[0] = v_pair3<0>(w, hi, c); r[1] = v_pair3<1>(w, hi, c); r[2] = v_pair3<2>(w, hi, c); r[3] = v_pair3<3>(w, hi, c);
    } else {
      r[0] = v_pair3<4>(w, hi, c); r[1] = v_pair3<5>(w, hi, c); r[2] = v_pair3<6>(w, hi, c); r[3] = v_pair3<7>(w, hi, c);
    }
  }
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ i32x4 k_operand(unsigned w) {
  i32x4 r;
  r[0] = (int)(w & 0x03030303u);
  r[1] = (int)((w >> 2) & 0x03030303u);
  r[2] = (int)((w >> 4) & 0x03030303u);
  r[3] = (int)((w >> 6) & 0x03030303u);
  return r;
}

template <int G>
__device__ __forceinline__ float head_max(float x) {
  if constexpr (G == 4) {
    x = fmaxf(x, dpp<0x124>(x, x));
    x = fmaxf(x, dpp<0x128>(x, x));
  } else {
    x = fmaxf(x, dpp<0x128>(x, x));
  }
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

template <int G>
__device__ __forceinline__ float head_sum(float x) {
  if constexpr (G == 4) {
    x += dpp<0x124>(x, x);
    x += dpp<0x128>(x, x);
  } else {
    x += dpp<0x128>(x, x);
  }
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int NGRP>
struct SetData {
  u32x2 kw[4];          // key codes: words 2*q4, 2*q4+1 of rows 16T + col
  u32x4 vw0, vw1, vh;   // value words of this lane (8 column tiles), 3rd-bit plane
  u32x4 kp[NGRP], vp[NGRP];  // per-token parameters of this lane's 4 packed tokens
};

typedef __attribute__((address_space(3))) void lds_void;

// Queue the loads of body set `set` into the wave's ring slot `st` (load-to-LDS:
// lane i's bytes land at the slot offset + i * size).  Stage<BV>::DMAS instructions.
template <int BV>
__device__ __forceinline__ void stage_set(const DecodeArgs &a, const uint8_t *kplane, const uint8_t *vplane,
                                          const uint8_t *kpar, const uint8_t *vpar, int64_t set, uint8_t *st) {
  using S = Stage<BV>;
  const int lane = threadIdx.x & 63;
  constexpr int aux = 2;   // nontemporal: streamed once
  const uint8_t *kg = kplane + (size_t)set * 2048;
  __builtin_amdgcn_global_load_lds(kg + 16 * lane, (lds_void *)(st + S::K), 16, 0, aux);
  __builtin_amdgcn_global_load_lds(kg + 1024 + 16 * lane, (lds_void *)(st + S::K + 1024), 16, 0, aux);
  const uint8_t *vg = vplane + (size_t)set * a.vset_bytes;
  __builtin_amdgcn_global_load_lds(vg + 16 * lane, (lds_void *)(st + S::V), 16, 0, aux);
  __builtin_amdgcn_global_load_lds(vg + 1024 + 16 * lane, (lds_void *)(st + S::V + 1024), 16, 0, aux);
  if constexpr (BV == 3) __builtin_amdgcn_global_load_lds(vg + 2048 + 16 * lane, (lds_void *)(st + S::VH), 16, 0, aux);
  // parameters, one instruction: lanes 0-15 the keys', 16-31 the values' (64 tokens x
  // 2 or 4 bytes each; lane 0 is always active, so the instruction always issues)
  const int kb = a.kpar_n * 2, vbn = a.vpar_n * 2;
  const bool pk = lane < 4 * kb, pv = lane >= 16 && lane - 16 < 4 * vbn;
  if (pk || pv) {
    const uint8_t *src = pk ? kpar + (size_t)set * 64 * kb + 16 * lane : vpar + (size_t)set * 64 * vbn + 16 * (lane - 16);
    __builtin_amdgcn_global_load_lds(src, (lds_void *)(st + S::KP), 16, 0, aux);
  }
}

// Row of window-list token t: sink row t, or the ring slot of the t-th token after the
// sink (first_slot = slot of the oldest recent token); the sign bit marks the ring.
__device__ __forceinline__ int window_row(int t, int ns, unsigned first_slot, unsigned ring) {
  return t < ns ? t : (int)(((first_slot + (unsigned)(t - ns)) % ring) | 0x80000000u);
}

// Queue window-list tokens [t0, t0 + cnt), cnt <= 8, into a ring slot: 8 key rows and
// 8 value rows of 256 bytes (lanes past cnt re-read token t0, so every instruction
// issues with all lanes), plus DMAS - 4 single-lane filler loads into the slot's
// unused parameter area so a window slot counts like a body slot.
template <int BV>
__device__ __forceinline__ void stage_window(const uint8_t *sinkk, const uint8_t *sinkv, const uint8_t *ringk,
                                             const uint8_t *ringv, int t0, int cnt, int ns, unsigned first_slot,
                                             unsigned rsz, const void *filler, uint8_t *st) {
  using S = Stage<BV>;
  const int lane = threadIdx.x & 63;
  constexpr int aux = 2;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = 4 * i + (lane >> 4);
    const int r = window_row(t0 + (j < cnt ? j : 0), ns, first_slot, rsz);
    const size_t off = (size_t)(r & 0x7FFFFFFF) * 256 + 16 * (lane & 15);
    __builtin_amdgcn_global_load_lds((r >= 0 ? sinkk : ringk) + off, (lds_void *)(st + S::WK + 1024 * i), 16, 0, aux);
    __builtin_amdgcn_global_load_lds((r >= 0 ? sinkv : ringv) + off, (lds_void *)(st + S::WV + 1024 * i), 16, 0, aux);
  }
#pragma unroll
  for (int i = 0; i < S::DMAS - 4; ++i)
    if (lane == 0) __builtin_amdgcn_global_load_lds(filler, (lds_void *)(st + S::KP + 64 * i), 16, 0, aux);
}

// Wait until at most `pending` staged sets' loads are still in flight.
template <int BV>
__device__ __forceinline__ void wait_staged(int pending) {
  constexpr int D = Stage<BV>::DMAS;
  if (pending <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
}

// This lane's operands of a staged set.
template <int NGRP, int TPG, int BV>
__device__ __forceinline__ void read_set(const DecodeArgs &a, const uint8_t *st, SetData<NGRP> &d) {
  using S = Stage<BV>;
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4, col = lane & 15;
  const int tcol = col / (16 / TPG);
#pragma unroll
  for (int T = 0; T < 4; ++T) d.kw[T] = *(const u32x2 *)(st + S::K + (16 * T + col) * 32 + 8 * q4);
  d.vw0 = *(const u32x4 *)(st + S::V + 32 * lane);
  d.vw1 = *(const u32x4 *)(st + S::V + 32 * lane + 16);
  if constexpr (BV == 3) d.vh = *(const u32x4 *)(st + S::VH + 16 * lane);
  else d.vh = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
  for (int gr = 0; gr < NGRP; ++gr) {
    const int t0 = 16 * (TPG * gr + tcol) + 4 * q4;
    if (a.quant_k == WUSHKV_Q_QUEST) {
      const u32x2 x = *(const u32x2 *)(st + S::KP + 2 * t0);
      d.kp[gr] = (u32x4){x[0], x[1], 0u, 0u};
    } else {
      d.kp[gr] = *(const u32x4 *)(st + S::KP + 4 * t0);
    }
    if (a.quant_v == WUSHKV_Q_QUEST) {
      const u32x2 x = *(const u32x2 *)(st + S::VP + 2 * t0);
      d.vp[gr] = (u32x4){x[0], x[1], 0u, 0u};
    } else {
      d.vp[gr] = *(const u32x4 *)(st + S::VP + 4 * t0);
    }
  }
}

template <int G, int BV>
__device__ void window_stage(FastSmem<G, BV> &sm, const uint8_t *st, int cnt, int w, float (&wm)[G],
                             float (&wl)[G], float (&wacc)[G][2]);

// One wave of a KV partition: its body sets [s0, s1), then its 8-token stages
// [ws0, ws1) of the FP16 window list, all streamed through the wave's LDS ring.
template <int G, int BV>
__device__ void body_wave(const DecodeArgs &a, FastSmem<G, BV> &sm, int bg, int64_t s0, int64_t s1, int ws0, int ws1,
                          f32x4 (&O)[8], float &m_out, float &l_out, float &z_out, float (&wm_out)[G],
                          float (&wl_out)[G], float (&wacc_out)[G][2]) {
  constexpr int TPG = 16 / G;          // tiles per packed register group
  constexpr int NGRP = 4 / TPG;        // groups per 64-token set
  constexpr int NMF = (3 * G + 15) / 16;  // QK MFMAs per (tile, k-step)
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4, col = lane & 15;
  const int hc = col % G;              // head of this lane's packed column
  const int tcol = col / G;            // tile within a packed group
  const float qk_scale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int Lk = 4, Lv = 1 << BV;

  // q~ digits as B operands: column c of MFMA mf holds digit dg of head h
  i32x4 bq[NMF][2];
#pragma unroll
  for (int mf = 0; mf < NMF; ++mf) {
    int dg, h;
    bool live;
    if constexpr (G == 4) { dg = col >> 2; h = col & 3; live = col < 12; }
    else { dg = mf == 0 ? (col >> 3) : 2; h = col & 7; live = mf == 0 || col < 8; }
    const float inv_alpha = live ? 1.0f / sm.alpha[h] : 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        unsigned word = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int ch = 16 * (2 * q4 + s) + 4 * bb + k;
          const int dig = live ? digit_of(sm.qt[h][ch], inv_alpha, dg) : 0;
          word |= ((unsigned)dig & 0xFFu) << (8 * bb);
        }
        bq[mf][s][k] = (int)word;
      }
    }
  }
  const float a_sc = sm.alpha[hc] * 65536.0f * qk_scale;
  const float b_sc = sm.sq[hc] * qk_scale;
  const VConst vc = make_vconst();
  // digit weights as VGPR values so the DPP reads fuse into v_fmac_f32_dpp
  const float inv256 = __uint_as_float(vconst(0x3B800000u));    // 2^-8
  const float inv65536 = __uint_as_float(vconst(0x37800000u));  // 2^-16
  // BASE of the value operand that multiplies this lane's weights W[i] of packed
  // group gr: the lane's tile T sits in PV instruction T/2 at pair 2T + i/2
  float vbase[NGRP][2];
#pragma unroll
  for (int gr = 0; gr < NGRP; ++gr) {
    const int T = TPG * gr + tcol;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) vbase[gr][hf] = BV == 2 ? vbase2(2 * T + hf) : 16.0f;
  }

  const uint8_t *kplane = a.codes_k + (size_t)bg * a.kcode_bytes;
  const uint8_t *vplane = a.codes_v + (size_t)bg * a.vcode_bytes;
  const uint8_t *kpar = (const uint8_t *)a.par_k + (size_t)bg * a.kpar_bytes;
  const uint8_t *vpar = (const uint8_t *)a.par_v + (size_t)bg * a.vpar_bytes;
  const int w = threadIdx.x >> 6;
  uint8_t *ring = &sm.u.ring[w][0][0];
  constexpr int SB = Stage<BV>::SIZE;
  // items of this wave: body sets s0 .. s1-1, then 8-token window stages ws0 .. ws1-1
  const int nb = (int)(s1 - s0), nitems = nb + (ws1 - ws0);
  const int ns = (int)(a.n < a.S ? a.n : a.S);
  const int nw = ns + (int)(a.n - a.S - a.nq > 0 ? a.n - a.S - a.nq : 0);
  const unsigned rsz = (unsigned)(a.R + a.C);
  const unsigned first_slot = (unsigned)(a.nq % rsz);
  const uint8_t *sinkk = (const uint8_t *)a.sink_k + (size_t)bg * a.sink_bytes;
  const uint8_t *sinkv = (const uint8_t *)a.sink_v + (size_t)bg * a.sink_bytes;
  const uint8_t *ringk = (const uint8_t *)a.ring_k + (size_t)bg * a.ring_bytes;
  const uint8_t *ringv = (const uint8_t *)a.ring_v + (size_t)bg * a.ring_bytes;
  auto issue = [&](int item, uint8_t *dst) {
    if (item < nb) {
      stage_set<BV>(a, kplane, vplane, kpar, vpar, s0 + item, dst);
    } else {
      const int t0 = 8 * (ws0 + item - nb);
      stage_window<BV>(sinkk, sinkv, ringk, ringv, t0, nw - t0 < 8 ? nw - t0 : 8, ns, first_slot, rsz, a.qt, dst);
    }
  };
  if (nitems > 0) issue(0, ring);

  float m_run = -INFINITY, l_lane = 0.f, zacc = 0.f;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) O[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const bool kq = a.quant_k == WUSHKV_Q_QUEST, vq = a.quant_v == WUSHKV_Q_QUEST;

  // one 64-token set: QK, softmax update, PV.  FULL: every token of the set is in
  // the body (no validity selects).
  auto compute = [&](auto full_tag, int64_t set, const SetData<NGRP> &cur) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t base = set * kSet;
    const u32x2 *kw = cur.kw;
    const u32x4 vw0 = cur.vw0, vw1 = cur.vw1, vh = cur.vh;
    const u32x4 *kp = cur.kp, *vp = cur.vp;

    // ---- QK on the int8 MFMA (all tiles' first k-step before any second one, so no
    // MFMA waits on the one just issued), digit recombination, packing
    float C[NGRP][4];
    i32x4 dq[4][NMF];
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
        dq[T][mf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k_operand(kw[T][0]), bq[mf][0], (i32x4){0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int mf = 0; mf < NMF; ++mf)
        dq[T][mf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(k_operand(kw[T][1]), bq[mf][1], dq[T][mf], 0, 0, 0);
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      float r[4];
      if constexpr (G == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // digit columns h, h+4, h+8 -> lane h; columns 12..15 hold zeros, so the first
          // step leaves lanes 8..11 (read by the second) unchanged
          float f = (float)dq[T][0][i];
          fmac_shl4(f, f, inv256);
          fmac_shl8(f, f, inv65536);
          r[i] = f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float f = (float)dq[T][0][i];
          fmac_shl8(f, f, inv256);
          r[i] = fmaf((float)dq[T][1][i], inv65536, f);
        }
      }
      const int gr = T / TPG, tp = T % TPG;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (G == 4) {
          if (tp == 0) C[gr][i] = r[i];
          else if (tp == 1) C[gr][i] = dpp<0x114, 0x2>(C[gr][i], r[i]);
          else if (tp == 2) C[gr][i] = dpp<0x118, 0x4>(C[gr][i], r[i]);
          else C[gr][i] = dpp<0x11C, 0x8>(C[gr][i], r[i]);
        } else {
          if (tp == 0) C[gr][i] = r[i];
          else C[gr][i] = dpp<0x118, 0xC>(C[gr][i], r[i]);
        }
      }
    }

    // ---- scores and online softmax (base 2)
    float sc[NGRP][4];
    float mx = -INFINITY;
#pragma unroll
    for (int gr = 0; gr < NGRP; ++gr) {
      const int64_t t0 = base + 16 * (TPG * gr + tcol) + 4 * q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s_t, z_t;
        if (kq) {
          const unsigned pw = kp[gr][i >> 1];
          s_t = (i & 1) ? h_hi(pw) : h_lo(pw);
          z_t = -0.5f * (Lk - 1) * s_t;
        } else {
          s_t = h_lo(kp[gr][i]);
          z_t = h_hi(kp[gr][i]);
        }
        const bool valid = FULL || t0 + i < a.nq;
        sc[gr][i] = valid ? fmaf(s_t, C[gr][i] * a_sc, z_t * b_sc) : -INFINITY;
        mx = fmaxf(mx, sc[gr][i]);
      }
    }
    mx = head_max<G>(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__any(alpha != 1.0f)) {
      l_lane *= alpha;
      zacc *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = (4 * q4 + i) % G;  // packed column of head (4*q4+i) % G, row 0
        const float f = __shfl(alpha, src);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) O[ct][i] *= f;
      }
    }
    m_run = m_new;

    unsigned wp[NGRP][2], wl[NGRP][2];
#pragma unroll
    for (int gr = 0; gr < NGRP; ++gr) {
      const int64_t t0 = base + 16 * (TPG * gr + tcol) + 4 * q4;
      float W[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[gr][i] - m_run);
        float s_t, z_t;
        if (vq) {
          const unsigned pw = vp[gr][i >> 1];
          s_t = (i & 1) ? h_hi(pw) : h_lo(pw);
          z_t = -0.5f * (Lv - 1) * s_t;
        } else {
          s_t = h_lo(vp[gr][i]);
          z_t = h_hi(vp[gr][i]);
        }
        // W = p s enters the MFMA as fp16 hi + lo (~22 bits) against BASE + c; the
        // zero term takes p z - BASE W, with W in place of hi + lo (they differ by
        // ~2^-22 W, i.e. ~1.5e-5 W at BASE = 64)
        const bool valid = FULL || t0 + i < a.nq;
        l_lane += p;
        W[i] = valid ? p * s_t : 0.f;
        const float zb = fmaf(-vbase[gr][i >> 1], s_t, z_t);
        zacc = valid ? fmaf(p, zb, zacc) : zacc;
      }
      wp[gr][0] = pack_h2(W[0], W[1]);
      wp[gr][1] = pack_h2(W[2], W[3]);
      wl[gr][0] = pack_h2(W[0] - h_lo(wp[gr][0]), W[1] - h_hi(wp[gr][0]));
      wl[gr][1] = pack_h2(W[2] - h_lo(wp[gr][1]), W[3] - h_hi(wp[gr][1]));
    }

    // ---- PV on the f16 MFMA: instruction iota covers tiles 2*iota, 2*iota+1
    const unsigned vws[8] = {vw0[0], vw0[1], vw0[2], vw0[3], vw1[0], vw1[1], vw1[2], vw1[3]};
    unsigned hws[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if constexpr (BV == 3) {
        const unsigned h16 = (vh[ct >> 1] >> (16 * (ct & 1))) & 0xFFFFu;
        hws[ct] = ((h16 & 0xFFu) << 8) | ((h16 & 0xFF00u) << 16);
      } else {
        hws[ct] = 0u;
      }
    }
#pragma unroll
    for (int iota = 0; iota < 2; ++iota) {
      const int T = TPG * ((G == 4) ? 0 : iota) + tcol;  // lane's tile for this instruction's group
      const int gr = (G == 4) ? 0 : iota;
      const bool mine = (T >> 1) == iota;
      const int vp2 = 2 * (T & 1);
      u32x4 av, al;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        av[v] = (mine && v == vp2) ? wp[gr][0] : ((mine && v == vp2 + 1) ? wp[gr][1] : 0u);
        al[v] = (mine && v == vp2) ? wl[gr][0] : ((mine && v == vp2 + 1) ? wl[gr][1] : 0u);
      }
      const f16x8 Ah = __builtin_bit_cast(f16x8, av);
      const f16x8 Al = __builtin_bit_cast(f16x8, al);
      // four column tiles at a time, hi parts before lo parts: each accumulator's
      // second MFMA is issued three independent MFMAs after its first
#pragma unroll
      for (int ct0 = 0; ct0 < 8; ct0 += 4) {
        f16x8 Bv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) Bv[c] = v_operand<BV>(vws[ct0 + c], hws[ct0 + c], iota, vc);
#pragma unroll
        for (int c = 0; c < 4; ++c) O[ct0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bv[c], O[ct0 + c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) O[ct0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bv[c], O[ct0 + c], 0, 0, 0);
      }
    }
  };

  // items: item k + 1 is staged while item k computes
  using FullTag = std::integral_constant<bool, true>;
  using TailTag = std::integral_constant<bool, false>;
  int it = 0;
  for (; it < nb; ++it) {
    const bool more = it + 1 < nitems;
    if (more) issue(it + 1, ring + ((it + 1) & 1) * SB);
    wait_staged<BV>(more ? 1 : 0);
    SetData<NGRP> cur;
    read_set<NGRP, TPG, BV>(a, ring + (it & 1) * SB, cur);
    const int64_t set = s0 + it;
    if ((set + 1) * kSet <= a.nq) compute(FullTag{}, set, cur);
    else compute(TailTag{}, set, cur);
  }
  float wm[G], wl[G], wacc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { wm[h] = -INFINITY; wl[h] = 0.f; wacc[h][0] = wacc[h][1] = 0.f; }
  for (; it < nitems; ++it) {
    const bool more = it + 1 < nitems;
    if (more) issue(it + 1, ring + ((it + 1) & 1) * SB);
    wait_staged<BV>(more ? 1 : 0);
    const int t0 = 8 * (ws0 + it - nb);
    window_stage<G, BV>(sm, ring + (it & 1) * SB, nw - t0 < 8 ? nw - t0 : 8, w, wm, wl, wacc);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    wm_out[h] = wm[h];
    wl_out[h] = wl[h];
    wacc_out[h][0] = wacc[h][0];
    wacc_out[h][1] = wacc[h][1];
  }

  // per-head totals; every lane of a head holds them
  m_out = m_run;
  l_out = head_sum<G>(l_lane);
  z_out = head_sum<G>(zacc);
}

// One window stage: cnt <= 8 FP16 window tokens in a ring slot, on fp32 VALU.  Scores:
// 8 lanes per token, 16 channels each, summed over the 8; values: lane = two
// channels.  The stage folds into this wave's window partial: per head the running
// max and sum (the same in every lane) and this lane's two weighted value channels.
template <int G, int BV>
__device__ void window_stage(FastSmem<G, BV> &sm, const uint8_t *st, int cnt, int w, float (&wm)[G],
                             float (&wl)[G], float (&wacc)[G][2]) {
  using S = Stage<BV>;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 3, cc = lane & 7;   // token of the stage, 16-channel chunk
  const float qk_scale = kLog2e * 0.08838834764831845f;
  const bool valid = j < cnt;
  const f16x8 k0 = *(const f16x8 *)(st + S::WK + 256 * j + 32 * cc);
  const f16x8 k1 = *(const f16x8 *)(st + S::WK + 256 * j + 32 * cc + 16);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 qv = *(const f32x4 *)&sm.q[h][16 * cc + 4 * c];
#pragma unroll
      for (int e = 0; e < 4; ++e) x = fmaf(qv[e], (float)(c < 2 ? k0[4 * c + e] : k1[4 * (c - 2) + e]), x);
    }
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    // every lane of token j holds its score; max and sum run over the 8 tokens
    const float sc = valid ? x * qk_scale : -INFINITY;
    float mx = fmaxf(sc, __shfl_xor(sc, 8));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(wm[h], mx);
    const float al = __builtin_amdgcn_exp2f(wm[h] - mn);
    const float pr = valid ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
    float ps = pr + __shfl_xor(pr, 8);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    if (cc == 0) sm.wp[w][h][j] = pr;
    wl[h] = wl[h] * al + ps;
    wm[h] = mn;
    wacc[h][0] *= al;
    wacc[h][1] *= al;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int u = 0; u < cnt; ++u) {
    const f16x2 vv = *(const f16x2 *)(st + S::WV + 256 * u + 4 * lane);
    const float v0 = (float)vv[0], v1 = (float)vv[1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = sm.wp[w][h][u];
      wacc[h][0] = fmaf(pr, v0, wacc[h][0]);
      wacc[h][1] = fmaf(pr, v1, wacc[h][1]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <int G, int BV>
__global__ void __launch_bounds__(kThreads) decode_fast_kernel(DecodeArgs a, int nwg_body) {
  __shared__ FastSmem<G, BV> sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int h0 = g * G;

  for (int i = tid; i < G * kD; i += kThreads) {
    const int hh = i / kD, j = i % kD;
    const size_t off = ((size_t)b * a.Hq + h0 + hh) * kD + j;
    sm.qt[hh][j] = a.qt[off];
    sm.q[hh][j] = load_in(a.q, a.q_dtype, off);
  }
  __syncthreads();
  if (tid < G) {
    float mxa = 0.f, s = 0.f;
    for (int j = 0; j < kD; ++j) {
      const float v = sm.qt[tid][j];
      mxa = fmaxf(mxa, fabsf(v));
      s += v;
    }
    // q~ ~ alpha * Q with |Q| <= 127 * 65536, split into three signed 8-bit digits
    sm.alpha[tid] = mxa > 0.f ? mxa / (127.0f * 65536.0f) : 1.0f;
    sm.sq[tid] = s;
  }
  __syncthreads();

  f32x4 O[8];
  float bm = -INFINITY, bl = 0.f, bz = 0.f;
  float wm[G], wl[G], wacc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { wm[h] = -INFINITY; wl[h] = 0.f; wacc[h][0] = wacc[h][1] = 0.f; }
  const int part = (int)blockIdx.x * kWaves + w;
  if (part < a.P) {
    const int64_t nsets = (a.nq + kSet - 1) / kSet;
    const int64_t s0 = nsets * part / a.P, s1 = nsets * (part + 1) / a.P;
    const int64_t ns = a.n < a.S ? a.n : a.S;
    const int64_t nw = ns + (a.n - a.S - a.nq > 0 ? a.n - a.S - a.nq : 0);
    const int64_t nws = (nw + 7) / 8;
    const int ws0 = (int)(nws * part / a.P), ws1 = (int)(nws * (part + 1) / a.P);
    body_wave<G, BV>(a, sm, bg, s0, s1, ws0, ws1, O, bm, bl, bz, wm, wl, wacc);
  }
  __syncthreads();  // every wave is done with its ring, which u.o and u.wo alias
#pragma unroll
  for (int h = 0; h < G; ++h) {
    sm.u.wo[w][h][2 * lane] = wacc[h][0];
    sm.u.wo[w][h][2 * lane + 1] = wacc[h][1];
    if (lane == 0) { sm.wmx[w][h] = wm[h]; sm.wls[w][h] = wl[h]; }
  }
  if (part < a.P) {
    if (lane < G) { sm.m[w][lane] = bm; sm.l[w][lane] = bl; sm.z[w][lane] = bz; }
    const int q4 = lane >> 4, col = lane & 15;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.o[w][4 * q4 + i][16 * ct + col] = O[ct][i];
  } else {
    if (lane < G) { sm.m[w][lane] = -INFINITY; sm.l[w][lane] = 0.f; sm.z[w][lane] = 0.f; }
    for (int r = 0; r < 16; ++r) {
      sm.u.o[w][r][2 * lane] = 0.f;
      sm.u.o[w][r][2 * lane + 1] = 0.f;
    }
  }
  __syncthreads();

  // ---- merge the 4 waves into this workgroup's partial
  const int P1 = a.P + 1;
  for (int i = tid; i < G * kD; i += kThreads) {
    const int hh = i / kD, j = i % kD;
    float mstar = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      if (sm.l[ww][hh] > 0.f) mstar = fmaxf(mstar, sm.m[ww][hh]);
      if (sm.wls[ww][hh] > 0.f) mstar = fmaxf(mstar, sm.wmx[ww][hh]);
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      if (sm.l[ww][hh] > 0.f) {
        const float f = __builtin_amdgcn_exp2f(sm.m[ww][hh] - mstar);
        float o = sm.z[ww][hh];
#pragma unroll
        for (int tp = 0; tp < 16 / G; ++tp) o += sm.u.o[ww][G * tp + hh][j];
        num = fmaf(f, o, num);
        den = fmaf(f, sm.l[ww][hh], den);
      }
      if (sm.wls[ww][hh] > 0.f) {
        const float f = __builtin_amdgcn_exp2f(sm.wmx[ww][hh] - mstar);
        num = fmaf(f, sm.u.wo[ww][hh][j], num);
        den = fmaf(f, sm.wls[ww][hh], den);
      }
    }
    const size_t row = ((size_t)b * a.Hq + h0 + hh) * P1 + blockIdx.x;
    a.part_o[row * kD + j] = num;
    if (j == 0) {
      a.part_ml[row * 2] = mstar;
      a.part_ml[row * 2 + 1] = den;
    }
  }

}

}  // namespace

bool decode_fast_supported(const DecodeArgs &a) {
  return a.d == 128 && a.bits_k == 2 && (a.bits_v == 2 || a.bits_v == 3) && (a.G == 4 || a.G == 8);
}

int decode_fast_partials(const DecodeArgs &a) { return (a.P + kWaves - 1) / kWaves; }

// Waves of the MFMA decode the GPU holds at once for (G, bits_v); 0 if unknown.
int decode_fast_resident_waves(int G, int bits_v) {
  static int cache[2][2] = {{-1, -1}, {-1, -1}};
  int &c = cache[G == 8][bits_v == 3];
  if (c >= 0) return c;
  const void *fn = (G == 4) ? (bits_v == 2 ? (const void *)decode_fast_kernel<4, 2> : (const void *)decode_fast_kernel<4, 3>)
                            : (bits_v == 2 ? (const void *)decode_fast_kernel<8, 2> : (const void *)decode_fast_kernel<8, 3>);
  int dev = 0, blocks = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kThreads, 0) != hipSuccess) {
    hipGetLastError();
    return 0;
  }
  c = blocks * kWaves * prop.multiProcessorCount;
  return c;
}

hipError_t launch_decode_fast(const DecodeArgs &a, hipStream_t s) {
  const int nwg = (a.P + kWaves - 1) / kWaves;
  dim3 grid(nwg, a.B * a.Hkv);
  if (a.G == 4 && a.bits_v == 2) hipLaunchKernelGGL((decode_fast_kernel<4, 2>), grid, dim3(kThreads), 0, s, a, nwg);
  else if (a.G == 4) hipLaunchKernelGGL((decode_fast_kernel<4, 3>), grid, dim3(kThreads), 0, s, a, nwg);
  else if (a.bits_v == 2) hipLaunchKernelGGL((decode_fast_kernel<8, 2>), grid, dim3(kThreads), 0, s, a, nwg);
  else hipLaunchKernelGGL((decode_fast_kernel<8, 3>), grid, dim3(kThreads), 0, s, a, nwg);
  return hipGetLastError();
}

}  // namespace wushkv
