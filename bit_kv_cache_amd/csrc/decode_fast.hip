// GQA decode attention over the quantized cache on MFMA (gfx950), head_dim 128,
// G = 4 or 8 query heads per KV head, 2-, 3- or 4-bit keys and values.
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
// KV partition through a two-slot LDS ring filled by load-to-LDS DMA (the next set is
// in flight while the current one is computed):
//   QK: v_mfma_scale_f32_16x16x128_f8f6f4 on fp4 x fp4, A = q~ as eight balanced
//       base-8 digits (integers in [-4, 3], exact in e2m1) on one fixed-point grid per
//       head, B = the key codes (a code c in a nibble's low bits is exactly c / 2), so
//       each dot product is exact and q~ keeps ~23 bits.  Rows of the result are (head,
//       digit), columns tokens; the digits are summed per lane, smallest first.
//   softmax: online, base 2, per head (DPP reductions over the 16 token columns);
//       W = p * s_V as an fp16 hi + lo pair, passed through LDS as the PV A operand.
//   PV: v_mfma_f32_16x16x32_f16.  A = W rows (head) over the set's tokens, B = value
//       codes read straight from the set layout: a field pair is one and/or with an
//       fp16 exponent pattern, giving BASE + c (BASE = 4, 16 or 64 by the pair's
//       position); BASE * W is removed exactly through the per-head zero term.  W
//       enters as two MFMAs (hi and lo fp16 parts), so its rounding does not show.
// The FP16 sink + recent tokens go through the same ring, 8 rows per stage, on fp32
// VALU in a softmax partial of their own.  Each workgroup merges its 4 waves in LDS
// and writes one partial (m, l, o); the merge kernel that follows on the stream
// combines the partials.
// With one 12-wave workgroup per KV head (the whole layout: 12 partitions, no merge
// kernel) each set is copied from its slot into registers as soon as it lands and the
// slot takes the next-but-one set at once, so two sets are in flight while one
// computes; the window stages go to the first wave of each SIMD, after its sets.
#include <type_traits>

#include "wushkv_internal.h"

namespace wushkv {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
// Waves per workgroup: kSplitWaves when a KV head's partitions span several workgroups
// (their partials merged by merge_kernel), kWholeWaves when one workgroup holds all of a
// KV head's partitions and writes its output directly.
constexpr int kSplitWaves = 4;
constexpr int kWholeWaves = 12;
constexpr float kLog2e = 1.4426950408889634f;

// DPP encodings (gfx9): row_ror:n = 0x120 + n rotates within a row of 16 lanes,
// quad_perm [2,3,0,1] = 0x4E and [1,0,3,2] = 0xB1 swap within groups of four lanes.
template <int CTRL, int BANK = 0xF>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, BANK, false));
}

// Byte layout of one ring slot.  A body set: key codes (64 rows verbatim: 2 KB at 2
// bits, 4 KB at 4 bits, each row its low-bit plane then its high-bit plane), value
// codes (2 KB: the first 16 bytes of each lane's 32, then the last 16), the values'
// second plane (3 bits: the third-bit plane, 1 KB verbatim; 4 bits: the high two bits,
// 2 KB laid out as the first), key then value parameters (up to 256 B each).  A window
// stage: 8 FP16 key rows (2 KB) then 8 FP16 value rows (2 KB).
// Both kinds are filled by exactly DMAS load-to-LDS instructions, so one vmcnt per
// pending slot covers either.
template <int BK, int BV>
struct Stage {
  static constexpr int KROW = 16 * BK;                     // key row bytes (d = 128)
  static constexpr int K = 0, V = 64 * KROW, VH = V + 2048;
  static constexpr int VHB = BV == 3 ? 1024 : (BV == 4 ? 2048 : 0);
  static constexpr int KP = VH + VHB, VP = KP + 256, SIZE = VP + 256;
  static constexpr int WK = 0, WV = 2048;
  static constexpr int DMAS = V / 1024 + 2 + VHB / 1024 + 1;
};

// Row pitch (dwords) of the W buffer: rows 16 banks apart, so the 64 lanes' W stores
// (4 heads x 16 tokens) hit each bank twice and the PV operand reads (16 rows x 4
// column quads) spread over all eight 4-bank groups.
constexpr int kWbPitch = 80;

constexpr int kStages = 2;   // ring slots per wave: the item computed and kStages - 1 ahead

template <int G, int BK, int BV, int NW>
struct __align__(16) FastSmem {
  unsigned qi[G][kD];             // q~ in fixed point, offset to unsigned (balanced digits)
  float q[G][kD];
  union {
    unsigned wb[NW][G][kWbPitch];   // body set: W as fp16 (hi | lo << 16) [head][token]
    float qT[kD][G];              // query setup: q transposed (a channel's G heads in one read)
  };
  unsigned wzero[kSet];           // zeros: the PV A rows past 2 G read these
  int qe[16];                     // per head: q~ = (qi - kDigitBias) 2^(e - 21)
  float wp[NW][G][8];             // window stage: probabilities [head][token]
  alignas(16) float wmx[16][NW];  // window partial: max and sum [head][wave]
  alignas(16) float wls[16][NW];
  union {
    uint8_t ring[NW][kStages][Stage<BK, BV>::SIZE];
    struct {
      float o[NW][2 * G][kD];     // per wave: PV rows (hi parts, then lo parts), channels
      float wo[NW][G][kD];        // window partial: weighted FP16 values [head][channel]
    };
  } u;
  float sq[16];                   // per head: sum of q~ (the zero-point term)
  alignas(16) float m[16][NW];    // body partial: max, sum, zero term [head][wave]
  alignas(16) float l[16][NW];
  alignas(16) float z[16][NW];
  unsigned aqw[G / 2][4][64];     // q~ digit operands [operand][register][lane], shared by the waves
};

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
// A 3-bit code c = c2 + 4 h enters as two operands on the same A: the 2-bit part c2
// as above, and h alone at mantissa bit p = 6 + (k & 3) of an fp16 whose unit there
// is 4, i.e. HBASE + 4 h with HBASE = 64 >> (k & 3).  The sixteen third bits of a word
// come as a halfword of the high-bit plane; a byte permute puts pair k's two bits at
// (k, 16 + k), and shifts by 6 (pairs 0-3) and 2 (pairs 4-7) carry them to p.
struct VConst {
  unsigned m2, m3, m4, e2, e3, e4;  // masks and exponent patterns of positions 2, 3, 4
  unsigned mh[4], eh[4];            // third bit at mantissa 6 + i, unit 4
};

__device__ __forceinline__ VConst make_vconst() {
  VConst c;
  c.m2 = vconst(0x00300030u); c.e2 = vconst(0x54005400u);
  c.m3 = vconst(0x00C000C0u); c.e3 = vconst(0x4C004C00u);
  c.m4 = vconst(0x03000300u); c.e4 = vconst(0x44004400u);
  c.mh[0] = vconst(0x00400040u); c.eh[0] = c.e2;                  // 2^6 (1 + m / 1024)
  c.mh[1] = vconst(0x00800080u); c.eh[1] = vconst(0x50005000u);   // 2^5
  c.mh[2] = vconst(0x01000100u); c.eh[2] = c.e3;                  // 2^4
  c.mh[3] = vconst(0x02000200u); c.eh[3] = vconst(0x48004800u);   // 2^3
  return c;
}

// The same masks with every exponent two higher: the fields read as 4 BASE + 4 c, the
// high two bits of a 4-bit value code at their weight.
__device__ __forceinline__ VConst make_vconst_x4() {
  VConst c = make_vconst();
  c.e2 = vconst(0x5C005C00u);
  c.e3 = vconst(0x54005400u);
  c.e4 = vconst(0x4C004C00u);
  return c;
}

__device__ __forceinline__ unsigned and_or(unsigned x, unsigned m, unsigned o) { return (x & m) | o; }

// BASE of value pair k for 2-bit codes (see above): k = 0,2,5 -> 64; 1,3,6 -> 16; 4,7 -> 4.
__device__ __forceinline__ float vbase2(int k) {
  return (k == 4 || k == 7) ? 4.0f : ((k == 1 || k == 3 || k == 6) ? 16.0f : 64.0f);
}

// B operand of PV instruction iota (pairs 4*iota .. 4*iota+3) from one value word,
// the 2-bit codes (or the low two bits of 3-bit codes).
__device__ __forceinline__ f16x8 v_operand2(unsigned w, int iota, const VConst &c) {
  u32x4 r;
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
  return __builtin_bit_cast(f16x8, r);
}

// The same for the third bits, x = the word's sixteen third bits with pair k at (k, 16 + k).
__device__ __forceinline__ f16x8 v_operand_hi(unsigned x, int iota, const VConst &c) {
  const unsigned xs = iota == 0 ? x << 6 : x << 2;
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = and_or(xs, c.mh[i], c.eh[i]);
  return __builtin_bit_cast(f16x8, r);
}

// QK on v_mfma_scale_f32_16x16x128_f8f6f4 with A = q~ digits and B = key codes, both
// fp4 e2m1 (a 2-bit code c in the low bits of a nibble is exactly c / 2).  Operand map
// of that instruction (16 x 16 x 128) for fp4: lane l holds row (A) / column (B) l % 16,
// K-slots 32 (l / 16) + nibble (low nibble first); the E8M0 scale byte of lane l scales
// its row (A) / column (B) over K-block l / 16.
// A key word (16 codes, code f at bits 2f) gives two B dwords with one mask each:
// (w & 0x33333333) holds the even codes, ((w >> 2) & 0x33333333) the odd ones, so
// K-slot 32 g + 8 d + i of lane group g reads channel 32 g + 16 (d >> 1) + 2 i + (d & 1).
__device__ __forceinline__ int kslot_channel(int k) {
  const int g = k >> 5, n = k & 31, d = n >> 3, i = n & 7;
  return 32 * g + 16 * (d >> 1) + 2 * i + (d & 1);
}


// q~ enters the QK MFMA as eight balanced base-8 digits, integers in [-4, 3], which
// e2m1 holds exactly: u = Q + kDigitBias (|Q| <= 2^22) makes them the unsigned 3-bit
// fields of u, digit j = field 7 - j minus 4.
constexpr unsigned kDigitBias = 0x924924u;
// e2m1 nibble of the digit with field value f (digit f - 4), nibble f of this word.
constexpr unsigned kDigitE2M1 = 0x5420ACDEu;

// Head and digit of row r of q~ operand m: head quad m / 2, rows 4 h + i hold digit
// 4 (m % 2) + i of head 4 (m / 2) + h, so a lane's four result rows are one head's digits.
__device__ __forceinline__ void digit_row(int m, int r, int &h, int &j) {
  h = 4 * (m >> 1) + (r >> 2);
  j = 4 * (m & 1) + (r & 3);
}

__device__ __forceinline__ i32x8 key_fp4(u32x2 w) {
  const unsigned M = 0x33333333u;
  return (i32x8){(int)(w[0] & M), (int)((w[0] >> 2) & M), (int)(w[1] & M), (int)((w[1] >> 2) & M), 0, 0, 0, 0};
}

// A 3-bit key row's third bits for the lane's 32 channels (one plane-1 word: channel f
// at bit 4 ((f >> 1) & 7) + (f & 1) + 2 (f >> 4)) as fp4 operand words in key_fp4's
// channel order: each set bit becomes bit 2 of its nibble, the e2m1 value 2.
__device__ __forceinline__ i32x8 key_bits_fp4(unsigned p) {
  const unsigned M = 0x44444444u;
  return (i32x8){(int)((p << 2) & M), (int)((p << 1) & M), (int)(p & M), (int)((p >> 1) & M), 0, 0, 0, 0};
}

// Max / sum over the 16 lanes of a row (DPP rotations within the row, then quad swaps).
// The max is one v_max_f32 with a DPP source per step (its inputs are never NaN); each
// s_nop 1 gives the two wait states a DPP read needs after a VALU write of its source.
__device__ __forceinline__ float row_max(float x) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(x));
  return x;
}

// W = p s as an fp16 pair, hi = fp16(p s) in the low half and lo = fp16(p s - hi) in the
// high half (s the fp16 in the low half of s16): one v_fma_mix each, the product exact
// inside both, so hi + lo is p s to about 2^-22.
__device__ __forceinline__ unsigned w_hilo(float p, unsigned s16) {
  unsigned pk;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mixhi_f16 %0, %1, %2, -%0 op_sel_hi:[0,1,1]"
      : "=&v"(pk)
      : "v"(p), "v"(s16));
  return pk;
}

__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0x128>(x, x);
  x += dpp<0x124>(x, x);
  x += dpp<0x4E>(x, x);
  x += dpp<0xB1>(x, x);
  return x;
}

typedef __attribute__((address_space(3))) void lds_void;

// Word 3 of a raw buffer resource on gfx9 (32-bit dword data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

// Where a wave's body sets come from: buffer resources over its KV head's key and
// value code planes (a set's offset goes in an SGPR, so the lanes do no address
// arithmetic) and the lane's base in the parameter planes.
struct SetSource {
  __amdgpu_buffer_rsrc_t k, v;
  const uint8_t *par;   // keys' parameters (lanes < 16) or values' (lanes 16-31)
  int pstride;          // the lane's parameter bytes per set
  int vset;             // value-set bytes
  bool pact;            // the lane carries parameter bytes
};

// Queue the loads of body set `set` into the wave's ring slot `st` (load-to-LDS:
// lane i's bytes land at the slot offset + i * size).  Stage<BK, BV>::DMAS instructions.
template <int BK, int BV>
__device__ __forceinline__ void stage_set(const SetSource &src, int set, uint8_t *st) {
  using S = Stage<BK, BV>;
  const int lane = threadIdx.x & 63;
  constexpr int aux = 2;   // nontemporal: streamed once
  const unsigned vo = 16u * (unsigned)lane;
  const int ko = set * S::V, vso = set * src.vset;
#pragma unroll
  for (int i = 0; i < S::V / 1024; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.k, (lds_void *)(st + S::K + 1024 * i), 16, vo, ko + 1024 * i, 0, aux);
  // value words: lane l's 32 bytes split into its first 16 (slot bytes 16 l) and last
  // 16 (1024 + 16 l), so each of the lane's two 16-byte reads is contiguous across lanes
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void *)(st + S::V), 16, 2 * vo, vso, 0, aux);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void *)(st + S::V + 1024), 16, 2 * vo, vso + 16, 0, aux);
  if constexpr (BV == 3)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void *)(st + S::VH), 16, vo, vso + 2048, 0, aux);
  if constexpr (BV == 4) {   // the high two bits, laid out as the low ones
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void *)(st + S::VH), 16, 2 * vo, vso + 2048, 0, aux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.v, (lds_void *)(st + S::VH + 1024), 16, 2 * vo, vso + 2048 + 16, 0,
                                             aux);
  }
  // parameters, one instruction: lanes 0-15 the keys', 16-31 the values' (64 tokens x
  // 2 or 4 bytes each; lane 0 is always active, so the instruction always issues)
  if (src.pact)
    __builtin_amdgcn_global_load_lds(src.par + (size_t)set * src.pstride, (lds_void *)(st + S::KP), 16, 0, aux);
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
template <int BK, int BV>
__device__ __forceinline__ void stage_window(const uint8_t *sinkk, const uint8_t *sinkv, const uint8_t *ringk,
                                             const uint8_t *ringv, int t0, int cnt, int ns, unsigned first_slot,
                                             unsigned rsz, const void *filler, uint8_t *st) {
  using S = Stage<BK, BV>;
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

// Wait until at most `pending` (< kStages) staged items' loads are still in flight.
template <int BK, int BV>
__device__ __forceinline__ void wait_staged(int pending) {
  constexpr int D = Stage<BK, BV>::DMAS;
  static_assert(kStages >= 2 && kStages <= 4, "ring depth");
  if (pending <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (kStages == 2 || pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory");
  else if (kStages == 3 || pending == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * D) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * D) : "memory");
}

template <int G, int BK, int BV, int NW>
__device__ void window_stage(FastSmem<G, BK, BV, NW> &sm, const uint8_t *st, int cnt, int w, float (&wm)[G],
                             float (&wl)[G], float (&wacc)[G][2]);

// The workgroup's query setup: q and q~ of its G heads into LDS, per head the exponent
// e of max |q~| and sum(q~), then q~ on its fixed-point grid.  Every wave calls it.
// With a.tinvt the workgroup forms q~ = T^{-T} q itself (WUSH-KV digest, "method key
// points": one d x d product per query), in the query transform kernel's arithmetic:
// per row i of T^{-T} four interleaved fp32 partial sums (channels j = k mod 4, in
// ascending order), added as (s0 + s1) + (s2 + s3), so q~ is bit-identical to that
// kernel's.  Here the four partial sums of a row are four adjacent lanes, so a
// 12-wave workgroup spreads the product over 512 threads.  The partition-0 workgroup
// writes q~ to a.qt_out.
template <int G, int BK, int BV, int NW>
__device__ void setup_queries(const DecodeArgs &a, FastSmem<G, BK, BV, NW> &sm, int b, int h0) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x;
  const bool fused = a.tinvt != nullptr;
  for (int i = tid; i < G * kD; i += NT) {
    const int hh = i / kD, j = i % kD;
    const size_t off = ((size_t)b * a.Hq + h0 + hh) * kD + j;
    if (!fused) sm.qi[hh][j] = __float_as_uint(a.qt[off]);
    const float qv = load_in(a.q, a.q_dtype, off);
    sm.q[hh][j] = qv;
    sm.qT[j][hh] = qv;
  }
  __syncthreads();
  if (fused) {
    const float *M = a.tinvt + (size_t)(h0 / G) * kD * kD;
    // thread t: row i = t / 4, partial sum k = t % 4 (4 kD = 512 threads, whole waves)
    for (int t = tid; t < 4 * kD; t += NT) {
      const int i = t >> 2, k = t & 3;
      float mv[kD / 4];
#pragma unroll
      for (int m = 0; m < kD / 4; ++m) mv[m] = M[(size_t)i * kD + 4 * m + k];
      float s[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
#pragma unroll 2
      for (int m = 0; m < kD / 4; ++m) {
        float qv[G];
#pragma unroll
        for (int c = 0; c < G; c += 4) *(f32x4 *)&qv[c] = *(const f32x4 *)&sm.qT[4 * m + k][c];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[hh] = fmaf(mv[m], qv[hh], s[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        // (s0 + s1) + (s2 + s3) in lane k = 0 of the row's quad
        const float p = s[hh] + __shfl_xor(s[hh], 1, 4);
        const float v = p + __shfl_xor(p, 2, 4);
        if (k == 0) {
          sm.qi[hh][i] = __float_as_uint(v);
          if (blockIdx.x == 0) a.qt_out[((size_t)b * a.Hq + h0 + hh) * kD + i] = v;
        }
      }
    }
    __syncthreads();
  }
  // per head (one wave each): max |q~| and sum(q~) over the 128 channels, lane l
  // holding channels l and l + 64, then row reductions and the four rows' lane 0
  for (int hh = tid >> 6; hh < G; hh += NW) {
    const int l = tid & 63;
    const float v0 = __uint_as_float(sm.qi[hh][l]), v1 = __uint_as_float(sm.qi[hh][l + 64]);
    const float mr = row_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float sr = row_sum(v0 + v1);
    float mxa = 0.f, s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mxa = fmaxf(mxa, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 16 * r)));
      s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sr), 16 * r));
    }
    // |q~| < 2^(e + 1); heads below 2^-100 count as zero (their digits are all zero)
    if (l == 0) {
      sm.qe[hh] = mxa >= 0x1p-100f ? ilogbf(mxa) : -100;
      sm.sq[hh] = s;
    }
  }
  if (tid < kSet) sm.wzero[tid] = 0u;
  __syncthreads();
  // fixed point: Q = rint(q~ 2^(21 - e)), |Q| <= 2^22, stored as Q + kDigitBias
  for (int i = tid; i < G * kD; i += NT) {
    const int hh = i / kD, j = i % kD;
    const float v = __uint_as_float(sm.qi[hh][j]);
    const int Q = (int)rintf(ldexpf(v, 21 - sm.qe[hh]));
    sm.qi[hh][j] = (unsigned)(Q + (int)kDigitBias);
  }
  __syncthreads();
  // the fp4 A operands of the QK MFMA, the same for every wave: register d of operand m
  // for lane l holds nibbles i = 0..7 at K-slot 32 (l / 16) + 8 d + i of row l % 16
  for (int e = tid; e < (G / 2) * 4 * 64; e += NT) {
    const int m = e >> 8, d = (e >> 6) & 3, l = e & 63;
    int h, j;
    digit_row(m, l & 15, h, j);
    const int sft = 21 - 3 * j;
    unsigned word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned f = (sm.qi[h][kslot_channel(32 * (l >> 4) + 8 * d + i)] >> sft) & 7u;
      word |= ((kDigitE2M1 >> (4 * f)) & 15u) << (4 * i);
    }
    sm.aqw[m][d][l] = word;
  }
  __syncthreads();
}

// One wave of a KV partition: its 8-token stages [ws0, ws1) of the FP16 window list,
// then its body sets [s0, s1), all streamed through the wave's LDS ring.
// Lane (h, t) = (lane / 16, lane % 16) scores token 16 T + t of each set (T = 0..3) for
// heads h + 4 qd (qd < G / 4).  PV output row r (O lane l holds rows 4 (l / 16) + i,
// channels 16 ct + l % 16) is head r's hi part for r < G and head r - G's lo part for
// G <= r < 2 G; the two are summed in the workgroup merge.
template <int G, int BK, int BV, int NW, bool PAGED, bool APPEND>
__device__ void body_wave(const DecodeArgs &a, FastSmem<G, BK, BV, NW> &sm, int bg, int64_t s0, int64_t s1, int ws0, int ws1,
                          f32x4 (&O)[8], float (&m_out)[G / 4], float (&l_out)[G / 4], float (&z_out)[G / 4],
                          float (&wm_out)[G], float (&wl_out)[G], float (&wacc_out)[G][2]) {
  constexpr int NQ = G / 4;            // head quads: QK MFMAs per tile
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, t16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float qk_scale = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const int Lv = 1 << BV;
  const SeqLen sl = seq_len(a, bg / a.Hkv);   // this sequence's tokens and body tokens

  // Body sets are addressed by slot: the set index within this KV head's planes, or
  // with a paged body the set's place in the pools, (page Hkv + g) sets_per_page + the
  // set's index within its page (the resources then span the pools).
  constexpr bool paged = PAGED;
  const int sets_per_page = paged ? (int)(a.pg.page_tokens / kSet) : 1;
  SetSource src;
  {
    const size_t pool_sets = paged ? (size_t)a.pg.num_pages * a.Hkv * sets_per_page : 0;
    const size_t hb = paged ? 0 : (size_t)bg;
    const uint8_t *kplane = a.codes_k + hb * a.kcode_bytes;
    const uint8_t *vplane = a.codes_v + hb * a.vcode_bytes;
    const uint8_t *kpar = (const uint8_t *)a.par_k + hb * a.kpar_bytes;
    const uint8_t *vpar = (const uint8_t *)a.par_v + hb * a.vpar_bytes;
    const int kbytes = (int)(paged ? pool_sets * kSet * a.kcode_row : a.kcode_bytes);
    const int vbytes = (int)(paged ? pool_sets * a.vset_bytes : a.vcode_bytes);
    src.k = __builtin_amdgcn_make_buffer_rsrc((void *)kplane, 0, kbytes, kRsrcWord3);
    src.v = __builtin_amdgcn_make_buffer_rsrc((void *)vplane, 0, vbytes, kRsrcWord3);
    const int kb = a.kpar_n * 2, vbn = a.vpar_n * 2;
    const bool pk = lane < 4 * kb;
    src.pact = pk || (lane >= 16 && lane - 16 < 4 * vbn);
    src.par = pk ? kpar + 16 * lane : vpar + 16 * (lane - 16);
    src.pstride = 64 * (pk ? kb : vbn);
    src.vset = (int)a.vset_bytes;
  }
  uint8_t *ring = &sm.u.ring[w][0][0];
  constexpr int SB = Stage<BK, BV>::SIZE;
  // items of this wave: 8-token window stages ws0 .. ws1-1 and body sets s0 .. s1-1
  const int nb = (int)(s1 - s0), nitems = nb + (ws1 - ws0);
  const int ns = (int)(sl.n < a.S ? sl.n : a.S);
  const int nw = ns + (int)(sl.n - a.S - sl.nq > 0 ? sl.n - a.S - sl.nq : 0);
  const unsigned rsz = (unsigned)(a.R + a.C);
  const unsigned first_slot = sl.nq < 0x80000000ll ? (unsigned)sl.nq % rsz : (unsigned)(sl.nq % rsz);
  const uint8_t *sinkk = (const uint8_t *)a.sink_k + (size_t)bg * a.sink_bytes;
  const uint8_t *sinkv = (const uint8_t *)a.sink_v + (size_t)bg * a.sink_bytes;
  const uint8_t *ringk = (const uint8_t *)a.ring_k + (size_t)bg * a.ring_bytes;
  const uint8_t *ringv = (const uint8_t *)a.ring_v + (size_t)bg * a.ring_bytes;
  // the split layout runs the window stages first (their VALU work then overlaps the
  // other waves' streaming rather than forming every wave's tail), then the body sets
  const int nwin = ws1 - ws0;
  const int bq = bg / a.Hkv, gq = bg % a.Hkv;
  // paged: the wave's pages are read once, lane i holding the (i + lp0)-th logical
  // page's physical page, and each set takes its own with a readlane; a range of more
  // than 64 pages reads the table per set.  An invalid entry reads page 0.
  int lp0 = 0, wave_pages = 0;
  bool pages_in_lanes = false;
  if constexpr (PAGED) {
    lp0 = (int)(s0 / sets_per_page);
    const int lp_end = (int)((s1 + sets_per_page - 1) / sets_per_page);
    pages_in_lanes = lp_end - lp0 <= 64;
    const int lp = lp0 + lane;
    int pg = 0;
    if (pages_in_lanes && lp < lp_end && lp < a.pg.max_pages) pg = a.pg.table[(int64_t)bq * a.pg.max_pages + lp];
    wave_pages = pg < 0 || pg >= a.pg.num_pages ? 0 : pg;
  }
  auto slot_of = [&](int set) {
    if (!paged) return set;
    const int lp = set / sets_per_page;
    int page;
    if (pages_in_lanes) {
      page = __builtin_amdgcn_readlane(wave_pages, lp - lp0);
    } else {
      page = lp < a.pg.max_pages ? a.pg.table[(int64_t)bq * a.pg.max_pages + lp] : 0;
      if (page < 0 || page >= a.pg.num_pages) page = 0;
    }
    return (page * a.Hkv + gq) * sets_per_page + (set - lp * sets_per_page);
  };
  // The whole layout runs its window stages after its sets (on the first wave of each
  // SIMD only: see decode_fast_kernel) and copies each set into registers as it lands.
  constexpr bool kWinLast = NW == kWholeWaves;
  constexpr bool kEarly = NW == kWholeWaves;
  const int set_item0 = kWinLast ? 0 : nwin, win_item0 = kWinLast ? nb : 0;
  auto issue = [&](int item, uint8_t *dst) {
    if (kWinLast ? item < nb : item >= nwin) {
      stage_set<BK, BV>(src, slot_of((int)s0 + item - set_item0), dst);
    } else {
      const int t0 = 8 * (ws0 + item - win_item0);
      stage_window<BK, BV>(sinkk, sinkv, ringk, ringv, t0, nw - t0 < 8 ? nw - t0 : 8, ns, first_slot, rsz, a.qt, dst);
    }
  };
  // prologue: the first kStages items fill the ring (item k lives in slot k % kStages),
  // queued before the query setup so that the setup overlaps their loads
  for (int k = 0; k < kStages && k < nitems; ++k) issue(k, ring + k * SB);
  // Fused append of the step's new token (position n - 1, the last of the window list),
  // by the wave whose window stages end the list: lanes 0-15 take its key, 16-31 its
  // value.  The loads are queued with the query setup's and the fp16 row is stored to
  // its sink row or ring slot after it (a token already quantized was written by the
  // flush); nothing waits for that store.  This wave's own window stage then reads the
  // row from registers instead: it is written over the stage's staged copy once that
  // has landed.
  const bool appender = APPEND && nwin > 0 && ws1 == (nw + 7) / 8;
  const int64_t p_new = sl.n - 1;
  float raw_new[8];
  if (appender && lane < 32) {
    const size_t src = (size_t)bg * kD + 8 * (lane & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) raw_new[e] = load_in(lane >= 16 ? a.v_new : a.k_new, a.in_dtype, src + e);
  }
  setup_queries(a, sm, bg / a.Hkv, (bg % a.Hkv) * G);
  f16x8 row_new;
  if (appender && lane < 32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) row_new[e] = (_Float16)raw_new[e];
    const bool in_sink = p_new < a.S, in_ring = p_new >= a.S + sl.nq;
    if (in_sink || in_ring) {
      const int isv = lane >> 4;
      const uint8_t *dst = in_sink ? (isv ? sinkv : sinkk) + (size_t)p_new * (kD * 2)
                                   : (isv ? ringv : ringk) + (size_t)((p_new - a.S) % rsz) * (kD * 2);
      *(f16x8 *)(const_cast<uint8_t *>(dst) + 16 * (lane & 15)) = row_new;
    }
  }

  // q~ as eight balanced base-8 digits (integers in [-4, 3], exact in e2m1) on one fixed
  // point grid per head, in the rows of NM fp4 A operands: row r of operand m holds
  // digit j of head h (digit_row), weighted 2^(e - 3 j) through the row's E8M0 scale.
  // On a common grid every product of a digit MFMA is a multiple of 1/2 of magnitude
  // at most 6, which the matrix core sums exactly (it does not for operands of mixed
  // exponents).  Lane (g4, t16)'s result rows 4 g4 + i are digits of one head.
  constexpr int NM = G / 2;
  i32x8 aq[NM];
  int sa[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    int h, j;
    digit_row(m, lane & 15, h, j);
    aq[m] = (i32x8){(int)sm.aqw[m][0][lane], (int)sm.aqw[m][1][lane], (int)sm.aqw[m][2][lane],
                    (int)sm.aqw[m][3][lane], 0, 0, 0, 0};
    sa[m] = 127 + sm.qe[h] - 3 * j;
  }
  // scores in units of 1 / a_sc: s (q~ . c / 2) + z sum(q~) / 2 (the MFMA sums
  // q~ . (c / 2)); a_sc = 2 log2(e) / sqrt(d) turns them into base-2 logits
  const float a_sc = 2.0f * qk_scale;
  float b_sc[NQ];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) b_sc[qd] = 0.5f * sm.sq[4 * qd + g4];
  const VConst vc = make_vconst();
  VConst vc4;
  if constexpr (BV == 4) vc4 = make_vconst_x4();
  // BASE of the value operand for token 16 T + t16: pair 2 T + (t16 & 3) / 2 of its word
  float vbase[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const int k = 2 * T + ((t16 & 3) >> 1);
    vbase[T] = BV == 4 ? 5.0f * vbase2(k) : vbase2(k) + (BV == 3 ? (float)(64 >> (k & 3)) : 0.0f);
  }
  // PV A rows: row r < G is head r's W hi part, G <= r < 2 G head r - G's lo part (the
  // two halves of one word of the W buffer), zeros past 2 G
  const int ar = lane & 15;
  const unsigned *arow = ar < 2 * G ? &sm.wb[w][ar < G ? ar : ar - G][0] : &sm.wzero[0];
  const unsigned asel = ar < G ? 0x05040100u : 0x07060302u;

  // Items [0, issued) are queued; item k lives in slot k % kStages.  Before item it
  // computes: queue item it + kStages - 1 if its slot's last item has not already
  // queued it, then wait until item it landed.  A body set is copied from its slot into
  // registers as soon as it lands and its slot then takes item it + kStages at once
  // (release), so two sets are in flight while a set computes; a window stage reads its
  // slot while it computes and hands it on at the next advance.
  int issued = kStages < nitems ? kStages : nitems;
  auto advance = [&](int it) {
    if (issued == it + kStages - 1 && issued < nitems) {
      issue(issued, ring + (issued % kStages) * SB);
      ++issued;
    }
    wait_staged<BK, BV>(issued - 1 - it);
    return ring + (it % kStages) * SB;
  };
  auto release = [&](int it) {
    if (issued == it + kStages && issued < nitems) {
      // the slot's LDS reads have returned their data before the loads that overwrite it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(issued, ring + (issued % kStages) * SB);
      ++issued;
    }
  };
  // A body set's operands, read out of its ring slot: per tile T the lane's key words
  // (row 16 T + t16, the lane's 32 channels) and the parameters of token 16 T + t16,
  // and the lane's value words.
  struct SetRegs {
    u32x2 kw[4], kh[4];   // key words; kh: the row's second plane (3- and 4-bit keys)
    unsigned kp[4], vp[4];   // key / value parameters (fp16 scale, or scale | zero << 16)
    u32x4 v0, v1, vh0, vh1;  // value words; vh0 / vh1: the values' second plane
  };
  auto load_keys = [&](auto kq_tag, const uint8_t *st, SetRegs &r) {
    constexpr bool KQ = decltype(kq_tag)::value;
    using S = Stage<BK, BV>;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const uint8_t *kr = st + S::K + (16 * T + t16) * S::KROW + 8 * g4;
      r.kw[T] = *(const u32x2 *)kr;
      if constexpr (BK == 4) r.kh[T] = *(const u32x2 *)(kr + 32);
      if constexpr (BK == 3) r.kh[T][0] = *(const unsigned *)(kr + 32 - 4 * g4);
      const int u = 16 * T + t16;
      if constexpr (KQ) r.kp[T] = *(const unsigned short *)(st + S::KP + 2 * u);
      else r.kp[T] = *(const unsigned *)(st + S::KP + 4 * u);
    }
  };
  auto load_values = [&](auto vq_tag, const uint8_t *st, SetRegs &r) {
    constexpr bool VQ = decltype(vq_tag)::value;
    using S = Stage<BK, BV>;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int u = 16 * T + t16;
      if constexpr (VQ) r.vp[T] = *(const unsigned short *)(st + S::VP + 2 * u);
      else r.vp[T] = *(const unsigned *)(st + S::VP + 4 * u);
    }
    r.v0 = *(const u32x4 *)(st + S::V + 16 * lane);
    r.v1 = *(const u32x4 *)(st + S::V + 1024 + 16 * lane);
    if constexpr (BV == 3) r.vh0 = *(const u32x4 *)(st + S::VH + 16 * lane);
    if constexpr (BV == 4) {
      r.vh0 = *(const u32x4 *)(st + S::VH + 16 * lane);
      r.vh1 = *(const u32x4 *)(st + S::VH + 1024 + 16 * lane);
    }
  };

  float m_run[NQ], l_lane[NQ], zacc[NQ];
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) { m_run[qd] = -INFINITY; l_lane[qd] = 0.f; zacc[qd] = 0.f; }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) O[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // A 64-token set in two phases.  FULL: every token of the set is in the body (no
  // validity selects); KQ / VQ: QuEST (one scale per token) rather than affine (scale,
  // zero) parameters for the keys / values.
  // Phase 1: QK and scores; mxr = each head's max over the set.  Returns whether any
  // head's running max rises (the same in every lane).
  auto phase1 = [&](auto full_tag, auto kq_tag, int64_t set, const SetRegs &rg, float (&sc)[NQ][4],
                    float (&mxr)[NQ]) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool KQ = decltype(kq_tag)::value;
    using S = Stage<BK, BV>;
    const int64_t base = set * kSet;

    // ---- QK: one scaled MFMA per (tile, head quad); the lane's 4 result rows are the
    // digits of its head, already weighted
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const i32x8 bk = key_fp4(rg.kw[T]);
      // 4-bit keys: the row's second plane holds the high two bits, c = lo + 4 hi; its
      // products enter the same accumulation with B scaled by 4 (E8M0 129)
      i32x8 bh;
      if constexpr (BK == 4) bh = key_fp4(rg.kh[T]);
      // 3-bit keys: the row's second plane holds the third bits, c = lo + 4 h; a set bit
      // enters as the e2m1 value 2 (= 4 h / 2, on the low plane's scale)
      if constexpr (BK == 3) bh = key_bits_fp4(rg.kh[T][0]);
      // per head quad: digits 4-7 accumulate onto the rows of digits 0-3
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[2 * qd], bk, (f32x4){0.f, 0.f, 0.f, 0.f}, 4, 4,
                                                                   0, sa[2 * qd], 0, 127);
        d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[2 * qd + 1], bk, d, 4, 4, 0, sa[2 * qd + 1], 0, 127);
        if constexpr (BK >= 3) {
          constexpr int SB = BK == 4 ? 129 : 127;
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[2 * qd], bh, d, 4, 4, 0, sa[2 * qd], 0, SB);
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[2 * qd + 1], bh, d, 4, 4, 0, sa[2 * qd + 1], 0, SB);
        }
        sc[qd][T] = (d[3] + d[2]) + (d[1] + d[0]);
      }
    }
    // ---- scores and online softmax (base 2)
    float mx[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) mx[qd] = -INFINITY;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int u = 16 * T + t16;
      float s_t, z_t;
      if constexpr (KQ) {
        s_t = (float)__builtin_bit_cast(_Float16, (unsigned short)rg.kp[T]);
        z_t = -0.5f * (float)((1 << BK) - 1) * s_t;
      } else {
        const f16x2 pz = __builtin_bit_cast(f16x2, rg.kp[T]);
        s_t = (float)pz[0];
        z_t = (float)pz[1];
      }
      const bool valid = FULL || base + u < sl.nq;
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        sc[qd][T] = valid ? fmaf(s_t, sc[qd][T], z_t * b_sc[qd]) : -INFINITY;
        mx[qd] = fmaxf(mx[qd], sc[qd][T]);
      }
    }
    bool up = false;
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      mxr[qd] = row_max(mx[qd]);
      up |= mxr[qd] > m_run[qd];
    }
    return __any(up);
  };
  // A set raised a running max: rescale O, l and z to it (rare once a partition is
  // under way; kept out of the common path so the accumulators stay in place).
  auto rescale = [&](const float (&mxr)[NQ]) {
    float alpha[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      const float m_new = fmaxf(m_run[qd], mxr[qd]);
      alpha[qd] = __builtin_amdgcn_exp2f((m_run[qd] - m_new) * a_sc);
      m_run[qd] = m_new;
    }
    // O row r = 4 (l / 16) + i holds head r % G (hi part for r < G, lo part after):
    // its factor sits in lane group i, head quad (r % G) / 4
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[0]), 16 * i));
      if constexpr (NQ == 2) {
        const float f1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[1]), 16 * i));
        f[i] = (g4 & 1) ? f1 : f[i];
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[ct][i] *= f[i];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) {
      l_lane[qd] *= alpha[qd];
      zacc[qd] *= alpha[qd];
    }
  };
  // Phase 2: p and W = p s_V against the running max, then PV.
  auto phase2 = [&](auto full_tag, auto vq_tag, int64_t set, const SetRegs &rg, const float (&sc)[NQ][4]) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool VQ = decltype(vq_tag)::value;
    using S = Stage<BK, BV>;
    const int64_t base = set * kSet;
    // ---- p, W = p s_V as fp16 hi + lo into the wave's W buffer, zero term
    float m_sc[NQ];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) m_sc[qd] = m_run[qd] * a_sc;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const int u = 16 * T + t16;
      float s_t, z_t;
      unsigned s16;   // the token's value scale, fp16 in the low half
      if constexpr (VQ) {
        s16 = rg.vp[T];
        s_t = (float)__builtin_bit_cast(_Float16, (unsigned short)s16);
        z_t = -0.5f * (Lv - 1) * s_t;
      } else {
        s16 = rg.vp[T];
        const f16x2 pz = __builtin_bit_cast(f16x2, s16);
        s_t = (float)pz[0];
        z_t = (float)pz[1];
      }
      const bool valid = FULL || base + u < sl.nq;
      // the MFMA forms sum (hi + lo) (BASE + c); the zero term takes p z - BASE W with
      // W in place of hi + lo (they differ by ~2^-22 W)
      const float zb = fmaf(-vbase[T], s_t, z_t);
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[qd][T], a_sc, -m_sc[qd]));
        l_lane[qd] += p;
        zacc[qd] = valid ? fmaf(p, zb, zacc[qd]) : zacc[qd];
        sm.wb[w][4 * qd + g4][u] = w_hilo(valid ? p : 0.f, s16);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV on the f16 MFMA: instruction iota covers tiles 2 iota, 2 iota + 1; A row
    // r = head, K-slots 8 c .. 8 c + 7 = tokens 16 a + 4 c + e of those tiles
    const u32x4 vw0 = rg.v0, vw1 = rg.v1;
    const unsigned vws[8] = {vw0[0], vw0[1], vw0[2], vw0[3], vw1[0], vw1[1], vw1[2], vw1[3]};
    unsigned hx[8];
    if constexpr (BV == 3) {
      const u32x4 vh = rg.vh0;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        hx[ct] = __builtin_amdgcn_perm(0u, vh[ct >> 1], (ct & 1) ? 0x0C030C02u : 0x0C010C00u);
    }
    if constexpr (BV == 4) {   // the high two bits' words, laid out as the low ones'
      const u32x4 h0 = rg.vh0, h1 = rg.vh1;
#pragma unroll
      for (int c = 0; c < 4; ++c) { hx[c] = h0[c]; hx[4 + c] = h1[c]; }
    }
#pragma unroll
    for (int iota = 0; iota < 2; ++iota) {
      const u32x4 x0 = *(const u32x4 *)(arow + 16 * (2 * iota) + 4 * g4);
      const u32x4 x1 = *(const u32x4 *)(arow + 16 * (2 * iota + 1) + 4 * g4);
      const u32x4 av = {__builtin_amdgcn_perm(x0[1], x0[0], asel), __builtin_amdgcn_perm(x0[3], x0[2], asel),
                        __builtin_amdgcn_perm(x1[1], x1[0], asel), __builtin_amdgcn_perm(x1[3], x1[2], asel)};
      const f16x8 Aw = __builtin_bit_cast(f16x8, av);
#pragma unroll
      for (int ct0 = 0; ct0 < 8; ct0 += 4) {
        f16x8 Bv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) Bv[c] = v_operand2(vws[ct0 + c], iota, vc);
#pragma unroll
        for (int c = 0; c < 4; ++c) O[ct0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aw, Bv[c], O[ct0 + c], 0, 0, 0);
        if constexpr (BV == 3) {
#pragma unroll
          for (int c = 0; c < 4; ++c) Bv[c] = v_operand_hi(hx[ct0 + c], iota, vc);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            O[ct0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aw, Bv[c], O[ct0 + c], 0, 0, 0);
        }
        if constexpr (BV == 4) {   // 4 BASE + 4 h on the same A
#pragma unroll
          for (int c = 0; c < 4; ++c) Bv[c] = v_operand2(hx[ct0 + c], iota, vc4);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            O[ct0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aw, Bv[c], O[ct0 + c], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // items: items it + 1 .. it + kStages - 1 are staged while item it computes.  The
  // loop takes the full sets; the rescale is marked unlikely, which keeps it out of line
  // and the PV accumulators in place from set to set (with it inline the compiler
  // copies them around every set).  The ragged last set, if any, comes after.
  using FullTag = std::integral_constant<bool, true>;
  using TailTag = std::integral_constant<bool, false>;
  auto body_sets = [&](auto kq_tag, auto vq_tag) {
    const int64_t full_end = sl.nq / kSet;   // sets below this index are full
    const int nfull = full_end <= s0 ? 0 : (int)(full_end - s0 < nb ? full_end - s0 : nb);
    float sc[NQ][4], mxr[NQ];
    SetRegs rg;
    int it = 0;
    // kEarly: the whole set into registers, then its slot is released; otherwise the
    // value half is read after the scores (fewer registers live through the QK part)
    for (; it < nfull; ++it) {
      const uint8_t *st = advance(set_item0 + it);
      load_keys(kq_tag, st, rg);
      if constexpr (kEarly) { load_values(vq_tag, st, rg); release(set_item0 + it); }
      if (__builtin_expect(phase1(FullTag{}, kq_tag, s0 + it, rg, sc, mxr), 0)) rescale(mxr);
      if constexpr (!kEarly) load_values(vq_tag, st, rg);
      phase2(FullTag{}, vq_tag, s0 + it, rg, sc);
    }
    for (; it < nb; ++it) {
      const uint8_t *st = advance(set_item0 + it);
      load_keys(kq_tag, st, rg);
      if constexpr (kEarly) { load_values(vq_tag, st, rg); release(set_item0 + it); }
      if (phase1(TailTag{}, kq_tag, s0 + it, rg, sc, mxr)) rescale(mxr);
      if constexpr (!kEarly) load_values(vq_tag, st, rg);
      phase2(TailTag{}, vq_tag, s0 + it, rg, sc);
    }
  };
  float wm[G], wl[G], wacc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { wm[h] = -INFINITY; wl[h] = 0.f; wacc[h][0] = wacc[h][1] = 0.f; }
  auto windows = [&]() {
  for (int it = 0; it < nwin; ++it) {
    const uint8_t *st = advance(win_item0 + it);
    const int t0 = 8 * (ws0 + it);
    if (appender && it == nwin - 1) {
      // the new token is row nw - 1 - t0 of the last stage (key rows at WK, values at WV)
      if (lane < 32)
        *(f16x8 *)(const_cast<uint8_t *>(st) + (lane < 16 ? Stage<BK, BV>::WK : Stage<BK, BV>::WV) +
                   256 * (nw - 1 - t0) + 16 * (lane & 15)) = row_new;
      __builtin_amdgcn_wave_barrier();
    }
    window_stage<G, BK, BV, NW>(sm, st, nw - t0 < 8 ? nw - t0 : 8, w, wm, wl, wacc);
  }
  };
  using Yes = std::true_type;
  using No = std::false_type;
  if (!kWinLast) windows();
  if (a.quant_k == WUSHKV_Q_QUEST) {
    if (a.quant_v == WUSHKV_Q_QUEST) body_sets(Yes{}, Yes{});
    else body_sets(Yes{}, No{});
  } else {
    if (a.quant_v == WUSHKV_Q_QUEST) body_sets(No{}, Yes{});
    else body_sets(No{}, No{});
  }
  if (kWinLast) windows();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    wm_out[h] = wm[h];
    wl_out[h] = wl[h];
    wacc_out[h][0] = wacc[h][0];
    wacc_out[h][1] = wacc[h][1];
  }

  // per-head totals; every lane of head 4 qd + lane / 16 holds them
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    m_out[qd] = m_run[qd] * a_sc;
    l_out[qd] = row_sum(l_lane[qd]);
    z_out[qd] = row_sum(zacc[qd]);
  }
}

// One window stage: cnt <= 8 FP16 window tokens in a ring slot, on fp32 VALU.  Scores:
// 8 lanes per token, 16 channels each, summed over the 8 with DPP; values: lane = two
// channels.  The stage folds into this wave's window partial: per head the running
// max and sum (the same in every lane) and this lane's two weighted value channels.
template <int G, int BK, int BV, int NW>
__device__ void window_stage(FastSmem<G, BK, BV, NW> &sm, const uint8_t *st, int cnt, int w, float (&wm)[G],
                             float (&wl)[G], float (&wacc)[G][2]) {
  using S = Stage<BK, BV>;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 3, cc = lane & 7;   // token of the stage, 16-channel chunk
  const float qk_scale = kLog2e * 0.08838834764831845f;
  const bool valid = j < cnt;
  const f16x8 k0 = *(const f16x8 *)(st + S::WK + 256 * j + 32 * cc);
  const f16x8 k1 = *(const f16x8 *)(st + S::WK + 256 * j + 32 * cc + 16);
  float kf[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kf[e] = (float)k0[e];
    kf[8 + e] = (float)k1[e];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 qv = *(const f32x4 *)&sm.q[h][16 * cc + 4 * c];
#pragma unroll
      for (int e = 0; e < 4; ++e) x = fmaf(qv[e], kf[4 * c + e], x);
    }
    // sum over the token's 8 lanes (quad swaps, then the half-row mirror pairs the quads)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf"
        : "+v"(x));
    // every lane of token j holds its score; a row holds tokens 2r and 2r + 1, so the
    // max and sum over the 8 tokens are a row_ror:8 step and the four rows' lane 0
    const float sc = valid ? x * qk_scale : -INFINITY;
    float mr = sc;
    asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf" : "+v"(mr));
    const float mx = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 0)),
                                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 16))),
                           fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 32)),
                                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr), 48))));
    const float mn = fmaxf(wm[h], mx);
    const float al = __builtin_amdgcn_exp2f(wm[h] - mn);
    const float pr = valid ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
    float pp = pr;
    asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf" : "+v"(pp));
    const float ps = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 0)) +
                      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 16))) +
                     (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 32)) +
                      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 48)));
    if (cc == 0) sm.wp[w][h][j] = pr;
    wl[h] = wl[h] * al + ps;
    wm[h] = mn;
    wacc[h][0] *= al;
    wacc[h][1] *= al;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // values: lane = two channels; rows past cnt hold a copy of the first token and have
  // probability 0
  f32x4 pw[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    pw[h][0] = *(const f32x4 *)&sm.wp[w][h][0];
    pw[h][1] = *(const f32x4 *)&sm.wp[w][h][4];
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const f16x2 vv = *(const f16x2 *)(st + S::WV + 256 * u + 4 * lane);
    const float v0 = (float)vv[0], v1 = (float)vv[1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = pw[h][u >> 2][u & 3];
      wacc[h][0] = fmaf(pr, v0, wacc[h][0]);
      wacc[h][1] = fmaf(pr, v1, wacc[h][1]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// nwg_body workgroups per KV head; with one, the workgroup's merge is the output.
template <int G, int BK, int BV, int NW, bool PAGED, bool APPEND>
__global__ void __launch_bounds__(64 * NW) decode_fast_kernel(DecodeArgs a, int nwg_body) {
  constexpr int NT = 64 * NW;
  __shared__ FastSmem<G, BK, BV, NW> sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int h0 = g * G;

  f32x4 O[8];
  float bm[G / 4], bl[G / 4], bz[G / 4];
#pragma unroll
  for (int qd = 0; qd < G / 4; ++qd) { bm[qd] = -INFINITY; bl[qd] = 0.f; bz[qd] = 0.f; }
  float wm[G], wl[G], wacc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { wm[h] = -INFINITY; wl[h] = 0.f; wacc[h][0] = wacc[h][1] = 0.f; }
  // every wave runs body_wave (its query setup is workgroup-wide); waves past the last
  // partition get empty ranges
  const int part = (int)blockIdx.x * NW + w;
  int64_t s0 = 0, s1 = 0;
  int ws0 = 0, ws1 = 0;
  if (part < a.P) {
    const SeqLen sl = seq_len(a, b);
    const int64_t nsets = (sl.nq + kSet - 1) / kSet;
    const int64_t ns = sl.n < a.S ? sl.n : a.S;
    const int64_t nw = ns + (sl.n - a.S - sl.nq > 0 ? sl.n - a.S - sl.nq : 0);
    const int64_t nws = (nw + 7) / 8;
    // (the whole layout runs only with P = kWholeWaves: a constant divisor there)
    const int64_t P = NW == kWholeWaves ? (int64_t)kWholeWaves : (int64_t)a.P;
    ws0 = (int)(nws * part / P);
    ws1 = (int)(nws * (part + 1) / P);
    const int64_t items = nsets + nws;
    if (NW == kWholeWaves && nsets >= P && items >= 3 * nws + P) {
      // Whole layout: every wave takes an equal share of all items, but the window
      // stages all go to waves 0-3, the first wave of each SIMD, which the SIMD's
      // instruction arbiter favours (those finish their share first, the SIMD's last
      // wave about a third of the body later); they run them after their sets, while
      // the other waves still stream.  Measured 2-3% faster than a window share per
      // wave run first, on the batched-serving shape.
      auto wb = [&](int p) { return nws * (p < 4 ? p : 4) / 4; };
      ws0 = (int)wb(part);
      ws1 = (int)wb(part + 1);
      s0 = items * part / P - ws0;
      s1 = items * (part + 1) / P - ws1;
    } else if (nsets >= P) {
      // an equal share of all items (window stages and sets) per partition: its window
      // stages as above, sets for the rest (the two shares rounded apart left the
      // partitions 45-47 items long on the serving shape, now 46 each)
      s0 = items * part / P - ws0;
      s1 = items * (part + 1) / P - ws1;
    } else {
      s0 = nsets * part / P;
      s1 = nsets * (part + 1) / P;
    }
  }
  body_wave<G, BK, BV, NW, PAGED, APPEND>(a, sm, bg, s0, s1, ws0, ws1, O, bm, bl, bz, wm, wl, wacc);
  // A wave's partial (PV rows, then window values) goes to its own ring slots when they
  // hold it (the whole layout: no wave reads another's slots and the wave's own loads
  // have all landed), so a wave writes it as soon as it is done; otherwise to u.o / u.wo,
  // which alias every wave's ring, after all waves are done.
  constexpr bool kOwnSlots = NW == kWholeWaves && kStages * Stage<BK, BV>::SIZE >= 3 * G * kD * 4;
  auto part_o = [&](int ww) -> float * {
    if constexpr (kOwnSlots) return (float *)&sm.u.ring[ww][0][0];
    else return &sm.u.o[ww][0][0];
  };
  auto part_w = [&](int ww) -> float * {
    if constexpr (kOwnSlots) return (float *)&sm.u.ring[ww][0][0] + 2 * G * kD;
    else return &sm.u.wo[ww][0][0];
  };
  if constexpr (!kOwnSlots) __syncthreads();  // every wave is done with its ring
  float *po = part_o(w), *pw = part_w(w);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    pw[h * kD + 2 * lane] = wacc[h][0];
    pw[h * kD + 2 * lane + 1] = wacc[h][1];
    if (lane == 0) { sm.wmx[h][w] = wm[h]; sm.wls[h][w] = wl[h]; }
  }
  {
    // rows of O are heads; lane 16 hh + t of head quad qd carries head 4 qd + hh's totals
    const int q4 = lane >> 4, col = lane & 15;
    if (col == 0) {
#pragma unroll
      for (int qd = 0; qd < G / 4; ++qd) {
        sm.m[4 * qd + q4][w] = bm[qd];
        sm.l[4 * qd + q4][w] = bl[qd];
        sm.z[4 * qd + q4][w] = bz[qd];
      }
    }
    if (4 * q4 < 2 * G) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) po[(4 * q4 + i) * kD + 16 * ct + col] = O[ct][i];
    }
  }
  __syncthreads();

  // ---- merge the workgroup's waves: its partial, or the output when it is the only
  // workgroup of its KV head.  Each thread takes four adjacent channels of one head and
  // forms its head's merge itself: the max over the waves' non-empty body and window
  // partials, each partial's factor 2^(m - max) (0 when empty), the denominator and the
  // weighted sums of the partials (per channel in the same order as one channel a thread).
  const int P1 = a.P + 1;
  const bool direct = nwg_body == 1;
  for (int i = tid; i < G * kD / 4; i += NT) {
    const int hh = i / (kD / 4), j = 4 * (i % (kD / 4));
    float mv[NW], lv[NW], zv[NW], wmv[NW], wlv[NW];
#pragma unroll
    for (int c = 0; c < NW; c += 4) {
      *(f32x4 *)&mv[c] = *(const f32x4 *)&sm.m[hh][c];
      *(f32x4 *)&lv[c] = *(const f32x4 *)&sm.l[hh][c];
      *(f32x4 *)&zv[c] = *(const f32x4 *)&sm.z[hh][c];
      *(f32x4 *)&wmv[c] = *(const f32x4 *)&sm.wmx[hh][c];
      *(f32x4 *)&wlv[c] = *(const f32x4 *)&sm.wls[hh][c];
    }
    float mstar = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (lv[ww] > 0.f) mstar = fmaxf(mstar, mv[ww]);
      if (wlv[ww] > 0.f) mstar = fmaxf(mstar, wmv[ww]);
    }
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      // an empty partial has factor 0 and finite (zero) sums
      const float fb = lv[ww] > 0.f ? __builtin_amdgcn_exp2f(mv[ww] - mstar) : 0.f;
      const float fw = wlv[ww] > 0.f ? __builtin_amdgcn_exp2f(wmv[ww] - mstar) : 0.f;
      den = fmaf(fb, lv[ww], den);
      den = fmaf(fw, wlv[ww], den);
      const float *o = part_o(ww);
      const f32x4 oh = *(const f32x4 *)&o[hh * kD + j], ol = *(const f32x4 *)&o[(G + hh) * kD + j];
      const f32x4 wv = *(const f32x4 *)&part_w(ww)[hh * kD + j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        num[e] = fmaf(fb, zv[ww] + (oh[e] + ol[e]), num[e]);
        num[e] = fmaf(fw, wv[e], num[e]);
      }
    }
    if (direct) {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = num[e] / den;
      *(f32x4 *)&a.out[((size_t)b * a.Hq + h0 + hh) * kD + j] = r;
    } else {
      const size_t row = ((size_t)b * a.Hq + h0 + hh) * P1 + blockIdx.x;
      *(f32x4 *)&a.part_o[row * kD + j] = num;
      if (j == 0) {
        a.part_ml[row * 2] = mstar;
        a.part_ml[row * 2 + 1] = den;
      }
    }
  }
}

}  // namespace

bool decode_fast_supported(const DecodeArgs &a) {
  // buffer resources address each KV head's code planes (or, paged, the whole pools)
  // with 31-bit offsets
  const size_t lim = (size_t)1 << 31;
  if (a.pg.table) {
    const size_t rows = (size_t)a.pg.num_pages * a.Hkv * a.pg.page_tokens;
    if (rows * a.kcode_row >= lim || rows / kSet * a.vset_bytes >= lim || rows * 2 * a.kpar_n >= lim ||
        rows * 2 * a.vpar_n >= lim)
      return false;
  }
  return a.d == 128 && a.bits_k >= 2 && a.bits_k <= 4 && a.bits_v >= 2 && a.bits_v <= 4 && (a.G == 4 || a.G == 8) &&
         a.kcode_bytes < lim && a.vcode_bytes < lim && a.kpar_bytes < lim && a.vpar_bytes < lim;
}

// The decode-step form (the new token's append fused into the decode) exists for 2-bit
// keys and 2- or 3-bit values; the wider codes' decode runs after a separate append.
bool decode_fast_appends(const DecodeArgs &a) {
  return decode_fast_supported(a) && a.bits_k == 2 && a.bits_v <= 3 && !a.pg.table;
}

// Launch shape: one kWholeWaves-wave workgroup per KV head when the split count equals
// it and there are at least as many KV heads as compute units (G = 4 with 2-bit keys and
// 2- or 3-bit values, whose LDS fits), else ceil(P / kSplitWaves) workgroups of
// kSplitWaves waves per KV head.
static int cu_count() {
  static int c = -1;
  if (c < 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      hipGetLastError();
      return 1 << 30;
    }
    c = prop.multiProcessorCount;
  }
  return c;
}

static bool whole_layout(const DecodeArgs &a) {
  return a.G == 4 && a.bits_k == 2 && a.bits_v <= 3 && a.P == kWholeWaves && a.B * a.Hkv >= cu_count();
}

int decode_fast_partials(const DecodeArgs &a) {
  return whole_layout(a) ? 1 : (a.P + kSplitWaves - 1) / kSplitWaves;
}

bool decode_fast_direct(const DecodeArgs &a) { return decode_fast_partials(a) == 1; }

// The split layout's plain kernel of (G, bits_k, bits_v).
static const void *split_kernel(int G, int bits_k, int bits_v) {
#define WUSHKV_K(G_, BK_, BV_) (const void *)decode_fast_kernel<G_, BK_, BV_, kSplitWaves, false, false>
#define WUSHKV_KV(G_, BK_) (bits_v == 2 ? WUSHKV_K(G_, BK_, 2) : bits_v == 3 ? WUSHKV_K(G_, BK_, 3) : WUSHKV_K(G_, BK_, 4))
  if (G == 4) return bits_k == 2 ? WUSHKV_KV(4, 2) : bits_k == 3 ? WUSHKV_KV(4, 3) : WUSHKV_KV(4, 4);
  return bits_k == 2 ? WUSHKV_KV(8, 2) : bits_k == 3 ? WUSHKV_KV(8, 3) : WUSHKV_KV(8, 4);
#undef WUSHKV_KV
#undef WUSHKV_K
}

// Waves of the MFMA decode the GPU holds at once for (G, bits_k, bits_v) in the split
// layout; 0 if unknown.
int decode_fast_resident_waves(int G, int bits_k, int bits_v) {
  static int cache[2][3][3] = {{{-1, -1, -1}, {-1, -1, -1}, {-1, -1, -1}}, {{-1, -1, -1}, {-1, -1, -1}, {-1, -1, -1}}};
  int &c = cache[G == 8][bits_k - 2][bits_v - 2];
  if (c >= 0) return c;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, split_kernel(G, bits_k, bits_v), 64 * kSplitWaves, 0) !=
      hipSuccess) {
    hipGetLastError();
    return 0;
  }
  c = blocks * kSplitWaves * cu_count();
  return c;
}

// KV partitions the split layout runs for a request of a.P: more partitions than the
// GPU holds resident decode waves per KV head would run as several rounds of
// workgroups, each round paying the query setup and the ring's fill again and the last
// its tail (long context, 8 x 8 KV heads: 128 partitions 214 us, 32 partitions 167 us).
// Then each wave takes ceil(P / P_run) consecutive logical partitions' tokens instead:
// the same attention, in coarser split-K partials.
int decode_fast_run_splits(const DecodeArgs &a) {
  if (whole_layout(a)) return a.P;
  const int r = decode_fast_resident_waves(a.G, a.bits_k, a.bits_v);
  const int64_t heads = (int64_t)a.B * a.Hkv;
  if (r <= 0 || heads <= 0) return a.P;
  int per_head = (int)(r / heads) / kSplitWaves * kSplitWaves;
  if (per_head < kSplitWaves) per_head = kSplitWaves;
  return a.P > per_head ? per_head : a.P;
}

hipError_t launch_decode_fast(const DecodeArgs &a, hipStream_t s) {
  const int nwg = decode_fast_partials(a);
  dim3 grid(nwg, a.B * a.Hkv);
  const bool pg = a.pg.table != nullptr;
  // (the fused append serves the unpaged one-token step of 2-bit keys and 2- or 3-bit
  // values only: decode_fast_appends)
#define WUSHKV_FAST(G, BK, BV, NW)                                                                                     \
  if (a.append_new) hipLaunchKernelGGL((decode_fast_kernel<G, BK, BV, NW, false, true>), grid, dim3(64 * NW), 0, s, a, \
                                       nwg);                                                                           \
  else if (pg) hipLaunchKernelGGL((decode_fast_kernel<G, BK, BV, NW, true, false>), grid, dim3(64 * NW), 0, s, a, nwg); \
  else hipLaunchKernelGGL((decode_fast_kernel<G, BK, BV, NW, false, false>), grid, dim3(64 * NW), 0, s, a, nwg)
#define WUSHKV_FAST_NA(G, BK, BV)                                                                                      \
  if (pg) hipLaunchKernelGGL((decode_fast_kernel<G, BK, BV, kSplitWaves, true, false>), grid, dim3(64 * kSplitWaves), 0, \
                             s, a, nwg);                                                                              \
  else hipLaunchKernelGGL((decode_fast_kernel<G, BK, BV, kSplitWaves, false, false>), grid, dim3(64 * kSplitWaves), 0, s, \
                          a, nwg)
  if (a.append_new && !decode_fast_appends(a)) return hipErrorInvalidValue;
  if (whole_layout(a)) {
    if (a.bits_v == 2) { WUSHKV_FAST(4, 2, 2, kWholeWaves); }
    else { WUSHKV_FAST(4, 2, 3, kWholeWaves); }
  } else if (a.bits_k == 2 && a.bits_v <= 3) {
    if (a.G == 4 && a.bits_v == 2) { WUSHKV_FAST(4, 2, 2, kSplitWaves); }
    else if (a.G == 4) { WUSHKV_FAST(4, 2, 3, kSplitWaves); }
    else if (a.bits_v == 2) { WUSHKV_FAST(8, 2, 2, kSplitWaves); }
    else { WUSHKV_FAST(8, 2, 3, kSplitWaves); }
  } else {
#define WUSHKV_FAST_BV(G, BK)                    \
  if (a.bits_v == 2) { WUSHKV_FAST_NA(G, BK, 2); } \
  else if (a.bits_v == 3) { WUSHKV_FAST_NA(G, BK, 3); } \
  else { WUSHKV_FAST_NA(G, BK, 4); }
    if (a.G == 4) {
      if (a.bits_k == 2) { WUSHKV_FAST_NA(4, 2, 4); }
      else if (a.bits_k == 3) { WUSHKV_FAST_BV(4, 3) }
      else { WUSHKV_FAST_BV(4, 4) }
    } else {
      if (a.bits_k == 2) { WUSHKV_FAST_NA(8, 2, 4); }
      else if (a.bits_k == 3) { WUSHKV_FAST_BV(8, 3) }
      else { WUSHKV_FAST_BV(8, 4) }
    }
#undef WUSHKV_FAST_BV
  }
#undef WUSHKV_FAST_NA
#undef WUSHKV_FAST
  return hipGetLastError();
}

}  // namespace wushkv
