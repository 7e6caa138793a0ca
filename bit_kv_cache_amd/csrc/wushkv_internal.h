// Internal definitions shared by the host ABI layer and the HIP kernels of
// libwushkv.  Nothing here is part of the public ABI (include/wushkv.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/wushkv.h"

namespace wushkv {

constexpr int kSet = 64;           // tokens per V-code set
constexpr int kMaxOrderStats = 8;  // order statistics kept per end for percentiles

// Geometry derived from a cache descriptor (host side, validated).
struct Geom {
  int B, Hkv, d, S, R, C;
  int64_t cap, body_cap;
  int bits_k, bits_v, quant_k, quant_v;
  float clip;
  // percentile interpolation: value = xs[i] + t * (xs[i+1] - xs[i]) with xs sorted ascending;
  // lo uses (lo_i, lo_t) counted from the bottom, hi uses (hi_i, hi_t) counted from the bottom.
  int lo_i, hi_i;
  float lo_t, hi_t;
  double lo_t64, hi_t64; // the same weights in fp64 (exact re-decisions)
  int need_lo, need_hi;  // smallest / largest order statistics a row needs
  // per-(b, g) sizes in bytes
  size_t sink_bytes, ring_bytes, kcode_row, kcode_bytes, vset_bytes, vcode_bytes, kpar_bytes, vpar_bytes;
  int kpar_n, vpar_n;    // fp16 parameters per token (1 QuEST, 2 affine)
};

int make_geom(const wushkv_cache *c, Geom *g);

__host__ __device__ inline int64_t n_quantized(int64_t n, int S, int R, int C) {
  int64_t e = n - S - R;
  return e > 0 ? (int64_t)C * (e / C) : 0;
}

// Ragged batches: per-sequence token counts travel in the argument blocks (by value,
// so a call allocates and copies nothing), for at most this many sequences.  Or they
// live in device memory (int32 per sequence), read by the kernels themselves, so that
// a captured call sequence does not bake them in.
constexpr int kMaxRagged = 256;
enum { kUniform = 0, kRaggedHost = 1, kRaggedDevice = 2 };

// Paged body: the code and parameter planes are pools [num_pages][Hkv][page_tokens
// rows], and table[b][lp] names the physical page of sequence b's logical page lp (body
// rows lp * page_tokens ..).  page_tokens is a multiple of 64, so a 64-token value set
// never spans two pages.  table == nullptr: contiguous planes [B][Hkv][body_cap rows].
struct PageTable {
  const int32_t *table;
  int64_t page_tokens;
  int max_pages, num_pages;
};

// Plain-old-data argument blocks handed to kernels by value.
struct FlushArgs {
  int B, Hkv, d, S, R, C;
  int64_t n_before, n_new;
  int64_t u0, u1;                 // body rows [u0, u1) flushed by this call (uniform batch)
  int ragged;                     // kRaggedHost: sequence b holds seq_nb[b] tokens before the
  int32_t seq_nb[kMaxRagged];     // call; kRaggedDevice: dev_n[b] (device memory)
  const int32_t *dev_n;
  int64_t cap;                    // capacity (device counts are checked against it)
  int in_dtype;
  const void *k_new, *v_new;      // [B][Hkv][n_new][d]
  const _Float16 *tk;             // [Hkv][d][d]
  const _Float16 *ring_k, *ring_v;
  uint8_t *codes_k, *codes_v;
  _Float16 *par_k, *par_v;
  size_t ring_bytes, kcode_row, kcode_bytes, vset_bytes, vcode_bytes, kpar_bytes, vpar_bytes;
  int bits_k, bits_v, quant_k, quant_v, kpar_n, vpar_n;
  float clip;
  int lo_i, hi_i, need_lo, need_hi;
  float lo_t, hi_t;
  double lo_t64, hi_t64;
  PageTable pg;
  int64_t body_cap;
  float had;                      // nonzero: T_K = had * H (Sylvester-Hadamard), tk unused
  // Fused window append (uniform counts, every flushed row from the input, so no ring
  // slot the flush reads is written): the last append_x workgroups of the grid's x
  // dimension write the call's sink and ring rows, as append_kernel would; 0: none.
  int append_x;
  _Float16 *sink_k, *sink_v;
  size_t sink_bytes;
};

struct AppendArgs {
  int B, Hkv, d, S, R, C;
  int64_t n_before, n_new, q_after;
  int ragged;                     // as FlushArgs
  int32_t seq_nb[kMaxRagged];
  const int32_t *dev_n;
  int64_t cap;
  int in_dtype;
  const void *k_new, *v_new;
  _Float16 *sink_k, *sink_v, *ring_k, *ring_v;
  size_t sink_bytes, ring_bytes;
};

struct QtArgs {
  const float *tinvt;
  const void *q;
  float *qt;
  int q_dtype, B, Hq, Hkv, d;
};

struct DecodeArgs {
  int B, Hkv, Hq, G, d, S, R, C;
  int64_t n, nq;                  // tokens attended, body tokens Q(n) (the largest, if ragged)
  int ragged;                     // kRaggedHost: sequence b attends seq_n[b] tokens;
  int32_t seq_n[kMaxRagged];      // kRaggedDevice: dev_n[b] + dev_add (device memory), at most max_n
  const int32_t *dev_n;
  int64_t max_n;
  int dev_add;
  int P;                          // body partitions
  const void *q;
  int q_dtype;
  const float *qt;
  const float *tinvt;             // non-null: the decode forms q~ = T^{-T} q itself and
  float *qt_out;                  // writes it here (else q~ is read from qt)
  const _Float16 *sink_k, *sink_v, *ring_k, *ring_v;
  const uint8_t *codes_k, *codes_v;
  const _Float16 *par_k, *par_v;
  size_t sink_bytes, ring_bytes, kcode_row, kcode_bytes, vset_bytes, vcode_bytes, kpar_bytes, vpar_bytes;
  int bits_k, bits_v, quant_k, quant_v, kpar_n, vpar_n;
  float *part_o, *part_ml;        // workspace: [B][Hq][P+1][d], [B][Hq][P+1][2]
  float *out;                     // [B][Hq][d]
  int force_generic;              // the generic kernel for every shape (wushkv_decode_attention_generic)
  PageTable pg;
  int64_t body_cap;
  // One new token per sequence, appended by the decode itself (MFMA path): token n - 1
  // of each sequence comes from k_new / v_new [B][Hkv][1][d] in in_dtype.
  int append_new, in_dtype;
  const void *k_new, *v_new;
};

// Calibration sums S_g = sum x x^T over the rows of heads h with h / group == g.
struct CalibArgs {
  const void *x;                  // [B][H][T][128] bf16 or f16
  int dtype, B, H, group;
  int64_t T;
  int bpw;                        // batch rows per workgroup
  int nparts;                     // partials per group (set by launch_calib)
  float *partials;                // workspace: [H / group][nparts][10 tiles][32][32]
  float *out;                     // [H / group][128][128]
};

// wushkv_decode_attention with every check and, unless validate_only, the launch.
int decode_attention_checked(const wushkv_cache *c, int64_t n_tokens, const void *q, int32_t q_dtype, const float *q_t,
                             int32_t num_q_heads, int32_t num_splits, void *workspace, size_t workspace_bytes,
                             float *out, void *stream, bool validate_only);

hipError_t launch_append(const AppendArgs &a, hipStream_t s);
// Workgroups of the window append of a uniform call (FlushArgs::append_x).
int append_workgroups(int64_t n_before, int64_t n_new, int64_t q_after, int S, int d);
hipError_t launch_advance(int32_t *dev_n, int B, int n_new, int64_t cap, hipStream_t s);
hipError_t launch_calib(const CalibArgs &a, hipStream_t s);
int calib_batch_per_wg(int B, int groups);
size_t calib_partial_floats(int B, int H, int group);
hipError_t launch_flush(const FlushArgs &a, hipStream_t s);
hipError_t launch_qtransform(const QtArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_fast(const DecodeArgs &a, hipStream_t s);
bool decode_fast_supported(const DecodeArgs &a);
int decode_fast_partials(const DecodeArgs &a);
bool decode_fast_direct(const DecodeArgs &a);   // the fast kernel writes out itself
int decode_fast_resident_waves(int G, int bits_k, int bits_v);
bool decode_fast_appends(const DecodeArgs &a);   // the decode-step form with the append fused
int decode_fast_run_splits(const DecodeArgs &a);   // partitions the MFMA kernel runs for a.P

// Device helpers ------------------------------------------------------------

// Byte offset of body row u of (batch row b, KV head g) in a plane whose rows are `row`
// bytes (value codes: a set's bytes / 64).  Contiguous planes: ((b Hkv + g) body_cap + u)
// row.  Paged: ((page Hkv + g) page_tokens + u mod page_tokens) row, or -1 when the
// logical page is past the table or its entry outside [0, num_pages).
template <bool PAGED = true>
__device__ __forceinline__ int64_t body_offset(const PageTable &pg, int Hkv, int64_t body_cap, int b, int g,
                                               int64_t u, int64_t row) {
  if (!PAGED || !pg.table) return (((int64_t)b * Hkv + g) * body_cap + u) * row;
  const int64_t lp = u / pg.page_tokens;
  const int page = lp < pg.max_pages ? pg.table[(int64_t)b * pg.max_pages + lp] : -1;
  if (page < 0 || page >= pg.num_pages) return -1;
  return (((int64_t)page * Hkv + g) * pg.page_tokens + (u - lp * pg.page_tokens)) * row;
}

// The same for reads: an invalid page reads page 0 (never outside the pool).
__device__ __forceinline__ int64_t body_read_offset(const PageTable &pg, int Hkv, int64_t body_cap, int b, int g,
                                                    int64_t u, int64_t row) {
  const int64_t off = body_offset(pg, Hkv, body_cap, b, g, u, row);
  return off >= 0 ? off : ((int64_t)g * pg.page_tokens + u % pg.page_tokens) * row;
}

// Tokens attended by sequence b and its body tokens Q(n).
struct SeqLen {
  int64_t n, nq;
};
// A device count outside [1, max_n] attends nothing, which makes the sequence's output
// rows NaN (an empty softmax) without touching its cache.
__device__ __forceinline__ SeqLen seq_len(const DecodeArgs &a, int b) {
  if (a.ragged == kUniform) return SeqLen{a.n, a.nq};
  int64_t n;
  if (a.ragged == kRaggedDevice) {
    n = (int64_t)a.dev_n[b] + a.dev_add;
    if (n < 1 || n > a.max_n) n = 0;
  } else {
    n = a.seq_n[b];
  }
  return SeqLen{n, n_quantized(n, a.S, a.R, a.C)};
}

// Tokens sequence b holds before an append / flush call; -1 for a device count outside
// [0, capacity - n_new] (the call then leaves that sequence alone).
template <class Args>
__device__ __forceinline__ int64_t seq_before(const Args &a, int b) {
  if (a.ragged == kRaggedDevice) {
    const int64_t n = a.dev_n[b];
    return n >= 0 && n + a.n_new <= a.cap ? n : -1;
  }
  return a.ragged == kRaggedHost ? a.seq_nb[b] : a.n_before;
}

__device__ __forceinline__ float load_in(const void *p, int dtype, size_t i) {
  if (dtype == WUSHKV_DT_F32) return ((const float *)p)[i];
  if (dtype == WUSHKV_DT_BF16) {
    unsigned short b = ((const unsigned short *)p)[i];
    return __uint_as_float(((unsigned)b) << 16);
  }
  return (float)((const _Float16 *)p)[i];
}

}  // namespace wushkv
