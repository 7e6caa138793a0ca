// Host side of libwushkv: argument validation, plane geometry and dispatch of the
// gfx950 kernels.  Every check runs before anything is enqueued.
#include <math.h>
#include <string.h>

#include "wushkv_internal.h"

using namespace wushkv;

namespace {

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

int check_dtype(int dt) { return (dt == WUSHKV_DT_F32 || dt == WUSHKV_DT_BF16 || dt == WUSHKV_DT_F16); }


// Order statistics needed for the linear-interpolation percentile at pct: the lower
// index i and the weight t of the next one (fp32 and fp64).
void pct_index(int d, double pct, int *i, float *t, double *t64) {
  double h = (d - 1) * (pct / 100.0);
  int fi = (int)floor(h);
  if (fi >= d - 1) { *i = d - 1; *t = 0.0f; *t64 = 0.0; return; }
  *i = fi;
  *t64 = h - fi;
  *t = (float)*t64;
}

}  // namespace

namespace wushkv {

int make_geom(const wushkv_cache *c, Geom *g) {
  if (!c) return WUSHKV_ERR_NULL;
  if (c->batch < 1 || c->num_kv_heads < 1) return WUSHKV_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return WUSHKV_ERR_SHAPE;
  if (c->sink < 0 || c->recent < 0 || c->chunk < 1 || c->recent % c->chunk != 0) return WUSHKV_ERR_SHAPE;
  if (c->capacity < 1 || c->capacity > ((int64_t)1 << 40)) return WUSHKV_ERR_SHAPE;
  for (int b : {c->bits_k, c->bits_v})
    if (b < 2 || b > 4) return WUSHKV_ERR_SHAPE;
  for (int q : {c->quant_k, c->quant_v})
    if (q != WUSHKV_Q_QUEST && q != WUSHKV_Q_AFFINE_PCT) return WUSHKV_ERR_SHAPE;
  bool any_quest = c->quant_k == WUSHKV_Q_QUEST || c->quant_v == WUSHKV_Q_QUEST;
  bool any_aff = c->quant_k == WUSHKV_Q_AFFINE_PCT || c->quant_v == WUSHKV_Q_AFFINE_PCT;
  if (any_quest && !(c->clip_mult > 0.0f && isfinite(c->clip_mult))) return WUSHKV_ERR_SHAPE;
  if (any_aff && !(c->pct_lo >= 0.0f && c->pct_hi <= 100.0f && c->pct_lo < c->pct_hi)) return WUSHKV_ERR_SHAPE;
  if (c->batch > 65535 || c->num_kv_heads > 4096) return WUSHKV_ERR_SHAPE;

  Geom &G = *g;
  G.B = c->batch; G.Hkv = c->num_kv_heads; G.d = c->head_dim;
  G.S = c->sink; G.R = c->recent; G.C = c->chunk;
  G.cap = c->capacity;
  int64_t body = c->capacity - c->sink;
  if (body < 0) body = 0;
  G.body_cap = (body + kSet - 1) / kSet * kSet;
  G.bits_k = c->bits_k; G.bits_v = c->bits_v;
  G.quant_k = c->quant_k; G.quant_v = c->quant_v;
  G.clip = c->clip_mult;
  G.lo_i = G.hi_i = 0; G.lo_t = G.hi_t = 0.0f; G.lo_t64 = G.hi_t64 = 0.0; G.need_lo = G.need_hi = 0;
  if (any_aff) {
    pct_index(G.d, c->pct_lo, &G.lo_i, &G.lo_t, &G.lo_t64);
    pct_index(G.d, c->pct_hi, &G.hi_i, &G.hi_t, &G.hi_t64);
    G.need_lo = (G.lo_i + 2 < G.d) ? G.lo_i + 2 : G.d;
    G.need_hi = G.d - G.hi_i;
    if (G.need_lo > kMaxOrderStats || G.need_hi > kMaxOrderStats) return WUSHKV_ERR_UNSUPPORTED;
  }
  G.sink_bytes = (size_t)G.S * G.d * 2;
  G.ring_bytes = (size_t)(G.R + G.C) * G.d * 2;
  G.kcode_row = (size_t)G.d * G.bits_k / 8;
  G.kcode_bytes = (size_t)G.body_cap * G.kcode_row;
  G.vset_bytes = (size_t)kSet * G.d * G.bits_v / 8;
  G.vcode_bytes = (size_t)(G.body_cap / kSet) * G.vset_bytes;
  G.kpar_n = c->quant_k == WUSHKV_Q_QUEST ? 1 : 2;
  G.vpar_n = c->quant_v == WUSHKV_Q_QUEST ? 1 : 2;
  G.kpar_bytes = (size_t)G.body_cap * G.kpar_n * 2;
  G.vpar_bytes = (size_t)G.body_cap * G.vpar_n * 2;
  return WUSHKV_OK;
}

}  // namespace wushkv

namespace {

int check_planes(const wushkv_cache *c) {
  const void *ps[] = {c->sink_k, c->sink_v, c->ring_k, c->ring_v, c->codes_k, c->codes_v, c->par_k, c->par_v};
  for (const void *p : ps)
    if (!p) return WUSHKV_ERR_NULL;
  for (const void *p : ps)
    if (misaligned(p)) return WUSHKV_ERR_ALIGN;
  return WUSHKV_OK;
}

// A page table's host-side checks; fills pg (table == nullptr when pages is null).
int check_pages(const wushkv_pages *pages, const Geom &g, PageTable *pg) {
  pg->table = nullptr;
  pg->page_tokens = 0;
  pg->max_pages = pg->num_pages = 0;
  if (!pages) return WUSHKV_OK;
  if (!pages->table) return WUSHKV_ERR_NULL;
  if (((uintptr_t)pages->table & 3u) != 0) return WUSHKV_ERR_ALIGN;
  if (pages->page_tokens < kSet || pages->page_tokens % kSet != 0 || pages->max_pages < 1 || pages->num_pages < 1)
    return WUSHKV_ERR_SHAPE;
  // every body row a sequence can hold has a logical page
  if ((int64_t)pages->max_pages * pages->page_tokens < g.body_cap) return WUSHKV_ERR_CAPACITY;
  pg->table = pages->table;
  pg->page_tokens = pages->page_tokens;
  pg->max_pages = pages->max_pages;
  pg->num_pages = pages->num_pages;
  return WUSHKV_OK;
}

int hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? WUSHKV_OK : WUSHKV_ERR_HIP;
}

// KV partitions of a decode: the caller's count, or (library's choice) as many
// partitions as the GPU holds resident decode waves, rounded up to whole 4-wave
// workgroups, but never more than there are 64-token body sets.
int32_t choose_splits(const Geom &g, int64_t nq, int32_t requested, int G) {
  if (requested > 0) return requested;
  const int64_t nsets = (nq + kSet - 1) / kSet;
  int64_t waves = 2048;
  if (g.d == 128 && g.bits_k >= 2 && g.bits_k <= 4 && g.bits_v >= 2 && g.bits_v <= 4 && (G == 4 || G == 8)) {
    const int r = decode_fast_resident_waves(G, g.bits_k, g.bits_v);
    if (r > 0) waves = r;
  }
  const int64_t heads = (int64_t)g.B * g.Hkv;
  int64_t want = (waves + heads - 1) / heads;
  want = (want + 3) / 4 * 4;
  // at least two 64-token sets per partition: below that a partition's fixed work (its
  // q~ setup and window stages) outweighs the parallelism (1 x 8 KV heads, 8192 tokens:
  // 136 partitions 16.7 us, 64 partitions 15.3 us)
  if (want > (nsets + 1) / 2) want = (nsets + 1) / 2;
  if (want < 1) want = 1;
  if (want > 4096) want = 4096;
  return (int32_t)want;
}

}  // namespace

extern "C" {

const char *wushkv_status_string(int s) {
  switch (s) {
    case WUSHKV_OK: return "ok";
    case WUSHKV_ERR_NULL: return "null pointer";
    case WUSHKV_ERR_SHAPE: return "invalid shape or option";
    case WUSHKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case WUSHKV_ERR_CAPACITY: return "token count exceeds cache capacity";
    case WUSHKV_ERR_WORKSPACE: return "decode workspace missing or too small";
    case WUSHKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case WUSHKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int wushkv_abi_version(void) { return WUSHKV_ABI_VERSION; }

int wushkv_cache_check(const wushkv_cache *c) {
  Geom g;
  return make_geom(c, &g);
}

size_t wushkv_plane_bytes(const wushkv_cache *c, int plane) {
  Geom g;
  if (make_geom(c, &g) != WUSHKV_OK) return 0;
  size_t heads = (size_t)g.B * g.Hkv;
  switch (plane) {
    case WUSHKV_PLANE_SINK_K: case WUSHKV_PLANE_SINK_V: return heads * g.sink_bytes;
    case WUSHKV_PLANE_RING_K: case WUSHKV_PLANE_RING_V: return heads * g.ring_bytes;
    case WUSHKV_PLANE_CODES_K: return heads * g.kcode_bytes;
    case WUSHKV_PLANE_CODES_V: return heads * g.vcode_bytes;
    case WUSHKV_PLANE_PAR_K: return heads * g.kpar_bytes;
    case WUSHKV_PLANE_PAR_V: return heads * g.vpar_bytes;
    default: return 0;
  }
}

size_t wushkv_pool_bytes(const wushkv_cache *c, const wushkv_pages *pages, int plane) {
  Geom g;
  PageTable pg;
  if (make_geom(c, &g) != WUSHKV_OK || !pages || check_pages(pages, g, &pg) != WUSHKV_OK) return 0;
  const size_t rows = (size_t)pg.num_pages * g.Hkv * pg.page_tokens;
  switch (plane) {
    case WUSHKV_PLANE_CODES_K: return rows * g.kcode_row;
    case WUSHKV_PLANE_CODES_V: return rows / kSet * g.vset_bytes;
    case WUSHKV_PLANE_PAR_K: return rows * 2 * g.kpar_n;
    case WUSHKV_PLANE_PAR_V: return rows * 2 * g.vpar_n;
    default: return wushkv_plane_bytes(c, plane);
  }
}

int32_t wushkv_decode_num_splits(const wushkv_cache *c, int64_t n_tokens, int32_t num_q_heads, int32_t num_splits) {
  Geom g;
  if (make_geom(c, &g) != WUSHKV_OK) return 0;
  if (n_tokens < 1 || n_tokens > g.cap || num_q_heads < 1 || num_q_heads % g.Hkv || num_splits < 0) return 0;
  return choose_splits(g, n_quantized(n_tokens, g.S, g.R, g.C), num_splits, num_q_heads / g.Hkv);
}

size_t wushkv_decode_workspace_bytes(const wushkv_cache *c, int64_t n_tokens, int32_t num_q_heads, int32_t num_splits) {
  Geom g;
  int32_t P = wushkv_decode_num_splits(c, n_tokens, num_q_heads, num_splits);
  if (P <= 0 || make_geom(c, &g) != WUSHKV_OK) return 0;
  size_t rows = (size_t)g.B * num_q_heads * (P + 1);
  size_t bytes = rows * g.d * 4 + rows * 2 * 4;
  return (bytes + 255) / 256 * 256;
}

}  // extern "C"

namespace {

// Append + flush for a uniform batch (seq_nb == dev_n == nullptr: every sequence holds
// n_before tokens), a ragged one (sequence b holds seq_nb[b]) or one whose counts live
// in device memory (dev_n[b]; the call then advances them by n_new).
// With `deferred`, the append itself is not launched: its arguments are returned for
// the caller to launch or to fold into the decode (the flush, when due, is launched).
int append_flush_impl(const wushkv_cache *c, const wushkv_pages *pages, int64_t n_before, const int64_t *seq_nb,
                      int32_t *dev_n, int32_t n_new, const void *k_new, const void *v_new, int32_t in_dtype,
                      const void *t_k_f16, void *stream, AppendArgs *deferred = nullptr, int64_t dev_cap = -1,
                      float had = 0.f) {
  Geom g;
  int st = make_geom(c, &g);
  if (st != WUSHKV_OK) return st;
  PageTable pg;
  if ((st = check_pages(pages, g, &pg)) != WUSHKV_OK) return st;
  if (dev_n) {
    if (((uintptr_t)dev_n & 3u) != 0) return WUSHKV_ERR_ALIGN;
    n_before = 0;   // the counts are checked by the kernels
  } else if (seq_nb) {
    if (g.B > kMaxRagged) return WUSHKV_ERR_UNSUPPORTED;
    n_before = 0;
    for (int b = 0; b < g.B; ++b) {
      if (seq_nb[b] < 0) return WUSHKV_ERR_SHAPE;
      if (seq_nb[b] > n_before) n_before = seq_nb[b];   // the longest, for the checks below
    }
  }
  if (n_before < 0 || n_new < 0 || !check_dtype(in_dtype)) return WUSHKV_ERR_SHAPE;
  if (n_before + n_new > g.cap) return WUSHKV_ERR_CAPACITY;
  if ((st = check_planes(c)) != WUSHKV_OK) return st;
  if (n_new == 0) return WUSHKV_OK;
  if (!k_new || !v_new || (!t_k_f16 && had == 0.f)) return WUSHKV_ERR_NULL;
  if (misaligned(k_new) || misaligned(v_new) || (had == 0.f && misaligned(t_k_f16))) return WUSHKV_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  int64_t n_after = n_before + n_new;
  int64_t qb = n_quantized(n_before, g.S, g.R, g.C), qa = n_quantized(n_after, g.S, g.R, g.C);
  bool flush = qa > qb;
  if (dev_n) {
    flush = true;   // whether one is due is decided per sequence on the device
  } else if (seq_nb) {
    flush = false;
    for (int b = 0; b < g.B; ++b)
      flush |= n_quantized(seq_nb[b] + n_new, g.S, g.R, g.C) > n_quantized(seq_nb[b], g.S, g.R, g.C);
  }
  (void)hipGetLastError();   // clear an earlier sticky error before launching
  // A uniform call whose flushed rows all come from the input (every prefill) writes its
  // window rows from extra workgroups of the flush launch: the flush then reads no ring
  // slot, so the two may run together, and the call is one launch.
  const bool fuse_append = flush && !dev_n && !seq_nb && !deferred && g.S + qb >= n_before;
  if (flush) {
    // The flush reads ring rows written by earlier calls, so it runs before this
    // call's ring writes (same stream, in order).
    FlushArgs f;
    memset(&f, 0, sizeof f);
    f.B = g.B; f.Hkv = g.Hkv; f.d = g.d; f.S = g.S; f.R = g.R; f.C = g.C;
    f.n_before = n_before; f.n_new = n_new; f.u0 = qb; f.u1 = qa; f.in_dtype = in_dtype;
    f.k_new = k_new; f.v_new = v_new; f.tk = (const _Float16 *)t_k_f16;
    f.ring_k = (const _Float16 *)c->ring_k; f.ring_v = (const _Float16 *)c->ring_v;
    f.codes_k = (uint8_t *)c->codes_k; f.codes_v = (uint8_t *)c->codes_v;
    f.par_k = (_Float16 *)c->par_k; f.par_v = (_Float16 *)c->par_v;
    f.ring_bytes = g.ring_bytes; f.kcode_row = g.kcode_row; f.kcode_bytes = g.kcode_bytes;
    f.vset_bytes = g.vset_bytes; f.vcode_bytes = g.vcode_bytes; f.kpar_bytes = g.kpar_bytes; f.vpar_bytes = g.vpar_bytes;
    f.bits_k = g.bits_k; f.bits_v = g.bits_v; f.quant_k = g.quant_k; f.quant_v = g.quant_v;
    f.kpar_n = g.kpar_n; f.vpar_n = g.vpar_n; f.clip = g.clip;
    f.lo_i = g.lo_i; f.hi_i = g.hi_i; f.lo_t = g.lo_t; f.hi_t = g.hi_t; f.need_lo = g.need_lo; f.need_hi = g.need_hi;
    f.lo_t64 = g.lo_t64; f.hi_t64 = g.hi_t64;
    f.cap = dev_cap >= 0 && dev_cap < g.cap ? dev_cap : g.cap;
    f.pg = pg;
    f.body_cap = g.body_cap;
    f.had = had;
    if (fuse_append) {
      f.append_x = append_workgroups(n_before, n_new, qa, g.S, g.d);
      f.sink_k = (_Float16 *)c->sink_k; f.sink_v = (_Float16 *)c->sink_v;
      f.sink_bytes = g.sink_bytes;
    }
    if (dev_n) {
      f.ragged = kRaggedDevice;
      f.dev_n = dev_n;
    } else if (seq_nb) {
      f.ragged = kRaggedHost;
      for (int b = 0; b < g.B; ++b) f.seq_nb[b] = (int32_t)seq_nb[b];
    }
    if (launch_flush(f, s) != hipSuccess) return WUSHKV_ERR_HIP;
    if (fuse_append) return hip_status();
  }
  AppendArgs a;
  memset(&a, 0, sizeof a);
  a.B = g.B; a.Hkv = g.Hkv; a.d = g.d; a.S = g.S; a.R = g.R; a.C = g.C;
  a.n_before = n_before; a.n_new = n_new; a.q_after = qa; a.in_dtype = in_dtype;
  a.k_new = k_new; a.v_new = v_new;
  a.sink_k = (_Float16 *)c->sink_k; a.sink_v = (_Float16 *)c->sink_v;
  a.ring_k = (_Float16 *)c->ring_k; a.ring_v = (_Float16 *)c->ring_v;
  a.sink_bytes = g.sink_bytes; a.ring_bytes = g.ring_bytes;
  a.cap = dev_cap >= 0 && dev_cap < g.cap ? dev_cap : g.cap;
  if (dev_n) {
    a.ragged = kRaggedDevice;
    a.dev_n = dev_n;
  } else if (seq_nb) {
    a.ragged = kRaggedHost;
    for (int b = 0; b < g.B; ++b) a.seq_nb[b] = (int32_t)seq_nb[b];
  }
  if (deferred) {
    *deferred = a;
    return hip_status();
  }
  if (launch_append(a, s) != hipSuccess) return WUSHKV_ERR_HIP;
  if (dev_n && launch_advance(dev_n, g.B, n_new, g.cap, s) != hipSuccess) return WUSHKV_ERR_HIP;
  return hip_status();
}

}  // namespace

extern "C" {

int wushkv_append_flush(const wushkv_cache *c, int64_t n_before, int32_t n_new, const void *k_new,
                        const void *v_new, int32_t in_dtype, const void *t_k_f16, void *stream) {
  return append_flush_impl(c, nullptr, n_before, nullptr, nullptr, n_new, k_new, v_new, in_dtype, t_k_f16, stream);
}

int wushkv_append_flush_hadamard(const wushkv_cache *c, int64_t n_before, int32_t n_new, const void *k_new,
                                 const void *v_new, int32_t in_dtype, float scale, void *stream) {
  // the scale must be a nonzero, finite fp16 value (T_K = scale * H is used as fp16)
  if (!(scale != 0.0f && isfinite(scale)) || (float)(_Float16)scale != scale) return WUSHKV_ERR_SHAPE;
  return append_flush_impl(c, nullptr, n_before, nullptr, nullptr, n_new, k_new, v_new, in_dtype, nullptr, stream,
                           nullptr, -1, scale);
}

int wushkv_append_flush_ragged(const wushkv_cache *c, const int64_t *n_before, int32_t n_new, const void *k_new,
                               const void *v_new, int32_t in_dtype, const void *t_k_f16, void *stream) {
  if (!n_before) return WUSHKV_ERR_NULL;
  return append_flush_impl(c, nullptr, 0, n_before, nullptr, n_new, k_new, v_new, in_dtype, t_k_f16, stream);
}

int wushkv_append_flush_paged(const wushkv_cache *c, const wushkv_pages *pages, const int64_t *n_before,
                              int32_t n_new, const void *k_new, const void *v_new, int32_t in_dtype,
                              const void *t_k_f16, void *stream) {
  if (!n_before || !pages) return WUSHKV_ERR_NULL;
  return append_flush_impl(c, pages, 0, n_before, nullptr, n_new, k_new, v_new, in_dtype, t_k_f16, stream);
}

int wushkv_append_flush_device(const wushkv_cache *c, int32_t *seq_n, int32_t n_new, const void *k_new,
                               const void *v_new, int32_t in_dtype, const void *t_k_f16, void *stream) {
  if (!seq_n) return WUSHKV_ERR_NULL;
  return append_flush_impl(c, nullptr, 0, nullptr, seq_n, n_new, k_new, v_new, in_dtype, t_k_f16, stream);
}

int wushkv_query_transform(const float *t_k_inv_t, const void *q, int32_t q_dtype, int32_t batch,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float *q_t,
                           void *stream) {
  if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads) return WUSHKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return WUSHKV_ERR_SHAPE;
  if (!check_dtype(q_dtype)) return WUSHKV_ERR_SHAPE;
  if (!t_k_inv_t || !q || !q_t) return WUSHKV_ERR_NULL;
  if (misaligned(t_k_inv_t) || misaligned(q) || misaligned(q_t)) return WUSHKV_ERR_ALIGN;
  QtArgs a{t_k_inv_t, q, q_t, q_dtype, batch, num_q_heads, num_kv_heads, head_dim};
  (void)hipGetLastError();   // clear an earlier sticky error before launching
  if (launch_qtransform(a, (hipStream_t)stream) != hipSuccess) return WUSHKV_ERR_HIP;
  return hip_status();
}

size_t wushkv_calib_workspace_bytes(int32_t batch, int32_t num_heads, int64_t tokens, int32_t head_dim,
                                    int32_t group) {
  if (batch < 1 || num_heads < 1 || tokens < 1 || head_dim != 128 || group < 1 || num_heads % group) return 0;
  return calib_partial_floats(batch, num_heads, group) * sizeof(float);
}

int wushkv_calib_stats(const void *x, int32_t dtype, int32_t batch, int32_t num_heads, int64_t tokens,
                       int32_t head_dim, int32_t group, void *workspace, size_t workspace_bytes, float *out,
                       void *stream) {
  if (batch < 1 || num_heads < 1 || tokens < 1 || group < 1 || num_heads % group) return WUSHKV_ERR_SHAPE;
  if (!check_dtype(dtype)) return WUSHKV_ERR_SHAPE;
  if (head_dim != 128 || dtype == WUSHKV_DT_F32) return WUSHKV_ERR_UNSUPPORTED;
  if (!x || !out) return WUSHKV_ERR_NULL;
  if (misaligned(x) || misaligned(out) || misaligned(workspace)) return WUSHKV_ERR_ALIGN;
  const size_t need = wushkv_calib_workspace_bytes(batch, num_heads, tokens, head_dim, group);
  if (!workspace || workspace_bytes < need) return WUSHKV_ERR_WORKSPACE;
  CalibArgs a{};
  a.x = x;
  a.dtype = dtype;
  a.B = batch;
  a.H = num_heads;
  a.group = group;
  a.T = tokens;
  a.bpw = calib_batch_per_wg(batch, num_heads / group);
  a.partials = (float *)workspace;
  a.out = out;
  (void)hipGetLastError();   // clear an earlier sticky error before launching
  if (launch_calib(a, (hipStream_t)stream) != hipSuccess) return WUSHKV_ERR_HIP;
  return hip_status();
}

}  // extern "C"

namespace {

// Decode with q~ given (tinvt == nullptr) or formed from q and T^{-T} into q_t.
// With dev_n, the counts are read on the device and n_tokens bounds them.
// validate_only: the checks alone, nothing launched.  app: the step's one-token append,
// done by the MFMA decode itself or, on the generic path, launched just before it.
int decode_impl(const wushkv_cache *c, const wushkv_pages *pages, int64_t n_tokens, const int64_t *seq_n,
                const int32_t *dev_n, const void *q, int32_t q_dtype, float *q_t, const float *tinvt,
                int32_t num_q_heads, int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                void *stream, const AppendArgs *app = nullptr, bool validate_only = false, int dev_add = 0,
                bool force_generic = false) {
  Geom g;
  int st = make_geom(c, &g);
  if (st != WUSHKV_OK) return st;
  PageTable pg;
  if ((st = check_pages(pages, g, &pg)) != WUSHKV_OK) return st;
  if (dev_n) {
    if (((uintptr_t)dev_n & 3u) != 0) return WUSHKV_ERR_ALIGN;
  } else if (seq_n) {   // ragged: the checks, split count and workspace follow the longest sequence
    if (g.B > kMaxRagged) return WUSHKV_ERR_UNSUPPORTED;
    n_tokens = 0;
    for (int b = 0; b < g.B; ++b) {
      if (seq_n[b] < 1) return WUSHKV_ERR_SHAPE;
      if (seq_n[b] > g.cap) return WUSHKV_ERR_CAPACITY;
      if (seq_n[b] > n_tokens) n_tokens = seq_n[b];
    }
  }
  if (num_q_heads < 1 || num_q_heads % g.Hkv || num_splits < 0 || !check_dtype(q_dtype)) return WUSHKV_ERR_SHAPE;
  int G = num_q_heads / g.Hkv;
  if (G > 16) return WUSHKV_ERR_SHAPE;
  if (n_tokens < 1) return WUSHKV_ERR_SHAPE;
  if (n_tokens > g.cap) return WUSHKV_ERR_CAPACITY;
  if ((st = check_planes(c)) != WUSHKV_OK) return st;
  if (!q || !q_t || !out) return WUSHKV_ERR_NULL;
  if (misaligned(q) || misaligned(q_t) || misaligned(out) || misaligned(tinvt)) return WUSHKV_ERR_ALIGN;
  size_t need = wushkv_decode_workspace_bytes(c, n_tokens, num_q_heads, num_splits);
  if (!workspace || need == 0 || workspace_bytes < need) return WUSHKV_ERR_WORKSPACE;
  if (misaligned(workspace)) return WUSHKV_ERR_ALIGN;
  int32_t P = wushkv_decode_num_splits(c, n_tokens, num_q_heads, num_splits);

  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.B = g.B; a.Hkv = g.Hkv; a.Hq = num_q_heads; a.G = G; a.d = g.d; a.S = g.S; a.R = g.R; a.C = g.C;
  a.n = n_tokens; a.nq = n_quantized(n_tokens, g.S, g.R, g.C); a.P = P;
  if (dev_n) {
    a.ragged = kRaggedDevice;
    a.dev_n = dev_n;
    a.max_n = n_tokens;
    a.dev_add = dev_add;
  } else if (seq_n) {
    a.ragged = kRaggedHost;
    for (int b = 0; b < g.B; ++b) a.seq_n[b] = (int32_t)seq_n[b];
  }
  a.pg = pg;
  a.body_cap = g.body_cap;
  a.q = q; a.q_dtype = q_dtype; a.qt = q_t;
  a.tinvt = tinvt; a.qt_out = tinvt ? q_t : nullptr;
  a.sink_k = (const _Float16 *)c->sink_k; a.sink_v = (const _Float16 *)c->sink_v;
  a.ring_k = (const _Float16 *)c->ring_k; a.ring_v = (const _Float16 *)c->ring_v;
  a.codes_k = (const uint8_t *)c->codes_k; a.codes_v = (const uint8_t *)c->codes_v;
  a.par_k = (const _Float16 *)c->par_k; a.par_v = (const _Float16 *)c->par_v;
  a.sink_bytes = g.sink_bytes; a.ring_bytes = g.ring_bytes; a.kcode_row = g.kcode_row; a.kcode_bytes = g.kcode_bytes;
  a.vset_bytes = g.vset_bytes; a.vcode_bytes = g.vcode_bytes; a.kpar_bytes = g.kpar_bytes; a.vpar_bytes = g.vpar_bytes;
  a.bits_k = g.bits_k; a.bits_v = g.bits_v; a.quant_k = g.quant_k; a.quant_v = g.quant_v;
  a.kpar_n = g.kpar_n; a.vpar_n = g.vpar_n;
  size_t rows = (size_t)g.B * num_q_heads * (P + 1);
  a.part_o = (float *)workspace;
  a.part_ml = a.part_o + rows * g.d;
  a.out = out;
  a.force_generic = force_generic;   // wushkv_decode_attention_generic
  if (validate_only) return WUSHKV_OK;
  (void)hipGetLastError();   // clear an earlier sticky error before launching
  if (app) {
    if (decode_fast_appends(a) && !a.force_generic) {
      a.append_new = 1;
      a.in_dtype = app->in_dtype;
      a.k_new = app->k_new;
      a.v_new = app->v_new;
    } else if (launch_append(*app, (hipStream_t)stream) != hipSuccess) {
      return WUSHKV_ERR_HIP;
    }
  }
  if (launch_decode(a, (hipStream_t)stream) != hipSuccess) return WUSHKV_ERR_HIP;
  return hip_status();
}

}  // namespace

namespace wushkv {

int decode_attention_checked(const wushkv_cache *c, int64_t n_tokens, const void *q, int32_t q_dtype, const float *q_t,
                             int32_t num_q_heads, int32_t num_splits, void *workspace, size_t workspace_bytes,
                             float *out, void *stream, bool validate_only) {
  return decode_impl(c, nullptr, n_tokens, nullptr, nullptr, q, q_dtype, const_cast<float *>(q_t), nullptr, num_q_heads,
                     num_splits, workspace, workspace_bytes, out, stream, nullptr, validate_only);
}

}  // namespace wushkv

extern "C" {

int wushkv_decode_attention(const wushkv_cache *c, int64_t n_tokens, const void *q, int32_t q_dtype,
                            const float *q_t, int32_t num_q_heads, int32_t num_splits, void *workspace,
                            size_t workspace_bytes, float *out, void *stream) {
  return decode_impl(c, nullptr, n_tokens, nullptr, nullptr, q, q_dtype, const_cast<float *>(q_t), nullptr, num_q_heads,
                     num_splits, workspace, workspace_bytes, out, stream);
}

int wushkv_decode_attention_fused(const wushkv_cache *c, int64_t n_tokens, const void *q, int32_t q_dtype,
                                  const float *t_k_inv_t, float *q_t, int32_t num_q_heads, int32_t num_splits,
                                  void *workspace, size_t workspace_bytes, float *out, void *stream) {
  if (!t_k_inv_t) return WUSHKV_ERR_NULL;
  return decode_impl(c, nullptr, n_tokens, nullptr, nullptr, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits, workspace,
                     workspace_bytes, out, stream);
}

int wushkv_decode_attention_ragged(const wushkv_cache *c, const int64_t *n_tokens, const void *q, int32_t q_dtype,
                                   const float *t_k_inv_t, float *q_t, int32_t num_q_heads, int32_t num_splits,
                                   void *workspace, size_t workspace_bytes, float *out, void *stream) {
  if (!n_tokens) return WUSHKV_ERR_NULL;
  return decode_impl(c, nullptr, 0, n_tokens, nullptr, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits, workspace,
                     workspace_bytes, out, stream);
}

int wushkv_decode_attention_generic(const wushkv_cache *c, const int64_t *n_tokens, const void *q, int32_t q_dtype,
                                    const float *t_k_inv_t, float *q_t, int32_t num_q_heads, int32_t num_splits,
                                    void *workspace, size_t workspace_bytes, float *out, void *stream) {
  if (!n_tokens) return WUSHKV_ERR_NULL;
  return decode_impl(c, nullptr, 0, n_tokens, nullptr, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits, workspace,
                     workspace_bytes, out, stream, nullptr, false, 0, true);
}

int wushkv_decode_attention_paged(const wushkv_cache *c, const wushkv_pages *pages, const int64_t *n_tokens,
                                  const void *q, int32_t q_dtype, const float *t_k_inv_t, float *q_t,
                                  int32_t num_q_heads, int32_t num_splits, void *workspace, size_t workspace_bytes,
                                  float *out, void *stream) {
  if (!n_tokens || !pages) return WUSHKV_ERR_NULL;
  return decode_impl(c, pages, 0, n_tokens, nullptr, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits, workspace,
                     workspace_bytes, out, stream);
}

int wushkv_decode_step(const wushkv_cache *c, int64_t n_before, const void *k_new, const void *v_new, int32_t in_dtype,
                       const void *t_k_f16, const void *q, int32_t q_dtype, const float *t_k_inv_t, float *q_t,
                       int32_t num_q_heads, int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                       void *stream) {
  if (!t_k_inv_t || !k_new || !v_new || !t_k_f16) return WUSHKV_ERR_NULL;
  if (n_before < 0) return WUSHKV_ERR_SHAPE;
  // every check first, so that a failing call enqueues nothing
  int st = decode_impl(c, nullptr, n_before + 1, nullptr, nullptr, q, q_dtype, q_t, t_k_inv_t, num_q_heads,
                       num_splits, workspace, workspace_bytes, out, stream, nullptr, true);
  if (st != WUSHKV_OK) return st;
  AppendArgs app;
  st = append_flush_impl(c, nullptr, n_before, nullptr, nullptr, 1, k_new, v_new, in_dtype, t_k_f16, stream, &app);
  if (st != WUSHKV_OK) return st;
  return decode_impl(c, nullptr, n_before + 1, nullptr, nullptr, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits,
                     workspace, workspace_bytes, out, stream, &app);
}

int wushkv_decode_step_device(const wushkv_cache *c, int32_t *seq_n, int64_t max_tokens, const void *k_new,
                              const void *v_new, int32_t in_dtype, const void *t_k_f16, const void *q, int32_t q_dtype,
                              const float *t_k_inv_t, float *q_t, int32_t num_q_heads, int32_t num_splits,
                              void *workspace, size_t workspace_bytes, float *out, void *stream) {
  if (!seq_n || !t_k_inv_t || !k_new || !v_new || !t_k_f16) return WUSHKV_ERR_NULL;
  // every check first, so that a failing call enqueues nothing
  int st = decode_impl(c, nullptr, max_tokens, nullptr, seq_n, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits,
                       workspace, workspace_bytes, out, stream, nullptr, true, 1);
  if (st != WUSHKV_OK) return st;
  AppendArgs app;
  // a sequence is stepped only while its next length fits max_tokens (<= capacity): the
  // flush, the append and the count update all skip it otherwise, and its rows are NaN
  st = append_flush_impl(c, nullptr, 0, nullptr, seq_n, 1, k_new, v_new, in_dtype, t_k_f16, stream, &app,
                         max_tokens);
  if (st != WUSHKV_OK) return st;
  st = decode_impl(c, nullptr, max_tokens, nullptr, seq_n, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits,
                   workspace, workspace_bytes, out, stream, &app, false, 1);
  if (st != WUSHKV_OK) return st;
  if (launch_advance(seq_n, c->batch, 1, max_tokens, (hipStream_t)stream) != hipSuccess) return WUSHKV_ERR_HIP;
  return hip_status();
}

int wushkv_decode_attention_device(const wushkv_cache *c, const int32_t *seq_n, int64_t max_tokens, const void *q,
                                   int32_t q_dtype, const float *t_k_inv_t, float *q_t, int32_t num_q_heads,
                                   int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                                   void *stream) {
  if (!seq_n) return WUSHKV_ERR_NULL;
  return decode_impl(c, nullptr, max_tokens, nullptr, seq_n, q, q_dtype, q_t, t_k_inv_t, num_q_heads, num_splits, workspace,
                     workspace_bytes, out, stream);
}

}  // extern "C"
