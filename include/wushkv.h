/*
 * wushkv.h -- C ABI of the WUSH-KV online hot path on AMD Instinct MI355X (gfx950).
 *
 * The method (WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms):
 *   - keys pass through a per-KV-head invertible d x d transform T_K applied
 *     after RMSNorm and RoPE, one d x d product per new token, and each query
 *     takes the matching inverse-transpose so that q . k is unchanged
 *     (WUSH-KV digest, slinene.github.io, section "method key points");
 *   - values need no online transform: their transform is folded into the
 *     value and output projection weights (same section);
 *   - the cache keeps an FP16 sink window and an FP16 recent window and
 *     quantizes tokens leaving the recent window in chunks of 8 or 16 (digest,
 *     sections "takeaways" and "method key points");
 *   - the per-token quantizer is QuEST INT (RMS-based scaling, bin-centre
 *     reconstruction; review blog "[논문리뷰] WUSH-KV", Key Terms) or an
 *     OSCAR-style percentile-clipped affine quantizer (digest, "takeaways").
 *   - several query heads share one KV head (grouped-query attention; review
 *     blog, Key Terms); query head h reads KV head h / G, G = Hq / Hkv.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers (hipMalloc / torch CUDA memory)
 *     owned by the caller; the library allocates nothing, keeps no data
 *     between calls (only cached device properties) and never synchronizes the
 *     stream.  It is thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work of a call is enqueued on that stream, in order.
 *   - Tensors are dense, row-major, in the shapes documented; every tensor
 *     pointer must be 16-byte aligned (WUSHKV_ERR_ALIGN otherwise), except the
 *     int32 token-count arrays and page tables, which need 4 bytes.
 *   - Every argument check runs on the host before any launch; a failing call
 *     enqueues nothing.  After launching, hipGetLastError() is checked and
 *     mapped to WUSHKV_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronization.  No C++ exception crosses the ABI.
 *   - Inputs must be finite with |x| < 65504 (the fp16 range); anything else
 *     gives unspecified (but memory-safe) results.
 */
#ifndef WUSHKV_H
#define WUSHKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: append/flush, query transform, decode (plain and fused).  2: adds the decode
 * step, ragged, device-count and paged calls, and the calibration sums.  3: adds
 * wushkv_decode_attention_generic (the per-call choice of the fp32 decode kernel).  4: adds
 * wushkv_decode_attention_noalloc.  5: adds wushkv_append_flush_hadamard. */
#define WUSHKV_ABI_VERSION 5

typedef enum {
  WUSHKV_OK = 0,
  WUSHKV_ERR_NULL = 1,        /* a required pointer is NULL                       */
  WUSHKV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent           */
  WUSHKV_ERR_UNSUPPORTED = 3, /* a valid request the library does not implement   */
  WUSHKV_ERR_CAPACITY = 4,    /* token count beyond the cache capacity            */
  WUSHKV_ERR_WORKSPACE = 5,   /* decode workspace missing or too small            */
  WUSHKV_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned                 */
  WUSHKV_ERR_HIP = 7          /* the HIP runtime reported an error at launch time */
} wushkv_status;

typedef enum { WUSHKV_DT_F32 = 0, WUSHKV_DT_BF16 = 1, WUSHKV_DT_F16 = 2 } wushkv_dtype;

/* QUEST: per-token step s = fp16(2 * clip_mult * rms(x) / L), L = 2^bits, code
 *   q = clamp(floor(x / s + L/2), 0, L-1), reconstruction (q - (L-1)/2) * s; a zero
 *   step gives code L/2.  AFFINE_PCT: lo / hi = the pct_lo / pct_hi percentiles of
 *   the token's d values (linear interpolation between order statistics at virtual
 *   index (d-1)*pct/100), scale s = fp16((hi - lo)/(L-1)), zero z = fp16(lo), code
 *   q = clamp(rint((x - z)/s), 0, L-1) (half to even), reconstruction z + q*s; a
 *   zero scale gives code 0.  Keys are quantized after the transform T_K, values
 *   as they are; the quantizer input is always the token's fp16 value. */
typedef enum { WUSHKV_Q_QUEST = 0, WUSHKV_Q_AFFINE_PCT = 1 } wushkv_quant;

enum {
  WUSHKV_PLANE_SINK_K = 0, WUSHKV_PLANE_SINK_V = 1,
  WUSHKV_PLANE_RING_K = 2, WUSHKV_PLANE_RING_V = 3,
  WUSHKV_PLANE_CODES_K = 4, WUSHKV_PLANE_CODES_V = 5,
  WUSHKV_PLANE_PAR_K = 6, WUSHKV_PLANE_PAR_V = 7,
  WUSHKV_NUM_PLANES = 8
};

/*
 * Cache descriptor: a host struct read at call time.  The planes are caller-owned
 * device buffers, each laid out [batch][num_kv_heads][...] with the per-(b, g)
 * part below; wushkv_plane_bytes() gives each plane's total size.
 *   S = sink, R = recent, C = chunk, body_cap = round_up(capacity - S, 64)
 *   sink_k/v   fp16 [S][d]        first S tokens (raw post-RoPE keys / values)
 *   ring_k/v   fp16 [R + C][d]    recent tokens; token p sits in slot (p - S) mod (R + C);
 *                                 keys are raw (untransformed) post-RoPE keys
 *   codes_k    u8   [body_cap][d*bits_k/8]   token-major rows of transformed-key codes
 *   codes_v    u8   [body_cap/64][8*d*bits_v] sets of 64 value-code tokens
 *   par_k/v    fp16 [body_cap][1 (QuEST step) | 2 (affine scale, zero)]
 * Code bit layout (body index u = p - S):
 *   K row:  plane 0 = d/16 u32 words, word w bits 2f..2f+1 = low 2 bits of channel 16w+f;
 *           plane 1 (bits 3) = d/32 u32, word w bit f = bit 2 of channel 32w+f;
 *           plane 1 (bits 4) = d/16 u32, word w bits 2f..2f+1 = bits 2..3 of channel 16w+f.
 *   V set:  token u = 64*sigma + 16*a + 4*c + e, channel j = 16*t + m go to lane 16*c+m,
 *           field f = 4*a + e.  plane 0 = u32 word [lane*(d/16) + t], low 2 bits of the
 *           code at bit 2*(f>>1) + 16*(f&1); plane 1 (bits 3) = u16 [lane*(d/16) + t] after
 *           plane 0, bit 2 of the code at bit (f>>1) + 8*(f&1); plane 1 (bits 4) = u32
 *           [lane*(d/16) + t] after plane 0, bits 2..3 at bit 2*(f>>1) + 16*(f&1).
 * Token p of an n-token cache is a sink token if p < S, a body token if
 * S <= p < S + Q(n) with Q(n) = C * floor(max(0, n - S - R) / C), and a recent
 * token otherwise: the ring holds up to R + C tokens and flushes its oldest C
 * when it fills.
 * Supported: head_dim in {64, 128}; bits in {2, 3, 4}; chunk >= 1; recent % chunk == 0;
 * sink >= 0; 0 <= pct_lo < pct_hi <= 100; clip_mult > 0.
 */
typedef struct {
  int32_t batch, num_kv_heads, head_dim;
  int32_t sink, recent, chunk;
  int64_t capacity;                 /* max tokens per sequence */
  int32_t bits_k, bits_v;           /* 2 | 3 | 4 */
  int32_t quant_k, quant_v;         /* wushkv_quant */
  float clip_mult;                  /* QuEST clip multiplier c (2.5) */
  float pct_lo, pct_hi;             /* affine percentiles (0.5, 99.5) */
  void *sink_k, *sink_v;
  void *ring_k, *ring_v;
  void *codes_k, *codes_v;
  void *par_k, *par_v;
} wushkv_cache;

/* Human-readable name of a status code (static string). */
const char *wushkv_status_string(int status);

/* ABI version (WUSHKV_ABI_VERSION) of the loaded library. */
int wushkv_abi_version(void);

/* Check a descriptor's sizes and options (pointers are not inspected).  Host only. */
int wushkv_cache_check(const wushkv_cache *c);

/* Total bytes of plane `plane` (WUSHKV_PLANE_*) over [batch][num_kv_heads]; 0 when
 * the descriptor fails wushkv_cache_check or the plane id is unknown. */
size_t wushkv_plane_bytes(const wushkv_cache *c, int plane);

/* The number of KV partitions wushkv_decode_attention will use for these arguments
 * (num_splits = 0 asks the library to choose); 0 when the arguments are invalid. */
int32_t wushkv_decode_num_splits(const wushkv_cache *c, int64_t n_tokens, int32_t num_q_heads,
                                 int32_t num_splits);

/* Bytes of decode workspace needed for these arguments (0 when invalid).  It takes
 * n_tokens because the split count, and so the partials' size, follow the body length
 * (num_splits = 0 lets the library pick it from the body's 64-token sets).  The
 * workspace holds the split-K partials (fp32 [batch][num_q_heads][splits + 1][d]
 * plus [..][2] maxima and sums); no initialisation is needed.  Calls that overlap
 * in time must not share a workspace. */
size_t wushkv_decode_workspace_bytes(const wushkv_cache *c, int64_t n_tokens, int32_t num_q_heads,
                                     int32_t num_splits);

/*
 * Append n_new tokens to every sequence of the cache, all of which hold n_before
 * tokens, and quantize every token the window policy flushes as a result
 * (WUSH-KV digest, "takeaways" and "method key points": FP16 sink/recent windows,
 * chunked flush; the key transform after RoPE).
 *   k_new, v_new  [batch][num_kv_heads][n_new][d] in in_dtype (F32, BF16 or F16):
 *                 post-RoPE keys and values (values already in the folded basis).
 *   t_k_f16       fp16 [num_kv_heads][d][d], row-major: the key transform, applied
 *                 as x = T_K k to each flushed key's fp16 value.
 * Sink tokens and tokens that end in the recent window are stored as fp16
 * (round-to-nearest-even); body tokens get codes and parameters.  Tokens that were
 * in the ring before the call and are flushed by it are read back from the ring.
 * Errors: NULL pointer -> ERR_NULL; bad descriptor or n_new < 0 or n_before < 0 ->
 * ERR_SHAPE; n_before + n_new > capacity -> ERR_CAPACITY; a percentile needing more
 * than 8 order statistics from either end -> ERR_UNSUPPORTED; misaligned -> ERR_ALIGN.
 * n_new == 0 is a no-op.
 */
int wushkv_append_flush(const wushkv_cache *c, int64_t n_before, int32_t n_new,
                        const void *k_new, const void *v_new, int32_t in_dtype,
                        const void *t_k_f16, void *stream);

/*
 * wushkv_append_flush with the fixed Hadamard key transform T_K = scale * H, H the
 * Sylvester-Hadamard matrix of order head_dim (H[j][i] = (-1)^popcount(i & j)), formed
 * by an in-register fast Walsh-Hadamard transform (head_dim log2(head_dim) additions per
 * key) instead of the d x d product (WUSH-KV digest, "motivation" and "key experiments":
 * fixed orthogonal transforms such as Hadamard are the baseline the data-adaptive
 * transform is compared against).  The result is that of wushkv_append_flush with t_k_f16
 * = scale * H in fp16; scale = fp16(1/sqrt(head_dim)) gives the orthonormal transform.
 * The decode takes T^{-T} = H / (scale * head_dim) as for any key transform.
 * Errors as wushkv_append_flush; scale zero, not finite or not exactly an fp16 value ->
 * ERR_SHAPE.
 */
int wushkv_append_flush_hadamard(const wushkv_cache *c, int64_t n_before, int32_t n_new,
                                 const void *k_new, const void *v_new, int32_t in_dtype,
                                 float scale, void *stream);

/*
 * Query transform q~[b][h] = T_{h/G}^{-T} q[b][h] (WUSH-KV digest, "method key
 * points": the query side takes one d x d product so that q~ . (T k) = q . k).
 *   t_k_inv_t  fp32 [num_kv_heads][d][d], row-major: T^{-T} itself, i.e. element
 *              [i][j] multiplies q[j] into q~[i]; the caller computes it (offline,
 *              like T_K) from the fp16 T_K actually used.
 *   q          [batch][num_q_heads][d] in q_dtype;  q_t  fp32 [batch][num_q_heads][d].
 * Errors: ERR_NULL, ERR_SHAPE (num_q_heads % num_kv_heads != 0, d not in {64, 128},
 * non-positive sizes), ERR_ALIGN.
 */
int wushkv_query_transform(const float *t_k_inv_t, const void *q, int32_t q_dtype,
                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, float *q_t, void *stream);

/*
 * GQA decode attention over the first n_tokens tokens of every sequence (review blog
 * "[논문리뷰] WUSH-KV", Key Terms & Definitions: grouped-query attention, several query
 * heads reading one KV head; WUSH-KV digest, "method key points": the query meets the
 * transformed keys through q~ = T^{-T} q, so q~ . (T k) = q . k, and the FP16 sink /
 * recent windows are attended unquantized):
 *   out[b][h] = sum_p softmax_p(s_p) v_p,  s_p = (q . k_p) / sqrt(d) on the FP16 sink
 *   and recent tokens (raw q, raw keys) and s_p = (q~ . x^_p) / sqrt(d) on the body
 *   (q~ from wushkv_query_transform, x^ the dequantized transformed key), v_p the
 *   fp16 value or the dequantized value.  Each KV head's data is read once for all
 *   G query heads of its group.  The body is split into num_splits KV partitions
 *   (0 = library's choice) whose partial (max, sum, weighted values) are merged with
 *   the online-softmax rule by a second kernel launched on the same stream.
 *   q      [batch][num_q_heads][d] in q_dtype;  q_t  fp32 [batch][num_q_heads][d]
 *   out    fp32 [batch][num_q_heads][d]
 *   workspace  device buffer of at least wushkv_decode_workspace_bytes() bytes.
 * Errors: ERR_NULL, ERR_SHAPE (including n_tokens < 1 and group sizes G > 16),
 * ERR_CAPACITY (n_tokens > capacity), ERR_WORKSPACE, ERR_ALIGN.
 */
int wushkv_decode_attention(const wushkv_cache *c, int64_t n_tokens,
                            const void *q, int32_t q_dtype, const float *q_t,
                            int32_t num_q_heads, int32_t num_splits,
                            void *workspace, size_t workspace_bytes,
                            float *out, void *stream);

/*
 * wushkv_decode_attention_generic: the decode of wushkv_decode_attention_ragged on the
 * plain fp32 kernel that serves every supported shape (no matrix cores; slower), chosen
 * per call.  It is a second, independent decode of the same cache, for callers that
 * cross-check the matrix-core path: the two agree within fp32 rounding (not bit for
 * bit).  Arguments, workspace and errors as wushkv_decode_attention_ragged.
 */
int wushkv_decode_attention_generic(const wushkv_cache *c, const int64_t *n_tokens,
                                    const void *q, int32_t q_dtype, const float *t_k_inv_t,
                                    float *q_t, int32_t num_q_heads, int32_t num_splits,
                                    void *workspace, size_t workspace_bytes,
                                    float *out, void *stream);

/*
 * wushkv_decode_attention with the query transform folded in (WUSH-KV digest,
 * "method key points": the query side of the key transform is one d x d product per
 * query): the decode forms q~ = T^{-T} q itself and also writes it to q_t.
 *   t_k_inv_t  fp32 [num_kv_heads][d][d], as for wushkv_query_transform.
 *   q_t        fp32 [batch][num_q_heads][d], output: exactly what
 *              wushkv_query_transform writes for the same q and t_k_inv_t.
 * out equals that of wushkv_query_transform followed by wushkv_decode_attention bit
 * for bit; one launch fewer (shapes the MFMA decode does not serve launch both).
 * Arguments, workspace and errors as wushkv_decode_attention; t_k_inv_t NULL -> ERR_NULL.
 */
int wushkv_decode_attention_fused(const wushkv_cache *c, int64_t n_tokens,
                                  const void *q, int32_t q_dtype, const float *t_k_inv_t,
                                  float *q_t, int32_t num_q_heads, int32_t num_splits,
                                  void *workspace, size_t workspace_bytes,
                                  float *out, void *stream);

/*
 * One decode step (WUSH-KV digest, "method key points": each generated token is
 * appended, the windows flush as they fill, and the query attends over the whole
 * cache): wushkv_append_flush of one token per sequence (k_new / v_new [batch]
 * [num_kv_heads][1][head_dim]) followed by wushkv_decode_attention_fused over the
 * n_before + 1 tokens, in one call.  On the MFMA path the decode writes the new token's
 * window rows itself (no separate append launch); the result is bit-identical to the two
 * calls.  Every check of both calls runs before anything is enqueued; errors as theirs.
 */
int wushkv_decode_step(const wushkv_cache *c, int64_t n_before, const void *k_new, const void *v_new,
                       int32_t in_dtype, const void *t_k_f16, const void *q, int32_t q_dtype,
                       const float *t_k_inv_t, float *q_t, int32_t num_q_heads, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, float *out, void *stream);

/*
 * wushkv_decode_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  The split-K
 * partials live in a fixed array inside the library (WUSHKV_NOALLOC_SCRATCH_BYTES per
 * GPU, held until the process ends) instead of a caller workspace; the call itself
 * allocates nothing.  Arguments, results and errors as wushkv_decode_attention minus
 * the workspace; a decode whose wushkv_decode_workspace_bytes() exceeds the array is
 * rejected with WUSHKV_ERR_WORKSPACE before anything is enqueued.  Every call on a GPU
 * shares that GPU's array (the partials need no clearing): calls that overlap in time
 * on one GPU, on any streams, race and must not be issued.
 */
#define WUSHKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int wushkv_decode_attention_noalloc(const wushkv_cache *c, int64_t n_tokens,
                                    const void *q, int32_t q_dtype, const float *q_t,
                                    int32_t num_q_heads, int32_t num_splits,
                                    float *out, void *stream);

/*
 * Ragged batches (the serving case of the WUSH-KV digest, "takeaways": the cache sits in
 * a serving stack where the sequences of a batch have different lengths).  Same cache
 * layout; each sequence keeps its own token count, and the window policy applies to each
 * sequence separately.  At most 256 sequences per cache (batch > 256 -> ERR_UNSUPPORTED).
 *
 * wushkv_append_flush_ragged: as wushkv_append_flush, with sequence b holding
 * n_before[b] tokens (host array [batch]) before the call; every sequence receives the
 * n_new tokens of its slice of k_new / v_new.  Errors as wushkv_append_flush
 * (n_before[b] < 0 -> ERR_SHAPE, n_before[b] + n_new > capacity -> ERR_CAPACITY,
 * n_before NULL -> ERR_NULL).
 */
int wushkv_append_flush_ragged(const wushkv_cache *c, const int64_t *n_before, int32_t n_new,
                               const void *k_new, const void *v_new, int32_t in_dtype,
                               const void *t_k_f16, void *stream);

/*
 * wushkv_decode_attention_ragged: the decode with sequence b attending its n_tokens[b]
 * tokens (host array [batch], each in [1, capacity]); the workspace is sized by
 * wushkv_decode_workspace_bytes for the longest sequence, and num_splits = 0 chooses
 * the split count for it.  t_k_inv_t NULL: q_t is the caller's q~ (as
 * wushkv_decode_attention); non-NULL: the decode forms q~ and writes it to q_t (as
 * wushkv_decode_attention_fused).  Errors as wushkv_decode_attention; n_tokens NULL ->
 * ERR_NULL.
 */
int wushkv_decode_attention_ragged(const wushkv_cache *c, const int64_t *n_tokens,
                                   const void *q, int32_t q_dtype, const float *t_k_inv_t,
                                   float *q_t, int32_t num_q_heads, int32_t num_splits,
                                   void *workspace, size_t workspace_bytes,
                                   float *out, void *stream);

/*
 * Device-resident token counts, for serving loops captured as a HIP graph (the same
 * serving case; a captured launch keeps the arguments it was recorded with, so counts
 * that change every step must come from memory).  seq_n is caller-owned device memory,
 * int32 [batch], 4-byte aligned; the kernels read it, and nothing else in the call
 * depends on its values, so one recorded append + decode replays as the next step.
 *
 * wushkv_append_flush_device: as wushkv_append_flush_ragged with n_before[b] = seq_n[b];
 * after its kernels (same stream) the call adds n_new to every seq_n[b].  The flush
 * kernel is always launched, sized for the most that n_new tokens can make due, and
 * sequences with nothing due return at once.  A count outside [0, capacity - n_new]
 * leaves that sequence, and its count, unchanged.  Errors: as wushkv_append_flush for
 * the host-side checks (n_new > capacity -> ERR_CAPACITY), seq_n NULL -> ERR_NULL,
 * seq_n not 4-byte aligned -> ERR_ALIGN.
 */
int wushkv_append_flush_device(const wushkv_cache *c, int32_t *seq_n, int32_t n_new, const void *k_new,
                               const void *v_new, int32_t in_dtype, const void *t_k_f16, void *stream);

/*
 * wushkv_decode_step_device: wushkv_decode_step with device counts, for a serving loop
 * recorded once into a graph: sequence b holds seq_n[b] tokens before the call, receives
 * one token, attends the seq_n[b] + 1 tokens, and its count is then advanced by one (three
 * launches: the flush, sized as in wushkv_append_flush_device; the decode, which appends
 * the token itself on the MFMA path; the count update).  The same result, bit for bit, as
 * wushkv_decode_step at the same counts.  max_tokens (host, in [1, capacity]) bounds the
 * lengths: a sequence is stepped while seq_n[b] is in [0, max_tokens - 1]; any other count
 * leaves that sequence's cache and count unchanged and makes its output rows NaN.
 */
int wushkv_decode_step_device(const wushkv_cache *c, int32_t *seq_n, int64_t max_tokens, const void *k_new,
                              const void *v_new, int32_t in_dtype, const void *t_k_f16, const void *q,
                              int32_t q_dtype, const float *t_k_inv_t, float *q_t, int32_t num_q_heads,
                              int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                              void *stream);

/*
 * wushkv_decode_attention_device: the decode with sequence b attending seq_n[b] tokens,
 * read on the device.  max_tokens (host, in [1, capacity]) bounds every count: the split
 * count (num_splits = 0) and the workspace size are those of a batch of max_tokens-token
 * sequences.  A count outside [1, max_tokens] makes that sequence's output rows NaN.
 * t_k_inv_t as in wushkv_decode_attention_ragged.  Errors as wushkv_decode_attention,
 * seq_n NULL -> ERR_NULL, seq_n not 4-byte aligned -> ERR_ALIGN.
 */
int wushkv_decode_attention_device(const wushkv_cache *c, const int32_t *seq_n, int64_t max_tokens,
                                   const void *q, int32_t q_dtype, const float *t_k_inv_t, float *q_t,
                                   int32_t num_q_heads, int32_t num_splits, void *workspace,
                                   size_t workspace_bytes, float *out, void *stream);

/*
 * Paged body (the serving case of the WUSH-KV digest, "takeaways": the cache sits in a
 * serving stack's cache manager, which hands out fixed-size blocks).  Only the quantized
 * body grows with a sequence, so only it is paged; the FP16 windows stay [batch]
 * [num_kv_heads][...] as in wushkv_cache.  With a page table the cache's code and
 * parameter planes are pools:
 *   codes_k  u8  [num_pages][num_kv_heads][page_tokens][d * bits_k / 8]
 *   codes_v  u8  [num_pages][num_kv_heads][page_tokens / 64][64-token value set]
 *   par_k/v  f16 [num_pages][num_kv_heads][page_tokens][1 or 2]
 * and body row u (token sink + u) of sequence b lives on page table[b][u / page_tokens],
 * row u mod page_tokens.  Each row has the same layout as in the contiguous planes.
 *   table        device int32 [batch][max_pages], caller-owned, 4-byte aligned; entries
 *                of pages a sequence does not reach are never read.
 *   page_tokens  a multiple of 64 (a value set never spans two pages).
 *   max_pages    logical pages per sequence: max_pages * page_tokens must cover the
 *                body of a full sequence (else ERR_CAPACITY).
 *   num_pages    physical pages in each pool.
 * An entry outside [0, num_pages) is never written through (the flush skips those rows)
 * and reads as page 0, so no access leaves the pools.  Which physical pages a sequence
 * uses, and their reuse, is the caller's business.
 */
typedef struct {
  const int32_t *table;
  int32_t page_tokens, max_pages, num_pages;
} wushkv_pages;

/* Bytes of plane `plane` of a paged cache: the pool size for code and parameter planes,
 * wushkv_plane_bytes for the window planes; 0 for invalid arguments. */
size_t wushkv_pool_bytes(const wushkv_cache *c, const wushkv_pages *pages, int plane);

/* wushkv_append_flush_ragged on a paged cache.  Errors as wushkv_append_flush_ragged,
 * plus the page-table checks (pages or its table NULL -> ERR_NULL, table misaligned ->
 * ERR_ALIGN, page_tokens / max_pages / num_pages invalid -> ERR_SHAPE, pages too few
 * for a full sequence -> ERR_CAPACITY). */
int wushkv_append_flush_paged(const wushkv_cache *c, const wushkv_pages *pages, const int64_t *n_before,
                              int32_t n_new, const void *k_new, const void *v_new, int32_t in_dtype,
                              const void *t_k_f16, void *stream);

/* wushkv_decode_attention_ragged on a paged cache; errors as that call plus the
 * page-table checks.  The workspace is sized by wushkv_decode_workspace_bytes as for the
 * unpaged cache. */
int wushkv_decode_attention_paged(const wushkv_cache *c, const wushkv_pages *pages, const int64_t *n_tokens,
                                  const void *q, int32_t q_dtype, const float *t_k_inv_t, float *q_t,
                                  int32_t num_q_heads, int32_t num_splits, void *workspace,
                                  size_t workspace_bytes, float *out, void *stream);

/*
 * Calibration statistics (WUSH-KV digest, "method key points": per KV head, the key
 * transform's Hessian is the sum of Q Q^T over the query heads that read the key and
 * the Gram matrices are the sums over the keys and values themselves; "takeaways": the
 * transforms come from one calibration pass):
 *   out[g] = sum over b, t and every head h with h / group == g of x[b][h][t] x[b][h][t]^T
 *   x      [batch][num_heads][tokens][head_dim] in dtype (BF16 or F16), e.g. post-RoPE
 *          keys (group 1: per-head Gram), values (group 1), or queries with group =
 *          num_q_heads / num_kv_heads (the key Hessian of each KV head).
 *   out    fp32 [num_heads / group][head_dim][head_dim], row-major, symmetric; written
 *          whole (no accumulation into it).
 *   workspace  device buffer of at least wushkv_calib_workspace_bytes() bytes (partial
 *          sums; no initialisation needed).
 * Products are exact in fp32 and summed in fp32 on the matrix cores; the partial sums of
 * a group are added in a fixed order, so the result is the same on every call.
 * Errors: ERR_SHAPE (non-positive sizes, num_heads % group != 0, unknown dtype),
 * ERR_UNSUPPORTED (head_dim != 128, F32 input), ERR_NULL, ERR_ALIGN (x, out or workspace
 * not 16-byte aligned), ERR_WORKSPACE.
 */
int wushkv_calib_stats(const void *x, int32_t dtype, int32_t batch, int32_t num_heads,
                       int64_t tokens, int32_t head_dim, int32_t group,
                       void *workspace, size_t workspace_bytes, float *out, void *stream);

/* Workspace bytes wushkv_calib_stats needs for these sizes; 0 for sizes it rejects. */
size_t wushkv_calib_workspace_bytes(int32_t batch, int32_t num_heads, int64_t tokens,
                                    int32_t head_dim, int32_t group);

#ifdef __cplusplus
}
#endif
#endif /* WUSHKV_H */
