"""CPU oracle of the WUSH-KV online hot path (plain numpy, float64).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check of __graft_entry__ and
the cpu_baseline leg of bench.py may import this module.  The product path
(bit_kv_cache_amd) never imports it and shares no code with it.

What it follows (cited by page title and section):

* WUSH-KV digest, slinene.github.io ("WUSH-KV：数据自适应变换的 KV Cache
  低比特量化"), section 方法关键点 (method key points): the key transform sits
  after RMSNorm and RoPE and costs one d x d product per new token and per
  query; the value transform is folded into W_V / W_O, so V is quantized as
  is; FP16 sink + recent windows with chunked flush.  Section 工作参考价值
  (takeaways) gives the sizes sink 64 / recent 256 / flush chunk 8 or 16 and
  names the two quantizers (QuEST INT, OSCAR-style percentile-clipped affine).
* Paper review blog ("[논문리뷰] WUSH-KV ..."), Key Terms & Definitions: QuEST is
  a per-token quantizer with RMS-based scaling and bin-centre reconstruction;
  in GQA several query heads share one KV head.
* Abstract (weekinpapers.com and fugumt.com pages): keys transformed after
  RoPE, values folded into weights, paired with clipped quantizers.

Where the pages leave a step open, the reading taken is noted on the function
and listed with the others in the design notes of the repository.

Pinned by tests/test_oracle_*.py against closed forms, library routines
(numpy.percentile, numpy.linalg.inv, torch scaled_dot_product_attention),
hand-worked fixtures under tests/golden/, and brute force on tiny inputs.
The pages print no worked example and every number they report needs trained
models and datasets, so none of those numbers pins anything here.
"""
import math

import numpy as np

QUEST = "quest"
AFFINE = "affine"


# ----------------------------------------------------------------------------
# dtype helpers
# ----------------------------------------------------------------------------

def f16(x):
    """Round to IEEE binary16, round-to-nearest-even, returned as float64.

    The FP16 windows and all stored quantizer parameters are fp16 (digest,
    takeaways: FP16 sink/recent windows; affine scale and zero in fp16)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def bf16(x):
    """Round float32 values to bfloat16 (round-to-nearest-even), as float64."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


# ----------------------------------------------------------------------------
# cache policy (digest, takeaways and method key points: FP16 sink + recent
# windows, tokens leaving the recent window quantized in chunks)
# ----------------------------------------------------------------------------

def n_quantized(n, sink, recent, chunk):
    """Number of quantized (body) tokens once n tokens are cached.

    Reading: the ring holds up to recent+chunk tokens; when it reaches
    recent+chunk the oldest `chunk` tokens are flushed, so the body grows in
    whole chunks and the recent window holds between `recent` and
    recent+chunk-1 tokens once it is full."""
    return chunk * (max(0, n - sink - recent) // chunk)


def region(p, n, sink, recent, chunk):
    """'sink' | 'body' | 'recent' for token position p of an n-token cache."""
    q = n_quantized(n, sink, recent, chunk)
    if p < sink:
        return "sink"
    if p < sink + q:
        return "body"
    return "recent"


def ring_slot(p, sink, recent, chunk):
    """Ring slot of a recent-window token (ring of recent+chunk fp16 rows).
    With recent a multiple of chunk, a flushed chunk occupies consecutive
    slots and never wraps."""
    return (p - sink) % (recent + chunk)


# ----------------------------------------------------------------------------
# quantizers
# ----------------------------------------------------------------------------

def quest_params(x, bits, clip_mult):
    """QuEST per-token step: r = RMS of the row, step = 2*c*r/L, stored fp16.

    Review blog, Key Terms: RMS-based scaling and bin-centre reconstruction.
    Reading: L = 2**bits equal bins over [-c*r, c*r] (c = clip multiplier,
    2.5 in the workloads), one fp16 step per token."""
    return f16(quest_step_exact(x, bits, clip_mult))


def quest_step_exact(x, bits, clip_mult):
    """The QuEST step 2*c*r/L before its fp16 rounding."""
    L = 2 ** bits
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1))
    return 2.0 * clip_mult * r / L


def quest_codes(x, step, bits):
    """Bin index floor(x/step + L/2) clipped to [0, L-1]; a zero step gives L/2.

    Codes use the stored fp16 step, so the half-bin error bound holds for the
    values actually reconstructed."""
    L = 2 ** bits
    x = np.asarray(x, dtype=np.float64)
    step = np.asarray(step, dtype=np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.floor(x / step + L / 2)
    q = np.where(step == 0, L // 2, q)
    return np.clip(q, 0, L - 1).astype(np.int64)


def quest_dequant(codes, step, bits):
    """Bin centre (q - (L-1)/2) * step."""
    L = 2 ** bits
    return (np.asarray(codes, dtype=np.float64) - (L - 1) / 2.0) * np.asarray(step, np.float64)[..., None]


def percentile_linear(x_sorted, pct):
    """Percentile of each sorted row with linear interpolation between order
    statistics (virtual index (d-1)*pct/100).  Reading: the pages name
    percentile clipping without fixing the convention; linear interpolation
    is the common default."""
    xs = np.asarray(x_sorted, dtype=np.float64)
    d = xs.shape[-1]
    h = (d - 1) * (pct / 100.0)
    i = int(math.floor(h))
    t = h - i
    if i + 1 >= d:
        return xs[..., d - 1].copy()
    return xs[..., i] + t * (xs[..., i + 1] - xs[..., i])


def affine_params(x, bits, pct_lo, pct_hi):
    """Percentile-clipped affine parameters of each token row.

    Digest, takeaways / method key points: OSCAR-style percentile-clipped
    affine quantizer.  Reading: lo/hi are the pct_lo / pct_hi percentiles of
    the row's d values, scale s = (hi - lo)/(L - 1) and zero z = lo, both
    stored fp16."""
    s, lo = affine_params_exact(x, bits, pct_lo, pct_hi)
    return f16(s), f16(lo)


def affine_params_exact(x, bits, pct_lo, pct_hi):
    """(scale, zero) of the affine quantizer before their fp16 rounding."""
    L = 2 ** bits
    xs = np.sort(np.asarray(x, dtype=np.float64), axis=-1)
    lo = percentile_linear(xs, pct_lo)
    hi = percentile_linear(xs, pct_hi)
    return (hi - lo) / (L - 1), lo


def affine_codes(x, scale, zero, bits):
    """Nearest level rint((x - z)/s) (half to even) clipped to [0, L-1];
    a zero scale gives code 0."""
    L = 2 ** bits
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)[..., None]
    z = np.asarray(zero, dtype=np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((x - z) / s)
    q = np.where(s == 0, 0, q)
    return np.clip(q, 0, L - 1).astype(np.int64)


def affine_dequant(codes, scale, zero):
    """Level value z + q*s."""
    return (np.asarray(zero, np.float64)[..., None]
            + np.asarray(codes, dtype=np.float64) * np.asarray(scale, np.float64)[..., None])


def quantize(x, quant, bits, clip_mult=2.5, pct_lo=0.5, pct_hi=99.5):
    """Quantize rows; returns (codes, params) with params shaped [..., 1] for
    QuEST (step) or [..., 2] for affine (scale, zero)."""
    if quant == QUEST:
        st = quest_params(x, bits, clip_mult)
        return quest_codes(x, st, bits), st[..., None]
    if quant == AFFINE:
        s, z = affine_params(x, bits, pct_lo, pct_hi)
        return affine_codes(x, s, z, bits), np.stack([s, z], axis=-1)
    raise ValueError(quant)


def params_exact(x, quant, bits, clip_mult=2.5, pct_lo=0.5, pct_hi=99.5):
    """Parameters before fp16 rounding, shaped like quantize()'s params."""
    if quant == QUEST:
        return quest_step_exact(x, bits, clip_mult)[..., None]
    s, z = affine_params_exact(x, bits, pct_lo, pct_hi)
    return np.stack([s, z], axis=-1)


def codes_from_params(x, quant, bits, params):
    """Codes of rows x under given (e.g. device-stored) parameters."""
    params = np.asarray(params, dtype=np.float64)
    if quant == QUEST:
        return quest_codes(x, params[..., 0], bits)
    return affine_codes(x, params[..., 0], params[..., 1], bits)


def dequantize(codes, quant, bits, params):
    params = np.asarray(params, dtype=np.float64)
    if quant == QUEST:
        return quest_dequant(codes, params[..., 0], bits)
    return affine_dequant(codes, params[..., 0], params[..., 1])


def decision_boundaries(quant, bits, params):
    """[..., L-1] decision boundaries of each row, and the bin width."""
    L = 2 ** bits
    params = np.asarray(params, dtype=np.float64)
    if quant == QUEST:
        st = params[..., 0:1]
        k = np.arange(1, L, dtype=np.float64)
        return (k - L / 2) * st, st[..., 0]
    s, z = params[..., 0:1], params[..., 1:2]
    k = np.arange(0, L - 1, dtype=np.float64)
    return z + (k + 0.5) * s, s[..., 0]


def near_boundary(x, quant, bits, params, rel=1e-6):
    """True where x lies within rel*max(|b|, bin width) of a decision boundary b."""
    b, width = decision_boundaries(quant, bits, params)
    x = np.asarray(x, dtype=np.float64)[..., :, None]
    tol = rel * np.maximum(np.abs(b), width[..., None])[..., None, :]
    return np.any(np.abs(x - b[..., None, :]) <= tol, axis=-1)


def fp16_midpoint_near(v, rel=1e-6):
    """True where v lies within rel of a rounding midpoint between two
    adjacent fp16 values (where a 1-ulp difference of the stored fp16 is a
    rounding-order effect, not an error)."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    hv = h.astype(np.float64)
    m1, m2 = (hv + up) / 2, (hv + dn) / 2
    tol = rel * np.maximum(np.abs(v), np.finfo(np.float16).tiny)
    return (np.abs(v - m1) <= tol) | (np.abs(v - m2) <= tol)


# ----------------------------------------------------------------------------
# transforms (digest, method key points: k' = T_K k after RoPE; the query takes
# the matching inverse-transpose so that q . k is unchanged)
# ----------------------------------------------------------------------------

def key_transform(t16, k16):
    """Transformed keys T k for rows k: [..., d] @ T^T.  T is the fp16 matrix
    actually used, converted exactly."""
    t = np.asarray(t16, dtype=np.float64)
    return np.asarray(k16, dtype=np.float64) @ t.T


def query_transform(t16, q):
    """q~ = T^{-T} q for rows q, with the inverse taken in float64 from the
    fp16 T, so that (T^{-T} q) . (T k) = q . k."""
    tinv = np.linalg.inv(np.asarray(t16, dtype=np.float64))
    return np.asarray(q, dtype=np.float64) @ tinv


# ----------------------------------------------------------------------------
# cache contents of one (batch row, KV head)
# ----------------------------------------------------------------------------

class HeadCache:
    """What the cache holds for one (batch row, KV head) after n tokens.

    Attributes (float64 unless stated):
      sink_k, sink_v   [min(n,S), d]  fp16 values of the first tokens
      recent_pos       positions of the recent-window tokens
      recent_k, recent_v [len, d]    fp16 values (raw post-RoPE keys)
      body_xk          [Q, d] transformed keys T k16 of the body (exact)
      body_xv          [Q, d] values v16 of the body
      codes_k/codes_v  [Q, d] int codes (None when quant is None)
      par_k/par_v      [Q, 1|2] fp16 parameters
      body_k/body_v    [Q, d] what the body reconstructs to (dequantized, or
                       the exact x when quant is None)
    """


def build_head_cache(k, v, t16, n, *, sink, recent, chunk, quant_k, quant_v,
                     bits_k, bits_v, clip_mult=2.5, pct_lo=0.5, pct_hi=99.5):
    """Cache contents of one (batch row, KV head) holding the first n tokens
    of the rows k, v ([>=n, d], the exact input values).

    Every token is stored as its fp16 value; body tokens are quantized from
    that fp16 value, keys after the transform T k16 and values as they are
    (their transform is folded into the weights).  quant_k/quant_v None keeps
    the body unquantized (exact x), for invariance checks."""
    c = HeadCache()
    k16 = f16(np.asarray(k, np.float64)[:n])
    v16 = f16(np.asarray(v, np.float64)[:n])
    q = n_quantized(n, sink, recent, chunk)
    ns = min(n, sink)
    c.n, c.sink_n, c.body_n = n, ns, q
    c.sink_k, c.sink_v = k16[:ns], v16[:ns]
    c.recent_pos = np.arange(sink + q, n) if n > sink else np.arange(0)
    c.recent_k, c.recent_v = k16[sink + q:n], v16[sink + q:n]
    c.body_xk = key_transform(t16, k16[sink:sink + q])
    c.body_xv = v16[sink:sink + q]
    for name, x, quant, bits in (("k", c.body_xk, quant_k, bits_k), ("v", c.body_xv, quant_v, bits_v)):
        if quant is None:
            codes, par, rec = None, None, x.copy()
        else:
            codes, par = quantize(x, quant, bits, clip_mult, pct_lo, pct_hi)
            rec = dequantize(codes, quant, bits, par)
        setattr(c, "codes_" + name, codes)
        setattr(c, "par_" + name, par)
        setattr(c, "body_" + name, rec)
    return c


# ----------------------------------------------------------------------------
# decode attention (GQA: query head h reads KV head floor(h / G))
# ----------------------------------------------------------------------------

def head_scores(c, q, qt):
    """Logits of one query head over the n cached tokens, in position order.

    FP16 tokens (sink, recent) hold raw keys and take the raw query; body
    tokens hold transformed keys and take q~ = T^{-T} q.  Scale 1/sqrt(d)."""
    d = len(q)
    q = np.asarray(q, np.float64)
    qt = np.asarray(qt, np.float64)
    s_sink = c.sink_k @ q
    s_body = c.body_k @ qt
    s_rec = c.recent_k @ q
    return np.concatenate([s_sink, s_body, s_rec]) / math.sqrt(d)


def head_values(c):
    return np.concatenate([c.sink_v, c.body_v, c.recent_v], axis=0)


def softmax_attend(scores, values):
    m = np.max(scores)
    w = np.exp(scores - m)
    return (w @ values) / np.sum(w)


def decode_head(c, q, qt):
    """Softmax attention output of one query head over its KV head's cache."""
    return softmax_attend(head_scores(c, q, qt), head_values(c))


def decode(caches, q, qt):
    """caches[b][g] HeadCache; q, qt [B, Hq, d] -> out [B, Hq, d] float64."""
    q = np.asarray(q, np.float64)
    qt = np.asarray(qt, np.float64)
    B, Hq, d = q.shape
    Hkv = len(caches[0])
    G = Hq // Hkv
    out = np.empty((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            out[b, h] = decode_head(caches[b][h // G], q[b, h], qt[b, h])
    return out


def partial_attend(scores, values):
    """(m, l, o) of one partition: max logit, sum of exp(s - m), unnormalised
    weighted sum.  An empty partition gives (-inf, 0, 0)."""
    if len(scores) == 0:
        return -np.inf, 0.0, np.zeros(values.shape[-1])
    m = np.max(scores)
    w = np.exp(scores - m)
    return m, float(np.sum(w)), w @ values


def merge_partials(parts):
    """Merge (m, l, o) partials: m* = max m_p, out = sum e^{m_p-m*} o_p /
    sum e^{m_p-m*} l_p, skipping empty partitions."""
    live = [p for p in parts if p[1] > 0]
    m_star = max(p[0] for p in live)
    num = sum(math.exp(p[0] - m_star) * p[2] for p in live)
    den = sum(math.exp(p[0] - m_star) * p[1] for p in live)
    return num / den


def decode_head_split(c, q, qt, bounds):
    """Decode one head with the token sequence cut at `bounds` (sorted
    positions) into partitions that are attended separately and merged."""
    s = head_scores(c, q, qt)
    v = head_values(c)
    edges = [0] + list(bounds) + [len(s)]
    parts = [partial_attend(s[a:b], v[a:b]) for a, b in zip(edges[:-1], edges[1:])]
    return merge_partials(parts)


# ----------------------------------------------------------------------------
# calibration statistics
# ----------------------------------------------------------------------------

def calib_stats(x, group=1):
    """Second-order calibration sums per KV head (digest, method key points: the key
    transform's Hessian is built from the query heads that consume the key, a sum of
    Q Q^T, and the Gram matrices from the keys and values themselves).

    x: [B, H, T, d] (any float dtype; taken exactly in float64).  Returns float64
    [H // group, d, d]: entry g sums x x^T over every row x[b, h, t] with
    h // group == g, i.e. X_g^T X_g for X_g the stacked rows of the group."""
    x = np.asarray(x, dtype=np.float64)
    B, H, T, d = x.shape
    if H % group:
        raise ValueError("num_heads must be a multiple of group")
    out = np.zeros((H // group, d, d))
    for g in range(H // group):
        rows = x[:, g * group:(g + 1) * group].reshape(-1, d)
        out[g] = rows.T @ rows
    return out


def calib_sum_abs(x, group=1):
    """Entrywise sum |x_i| |x_j| over the same rows: the scale of the rounding error of
    any fp32 evaluation of calib_stats (error <= n u sum |x_i x_j| for n sequential adds)."""
    return calib_stats(np.abs(np.asarray(x, dtype=np.float64)), group)


# ----------------------------------------------------------------------------
# module-output error (WUSH-KV digest, "key experiments": per attention module the
# error of the module's output with the quantized cache, summarized over modules by a
# geometric mean; the pages give the numbers but not the formula, so the plain reading
# is taken: relative Frobenius error of the attention output against full precision)

def attention_fp(q, k, v):
    """Full-precision softmax attention of query rows q [m, d] over keys k [n, d] and
    values v [n, d], scale 1/sqrt(d): the output [m, d] the quantized cache is judged
    against."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = q @ k.T / math.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    return (w @ v) / w.sum(axis=-1, keepdims=True)


def module_output_error(out, ref):
    """||out - ref||_F / ||ref||_F over all of one module's outputs."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(out - ref) / np.linalg.norm(ref))


def geometric_mean(errors):
    """exp(mean(log e)) over the modules' errors."""
    e = np.asarray(errors, np.float64)
    return float(np.exp(np.mean(np.log(e))))
