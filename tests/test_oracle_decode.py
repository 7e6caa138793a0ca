"""Pins of the oracle's decode attention (CPU only).

* Transform with no quantization reduces to textbook attention over the raw
  fp16 keys: checked against torch's scaled_dot_product_attention (float64,
  KV repeated G times; G = 1 is plain multi-head attention).
* With quantization, attention equals SDPA over effective keys whose body
  rows are T^{-1} applied to the reconstructed transformed keys (computed by
  numpy.linalg.solve), and the reconstructed values.
* A pure-Python brute force that replays the window policy token by token on
  tiny shapes matches the vectorised oracle.
* Splitting the tokens into partitions and merging (m, l, o) partials gives
  the same result as one softmax (associativity), empty partitions included.
"""
import math

import numpy as np
import pytest
import torch

from oracle import wushkv_ref as R


def _inputs(seed, B, Hkv, G, n, d, tscale=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, n, d)) * 2.0
    v = rng.standard_normal((B, Hkv, n, d))
    q = rng.standard_normal((B, Hkv * G, d))
    t = []
    for _ in range(Hkv):
        qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        s = 2.0 ** rng.uniform(-2, 2, d) if tscale else np.ones(d)
        t.append((qm * s[None, :]).astype(np.float16))
    return k, v, q, np.stack(t)


def _sdpa(q, k, v, G):
    """q [B,Hq,d], k/v [B,Hkv,n,d] -> [B,Hq,d] via torch SDPA in float64."""
    kk = torch.from_numpy(np.repeat(k, G, axis=1))
    vv = torch.from_numpy(np.repeat(v, G, axis=1))
    qq = torch.from_numpy(q)[:, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, :, 0, :].numpy()


def _caches(k, v, t, n, quant_k, quant_v, bits_k=2, bits_v=2, sink=64, recent=256, chunk=8):
    B, Hkv = k.shape[:2]
    return [[R.build_head_cache(k[b, g], v[b, g], t[g], n, sink=sink, recent=recent, chunk=chunk,
                                quant_k=quant_k, quant_v=quant_v, bits_k=bits_k, bits_v=bits_v)
             for g in range(Hkv)] for b in range(B)]


def _qt(q, t, G):
    return np.stack([np.stack([R.query_transform(t[h // G], q[b, h]) for h in range(q.shape[1])])
                     for b in range(q.shape[0])])


@pytest.mark.parametrize("G,n,d", [(4, 700, 64), (1, 500, 32), (2, 333, 16), (8, 64, 16), (4, 40, 16)])
def test_transform_without_quantization_is_plain_attention(G, n, d):
    B, Hkv = 2, 2
    k, v, q, t = _inputs(G + n, B, Hkv, G, n, d)
    caches = _caches(k, v, t, n, None, None)
    out = R.decode(caches, q, _qt(q, t, G))
    ref = _sdpa(q, R.f16(k), R.f16(v), G)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("qk,qv,bk,bv", [("quest", "quest", 2, 2), ("affine", "affine", 2, 3), ("quest", "affine", 4, 2)])
def test_quantized_decode_is_attention_over_reconstructed_cache(qk, qv, bk, bv):
    B, Hkv, G, n, d = 1, 2, 4, 900, 64
    k, v, q, t = _inputs(5, B, Hkv, G, n, d)
    caches = _caches(k, v, t, n, qk, qv, bk, bv)
    out = R.decode(caches, q, _qt(q, t, G))
    keff = R.f16(k).copy()
    veff = R.f16(v).copy()
    for b in range(B):
        for g in range(Hkv):
            c = caches[b][g]
            body = slice(64, 64 + c.body_n)
            keff[b, g, body] = np.linalg.solve(t[g].astype(np.float64), c.body_k.T).T
            veff[b, g, body] = c.body_v
            # the reconstruction really is lossy (the pin is not vacuous)
            assert np.max(np.abs(keff[b, g, body] - R.f16(k[b, g, body]))) > 1e-3
    ref = _sdpa(q, keff, veff, G)
    assert np.allclose(out, ref, rtol=1e-9, atol=1e-12)


def _brute_force_decode(k, v, t, q, n, sink, recent, chunk, quant, bits):
    """Token-by-token replay of the window policy, then one query head at a
    time with explicit loops and math.exp."""
    d = len(q)
    ring, body = [], []
    for p in range(n):
        if p < sink:
            continue
        ring.append(p)
        if len(ring) == recent + chunk:
            body += ring[:chunk]
            ring = ring[chunk:]
    tinv = np.linalg.inv(t.astype(np.float64))
    qt = [sum(tinv[i][j] * q[i] for i in range(d)) for j in range(d)]  # (T^{-T} q)_j = sum_i Tinv[i][j] q_i
    scores, vals = [], []
    for p in range(n):
        k16 = [float(np.float16(x)) for x in k[p]]
        v16 = [float(np.float16(x)) for x in v[p]]
        if p in body:
            x = [sum(float(t[i][j]) * k16[j] for j in range(d)) for i in range(d)]
            cx, px = R.quantize(np.array([x]), quant, bits)
            cv, pv = R.quantize(np.array([v16]), quant, bits)
            xh = R.dequantize(cx, quant, bits, px)[0]
            vh = R.dequantize(cv, quant, bits, pv)[0]
            s = sum(qt[j] * xh[j] for j in range(d))
            vals.append(list(vh))
        else:
            s = sum(q[j] * k16[j] for j in range(d))
            vals.append(v16)
        scores.append(s / math.sqrt(d))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    return [sum(w[p] * vals[p][j] for p in range(n)) / tot for j in range(d)]


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 9, 12, 13, 16])
def test_brute_force_tiny(n):
    quant = "quest"
    rng = np.random.default_rng(n)
    d, sink, recent, chunk = 4, 2, 4, 2
    k = rng.standard_normal((n, d)) * 3
    v = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    t = np.array([[1.5, 0.25, 0, 0], [0, 1, 0.5, 0], [0.125, 0, 2, 0], [0, 0, 0.75, 0.5]], dtype=np.float16)
    c = R.build_head_cache(k, v, t, n, sink=sink, recent=recent, chunk=chunk,
                           quant_k=quant, quant_v=quant, bits_k=2, bits_v=2)
    out = R.decode_head(c, q, R.query_transform(t, q))
    ref = _brute_force_decode(k, v, t, q, n, sink, recent, chunk, quant, 2)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny_affine():
    rng = np.random.default_rng(99)
    d, sink, recent, chunk, n = 4, 2, 4, 2, 15
    k = rng.standard_normal((n, d)) * 3
    v = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    t = np.array([[1.5, 0.25, 0, 0], [0, 1, 0.5, 0], [0.125, 0, 2, 0], [0, 0, 0.75, 0.5]], dtype=np.float16)
    c = R.build_head_cache(k, v, t, n, sink=sink, recent=recent, chunk=chunk,
                           quant_k="affine", quant_v="affine", bits_k=2, bits_v=2)
    out = R.decode_head(c, q, R.query_transform(t, q))
    ref = _brute_force_decode(k, v, t, q, n, sink, recent, chunk, "affine", 2)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_split_and_merge_equals_single_softmax():
    B, Hkv, G, n, d = 1, 1, 4, 1500, 64
    k, v, q, t = _inputs(11, B, Hkv, G, n, d)
    c = _caches(k, v, t, n, "affine", "quest", 2, 3)[0][0]
    rng = np.random.default_rng(0)
    for h in range(G):
        qt = R.query_transform(t[0], q[0, h])
        ref = R.decode_head(c, q[0, h], qt)
        for trial in range(5):
            cuts = sorted(rng.integers(0, n, size=rng.integers(1, 40)).tolist())
            cuts = cuts + cuts[:2]  # duplicate cuts make empty partitions
            got = R.decode_head_split(c, q[0, h], qt, sorted(cuts))
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    m, l, o = R.partial_attend(np.array([]), np.zeros((0, d)))
    assert m == -np.inf and l == 0.0 and not o.any()
