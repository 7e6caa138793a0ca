"""Helpers of the GPU parity tests: run the HIP path through the C ABI, read the
device planes back, and compare them with the CPU oracle element by element.

Parity rule (codes and parameters):
  * FP16 windows: bitwise equal.
  * Parameters: equal.  (The rule admits 1 fp16 ulp where the oracle's pre-rounding
    value lies within 1e-6 (relative) of an fp16 rounding midpoint; the flush decides
    such parameters again in fp64, so the tests require them equal.)
  * Codes: unpacked from the device planes and compared with the oracle's codes
    of its exact x under the device's stored parameters; a mismatch is allowed
    only within 1e-6*max(|b|, bin width) of a decision boundary b, and such
    mismatches may number at most 1e-5 of all elements.
Decode: relative L2 error over the step's outputs <= 2e-3 end to end (inputs ->
oracle), and the oracle run on the device's own cache contents and q~ isolates
the decode kernel.
"""
import math
import sys

import numpy as np
import torch

import bit_kv_cache_amd as W
from oracle import layout as LY
from oracle import wushkv_ref as R
from synth import gen

QN = {W.Q_QUEST: "quest", W.Q_AFFINE: "affine", "quest": "quest", "affine": "affine"}
QC = {"quest": W.Q_QUEST, "affine": W.Q_AFFINE}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def spec_of(w, capacity=None):
    return W.CacheSpec(batch=w.batch, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                       capacity=capacity or w.capacity, sink=w.sink, recent=w.recent, chunk=w.chunk,
                       bits_k=w.bits_k, bits_v=w.bits_v, quant_k=QC[w.quant_k], quant_v=QC[w.quant_v],
                       clip_mult=w.clip_mult, pct_lo=w.pct_lo, pct_hi=w.pct_hi)


def plane_arrays(cache):
    s = cache.spec
    B, H, d = s.batch, s.num_kv_heads, s.head_dim
    sizes = s.plane_bytes()
    pl = {p: cache.planes[p].cpu().numpy()[: sizes[p]] for p in W.PLANES}
    out = {
        "sink_k": pl["sink_k"].view(np.float16).reshape(B, H, s.sink, d),
        "sink_v": pl["sink_v"].view(np.float16).reshape(B, H, s.sink, d),
        "ring_k": pl["ring_k"].view(np.float16).reshape(B, H, s.recent + s.chunk, d),
        "ring_v": pl["ring_v"].view(np.float16).reshape(B, H, s.recent + s.chunk, d),
    }
    body_cap = -(-(s.capacity - s.sink) // 64) * 64
    kp = 1 if s.quant_k == W.Q_QUEST else 2
    vp = 1 if s.quant_v == W.Q_QUEST else 2
    out["par_k"] = pl["par_k"].view(np.float16).reshape(B, H, body_cap, kp)
    out["par_v"] = pl["par_v"].view(np.float16).reshape(B, H, body_cap, vp)
    out["codes_k"] = pl["codes_k"].reshape(B, H, -1)
    out["codes_v"] = pl["codes_v"].reshape(B, H, -1)
    out["body_cap"] = body_cap
    return out


def _param_check(gpu, exact, what):
    """gpu fp16 params vs the oracle's pre-rounding values rounded to fp16: equal.  Also
    counts the rows whose exact value lies within 1e-6 of an fp16 rounding midpoint (the
    ones the flush decides again in fp64); returns (mismatches, near-midpoint rows)."""
    g = gpu.astype(np.float64)
    want = R.f16(exact)
    bad = ~((g == want) | (np.isnan(g) & np.isnan(want)))
    near = R.fp16_midpoint_near(exact)
    assert not bad.any(), (f"{what}: {bad.sum()} parameters differ ({(bad & near).sum()} of them near a rounding "
                           f"midpoint); first at {np.argwhere(bad)[:3].tolist()} gpu={g[bad][:3]} want={want[bad][:3]} "
                           f"exact={np.asarray(exact)[bad][:3]}")
    return int(bad.sum()), int(near.sum())


def check_head(pa, spec, b, g, k_in, v_in, t16, n, stats):
    """Compare the device cache of (b, g) after n tokens with the oracle built
    from the exact inputs k_in/v_in [>=n, d] (float64 numpy)."""
    S, Rr, C, d = spec.sink, spec.recent, spec.chunk, spec.head_dim
    qk, qv = QN[spec.quant_k], QN[spec.quant_v]
    c = R.build_head_cache(k_in, v_in, t16, n, sink=S, recent=Rr, chunk=C, quant_k=qk, quant_v=qv,
                           bits_k=spec.bits_k, bits_v=spec.bits_v, clip_mult=spec.clip_mult,
                           pct_lo=spec.pct_lo, pct_hi=spec.pct_hi)
    ns, nb = c.sink_n, c.body_n
    # windows bitwise
    assert np.array_equal(pa["sink_k"][b, g, :ns].astype(np.float64), c.sink_k), "sink_k"
    assert np.array_equal(pa["sink_v"][b, g, :ns].astype(np.float64), c.sink_v), "sink_v"
    if len(c.recent_pos):
        slots = (c.recent_pos - S) % (Rr + C)
        assert np.array_equal(pa["ring_k"][b, g, slots].astype(np.float64), c.recent_k), "ring_k"
        assert np.array_equal(pa["ring_v"][b, g, slots].astype(np.float64), c.recent_v), "ring_v"
    if nb == 0:
        return c
    for name, x, quant, bits in (("k", c.body_xk, qk, spec.bits_k), ("v", c.body_xv, qv, spec.bits_v)):
        gp = pa["par_" + name][b, g, :nb].astype(np.float64)
        ex = R.params_exact(x, quant, bits, spec.clip_mult, spec.pct_lo, spec.pct_hi)
        nbad, nnear = _param_check(gp, ex, "par_" + name)
        stats["param_ulp"] = stats.get("param_ulp", 0) + nbad
        stats["param_near_mid"] = stats.get("param_near_mid", 0) + nnear
        if name == "k":
            codes = LY.unpack_k(pa["codes_k"][b, g], bits, d, nb)
        else:
            codes = LY.unpack_v(pa["codes_v"][b, g], bits, d, nb)
        want = R.codes_from_params(x, quant, bits, gp)
        mism = codes != want
        if mism.any():
            band = R.near_boundary(x, quant, bits, gp)
            outside = mism & ~band
            assert not outside.any(), f"codes_{name}: {outside.sum()} mismatches outside the boundary band, e.g. {np.argwhere(outside)[:3].tolist()}"
        stats["code_mism"] = stats.get("code_mism", 0) + int(mism.sum())
        stats["code_total"] = stats.get("code_total", 0) + mism.size
        assert codes.min() >= 0 and codes.max() < 2 ** bits
    return c


def device_head_cache(pa, spec, b, g, n):
    """An oracle HeadCache holding exactly the device's cache contents."""
    S, Rr, C, d = spec.sink, spec.recent, spec.chunk, spec.head_dim
    qk, qv = QN[spec.quant_k], QN[spec.quant_v]
    c = R.HeadCache()
    nb = R.n_quantized(n, S, Rr, C)
    ns = min(n, S)
    c.sink_k = pa["sink_k"][b, g, :ns].astype(np.float64)
    c.sink_v = pa["sink_v"][b, g, :ns].astype(np.float64)
    pos = np.arange(S + nb, n) if n > S else np.arange(0)
    slots = (pos - S) % (Rr + C)
    c.recent_k = pa["ring_k"][b, g, slots].astype(np.float64)
    c.recent_v = pa["ring_v"][b, g, slots].astype(np.float64)
    pk = pa["par_k"][b, g, :nb].astype(np.float64)
    pv = pa["par_v"][b, g, :nb].astype(np.float64)
    ck = LY.unpack_k(pa["codes_k"][b, g], spec.bits_k, d, nb)
    cv = LY.unpack_v(pa["codes_v"][b, g], spec.bits_v, d, nb)
    c.body_k = R.dequantize(ck, qk, spec.bits_k, pk)
    c.body_v = R.dequantize(cv, qv, spec.bits_v, pv)
    return c


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def max_head_rel(a, b):
    """The largest relative L2 error of one (batch row, query head) output row."""
    a = np.asarray(a, np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, np.float64).reshape(-1, np.shape(b)[-1])
    return float(np.max(np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)))


def paged_plane_arrays(pc):
    """plane_arrays of a paged cache, each sequence's body rows gathered from the pools
    through its page table into the contiguous layout, so that check_head and
    device_head_cache read the paged cache itself."""
    s = pc.spec
    B, H, d = s.batch, s.num_kv_heads, s.head_dim
    body_cap = -(-(s.capacity - s.sink) // 64) * 64
    page = pc.pages.page_tokens
    npages = pc.pages.num_pages
    table = pc.table.cpu().numpy()
    rows = {"codes_k": d * s.bits_k // 8, "codes_v": d * s.bits_v // 8,
            "par_k": 2 * (1 if s.quant_k == W.Q_QUEST else 2), "par_v": 2 * (1 if s.quant_v == W.Q_QUEST else 2)}
    out = {}
    for p in ("sink_k", "sink_v", "ring_k", "ring_v"):
        n = {"sink": s.sink, "ring": s.recent + s.chunk}[p[:4]]
        out[p] = pc.planes[p].cpu().numpy()[: B * H * n * d * 2].view(np.float16).reshape(B, H, n, d)
    for p, r in rows.items():
        pool = pc.planes[p].cpu().numpy()[: npages * H * page * r].reshape(npages, H, page, r)
        cont = np.zeros((B, H, body_cap, r), dtype=np.uint8)
        for b in range(B):
            for lp in range(-(-body_cap // page)):
                n = min(page, body_cap - lp * page)
                cont[b, :, lp * page:lp * page + n] = pool[table[b, lp], :, :n]
        out[p] = cont
    kp, vp = rows["par_k"] // 2, rows["par_v"] // 2
    out["par_k"] = out["par_k"].reshape(B, H, -1).view(np.float16).reshape(B, H, body_cap, kp)
    out["par_v"] = out["par_v"].reshape(B, H, -1).view(np.float16).reshape(B, H, body_cap, vp)
    out["codes_k"] = out["codes_k"].reshape(B, H, -1)
    out["codes_v"] = out["codes_v"].reshape(B, H, -1)
    out["body_cap"] = body_cap
    return out


def check_decode_lengths(pa, spec, w, k, v, t16, lengths, q, qt, out, heads=None, what="decode", tol=2e-3):
    """The decode of sequences holding lengths[b] tokens against the oracle, on the
    sampled (batch row, KV head) pairs (default: all): end to end (the oracle's own cache
    from the inputs k, v [B, Hkv, >=n, d] and its exact q~), and on the device's own cache
    contents with the device's q~ (the decode kernel alone).  Reports the pooled and the
    largest per-(batch row, query head) relative L2 errors."""
    G = w.group
    heads = heads or [(b, g) for b in range(len(lengths)) for g in range(w.num_kv_heads)]
    qn = q.float().cpu().numpy().astype(np.float64)
    qtn = qt.cpu().numpy().astype(np.float64)
    on = out.cpu().numpy().astype(np.float64)
    got, ref_e2e, ref_dev = [], [], []
    for b, g in heads:
        n = int(lengths[b])
        kk = k[b, g].float().cpu().numpy().astype(np.float64)
        vv = v[b, g].float().cpu().numpy().astype(np.float64)
        t = t16[g].numpy() if hasattr(t16[g], "numpy") else t16[g]
        c_or = R.build_head_cache(kk, vv, t, n, sink=w.sink, recent=w.recent, chunk=w.chunk, quant_k=w.quant_k,
                                  quant_v=w.quant_v, bits_k=w.bits_k, bits_v=w.bits_v, clip_mult=w.clip_mult,
                                  pct_lo=w.pct_lo, pct_hi=w.pct_hi)
        c_dev = device_head_cache(pa, spec, b, g, n)
        for h in range(g * G, (g + 1) * G):
            got.append(on[b, h])
            ref_e2e.append(R.decode_head(c_or, qn[b, h], R.query_transform(t, qn[b, h])))
            ref_dev.append(R.decode_head(c_dev, qn[b, h], qtn[b, h]))
    e2e, dev = rel_l2(got, ref_e2e), rel_l2(got, ref_dev)
    e2e_max, dev_max = max_head_rel(got, ref_e2e), max_head_rel(got, ref_dev)
    say(f"[{what} parity] {len(heads)} KV heads: rel-L2 end-to-end {e2e:.3e} (max per head {e2e_max:.3e}); "
        f"vs device cache {dev:.3e} (max per head {dev_max:.3e})")
    assert np.all(np.isfinite(on))
    assert dev <= 1e-4, dev
    if tol is not None:
        assert e2e <= tol, e2e
    return dict(e2e=e2e, e2e_max=e2e_max, dev=dev, dev_max=dev_max)


class Run:
    """A workload run on the device: inputs, transforms, cache, decode steps."""

    def __init__(self, w, layer=0, n_total=None, device="cuda"):
        self.w = w
        self.layer = layer
        self.n_total = n_total or w.capacity
        say(f"[gen] {w.name} B={w.batch} Hkv={w.num_kv_heads} G={w.group} d={w.head_dim} n={self.n_total}")
        self.k, self.v = gen.kv_tensors(w, layer, self.n_total, device)
        t16, tinvt = gen.key_transforms(w, layer)
        self.t16_cpu = t16
        self.t16 = t16.to(device)
        self.tinvt = tinvt.to(device)
        self.spec = spec_of(w, capacity=self.n_total)
        self.cache = W.KVCache(self.spec, device)

    def append(self, n_new):
        n0 = self.cache.n
        say(f"[append_flush] n_before={n0} n_new={n_new}")
        W.append_flush(self.cache, self.k[:, :, n0:n0 + n_new].contiguous(), self.v[:, :, n0:n0 + n_new].contiguous(),
                       self.t16)

    def decode(self, step, num_splits=0):
        q = gen.queries(self.w, self.layer, step, self.k.device)
        say(f"[decode] n={self.cache.n} step={step} splits={num_splits}")
        qt = W.query_transform(self.tinvt, q, self.w.num_kv_heads)
        out = W.decode_attention(self.cache, q, qt, num_splits=num_splits)
        torch.cuda.synchronize()
        return q, qt, out

    def inputs_cpu(self, b, g):
        return (self.k[b, g].float().cpu().numpy().astype(np.float64),
                self.v[b, g].float().cpu().numpy().astype(np.float64))

    def check_cache(self, heads=None):
        torch.cuda.synchronize()
        pa = plane_arrays(self.cache)
        stats = {}
        heads = heads or [(b, g) for b in range(self.w.batch) for g in range(self.w.num_kv_heads)]
        for b, g in heads:
            k, v = self.inputs_cpu(b, g)
            check_head(pa, self.spec, b, g, k, v, self.t16_cpu[g].numpy(), self.cache.n, stats)
        if stats.get("code_total"):
            assert stats["code_mism"] <= 1e-5 * stats["code_total"], stats
        return pa, stats

    def check_decode(self, q, qt, out, heads=None, tol=2e-3):
        """End-to-end and kernel-isolated relative L2 over the sampled heads."""
        pa = plane_arrays(self.cache)
        w = self.w
        G = w.group
        heads = heads or [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
        qn = q.float().cpu().numpy().astype(np.float64)
        qtn = qt.cpu().numpy().astype(np.float64)
        on = out.cpu().numpy().astype(np.float64)
        ref_e2e, ref_dev, got = [], [], []
        for b, g in heads:
            k, v = self.inputs_cpu(b, g)
            t = self.t16_cpu[g].numpy()
            c_or = R.build_head_cache(k, v, t, self.cache.n, sink=w.sink, recent=w.recent, chunk=w.chunk,
                                      quant_k=w.quant_k, quant_v=w.quant_v, bits_k=w.bits_k, bits_v=w.bits_v,
                                      clip_mult=w.clip_mult, pct_lo=w.pct_lo, pct_hi=w.pct_hi)
            c_dev = device_head_cache(pa, self.spec, b, g, self.cache.n)
            for h in range(g * G, (g + 1) * G):
                ref_e2e.append(R.decode_head(c_or, qn[b, h], R.query_transform(t, qn[b, h])))
                ref_dev.append(R.decode_head(c_dev, qn[b, h], qtn[b, h]))
                got.append(on[b, h])
        e2e, dev = rel_l2(got, ref_e2e), rel_l2(got, ref_dev)
        e2e_max, dev_max = max_head_rel(got, ref_e2e), max_head_rel(got, ref_dev)
        say(f"[decode parity] rel-L2 end-to-end {e2e:.3e} (max per head {e2e_max:.3e})  "
            f"vs device cache {dev:.3e} (max per head {dev_max:.3e})")
        assert np.all(np.isfinite(on))
        assert dev <= 1e-4, dev
        assert e2e <= tol, e2e
        return e2e, dev
