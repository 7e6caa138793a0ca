"""wushkv_decode_step (append one token, flush if due, decode with the query transform,
in one call; on the MFMA path the decode writes the new token itself) against the two
calls it replaces, wushkv_append_flush and wushkv_decode_attention_fused, which the
parity tests hold to the oracle: caches and outputs bit for bit, over steps that cross
flushes, the sink boundary, the whole-workgroup layout, the split layout with 3-bit
values, and the generic kernel."""
import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from tests.parity_util import Run, check_decode_lengths, plane_arrays, say, spec_of

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, prefill tokens, steps); serving_whole: 32 x 8 KV heads with at
    # least 23 body sets, so the library picks 12 splits, the 12-wave layout
    "serving_whole": (configs.SERVING.scaled(batch=32), 1900, 40),
    "serving_sink": (configs.SERVING.scaled(batch=32), 60, 12),
    "long_split": (configs.LONG_CONTEXT.scaled(batch=4), 3000, 24),
    "generic": (configs.TINY.scaled(batch=3), 700, 20),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_step_equals_append_then_decode(case):
    w, n0, steps = CASES[case]
    cap = n0 + steps
    k, v = gen.kv_tensors(w, 0, cap, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.cuda(), tinvt.cuda()
    a = W.KVCache(spec_of(w, capacity=cap), "cuda")
    b = W.KVCache(spec_of(w, capacity=cap), "cuda")
    for c in (a, b):
        W.append_flush(c, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous(), t16)
    P = W.decode_num_splits(a, cap, w.num_q_heads, 0)
    if case == "serving_whole":
        assert P == 12 and W.decode_num_splits(a, n0 + 1, w.num_q_heads, 0) == 12, P
    for s in range(steps):
        ks, vs = k[:, :, n0 + s:n0 + s + 1].contiguous(), v[:, :, n0 + s:n0 + s + 1].contiguous()
        q = gen.queries(w, 0, s, "cuda")
        W.append_flush(a, ks, vs, t16)
        oa, qa = W.decode_attention_fused(a, q, tinvt, num_splits=P)
        ob, qb = W.decode_step(b, ks, vs, t16, q, tinvt, num_splits=P)
        torch.cuda.synchronize()
        assert torch.equal(qa, qb), (case, s)
        assert torch.equal(oa, ob), (case, s, float((oa - ob).abs().max()))
    for p in W.PLANES:
        assert torch.equal(a.planes[p], b.planes[p]), (case, p)
    say(f"[decode step {case}] {w.name}: {n0} -> {n0 + steps} tokens, {P} splits: equal to append + decode")


def test_decode_step_full_serving_shape_vs_oracle():
    """wushkv_decode_step at the batched-serving shape the benchmark times (32 sequences
    of 32768 tokens, 32 query / 8 KV heads, affine 2-bit K and V, chunk 16): the library's
    12 splits, so every step is one 12-wave workgroup per KV head with the new token's
    append fused into the decode (and the flush kernel when a chunk is due).  18 steps
    cross one flush; the outputs at the first, flush and last steps, and the cache after
    the last, are held to the oracle on sampled (batch row, KV head) pairs."""
    w = configs.SERVING
    steps = 18
    r = Run(w, n_total=w.context + steps)
    r.append(w.context)
    n0 = r.cache.n
    P = W.decode_num_splits(r.cache, n0 + 1, w.num_q_heads, 0)
    say(f"[decode step c2 full] B={w.batch} n={n0} -> {n0 + steps}, {P} splits, "
        f"{w.batch * w.num_kv_heads} KV heads: the 12-wave layout with the append fused")
    assert P == 12
    heads = [(0, 0), (13, 5), (31, 7)]
    q_of = lambda n: w.chunk * (max(0, n - w.sink - w.recent) // w.chunk)
    flush_steps = [s for s in range(steps) if q_of(n0 + s + 1) > q_of(n0 + s)]
    assert flush_steps, "the steps must cross a flush"
    check_at = sorted({0, flush_steps[0], steps - 1})
    for s in range(steps):
        n = r.cache.n
        ks, vs = r.k[:, :, n:n + 1].contiguous(), r.v[:, :, n:n + 1].contiguous()
        q = gen.queries(w, 0, s, "cuda")
        out, qt = W.decode_step(r.cache, ks, vs, r.t16, q, r.tinvt, num_splits=P)
        torch.cuda.synchronize()
        if s in check_at:
            pa = plane_arrays(r.cache)
            check_decode_lengths(pa, r.spec, w, r.k, r.v, r.t16_cpu, [r.cache.n] * w.batch, q, qt, out, heads=heads,
                                 what=f"decode step c2 full, step {s} (n={r.cache.n})")
    _, stats = r.check_cache(heads)
    say(f"[decode step c2 full] cache after {steps} steps (flushes at steps {flush_steps}): {stats}")
