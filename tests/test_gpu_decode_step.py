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
from tests.parity_util import say, spec_of

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, prefill tokens, steps)
    "serving_whole": (configs.SERVING.scaled(batch=32), 1500, 40),
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
