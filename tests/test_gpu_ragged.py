"""GPU parity of ragged batches (every sequence its own token count) against the oracle,
which builds each (batch row, KV head) cache from that sequence's own tokens.

Sequences are prefilled one by one through one-sequence views of the batch's cache,
then stepped together: each step appends one token to every sequence
(wushkv_append_flush_ragged) and decodes every sequence over its own length
(wushkv_decode_attention_ragged).  The lengths cover a single token, a partial sink,
exactly full windows (no body yet), the first flush, and a body of many sets with a
ragged tail; the 20 steps take the short ones across flush boundaries at different
steps."""
import numpy as np
import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from tests.parity_util import check_decode_lengths, check_head, plane_arrays, say, spec_of

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 320, 335, 1000, 2501]
STEPS = 20


def _setup(w, lengths, steps):
    cap = max(lengths) + steps
    k, v = gen.kv_tensors(w, 0, cap, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    cache = W.KVCache(spec_of(w, capacity=cap), "cuda")
    for b, n in enumerate(lengths):
        seq = cache.sequence(b)
        W.append_flush(seq, k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(), t16.cuda(), n_before=0)
    cache.seq_n = list(lengths)
    return cache, k, v, t16, tinvt


def _check_cache(cache, w, k, v, t16):
    torch.cuda.synchronize()
    pa = plane_arrays(cache)
    stats = {}
    for b, n in enumerate(cache.seq_n):
        for g in range(w.num_kv_heads):
            check_head(pa, cache.spec, b, g, k[b, g].float().cpu().numpy().astype(np.float64),
                       v[b, g].float().cpu().numpy().astype(np.float64), t16[g].numpy(), n, stats)
    if stats.get("code_total"):
        assert stats["code_mism"] <= 1e-5 * stats["code_total"], stats
    return pa, stats


def _check_decode(cache, w, k, v, t16, q, qt, out):
    """The decode against the oracle: end to end (the oracle's own cache built from each
    sequence's tokens, its exact q~) within 2e-3, and on the device's own cache with the
    device's q~ (the decode kernel alone) within 1e-4; with the cache's parameters
    bit-exact, the two agree."""
    return check_decode_lengths(plane_arrays(cache), cache.spec, w, k, v, t16, cache.seq_n, q, qt, out,
                                what=f"ragged {w.name} lengths {cache.seq_n}")


@pytest.mark.parametrize("wl", ["serving", "long"])
def test_ragged_prefill_steps_and_decode(wl):
    base = configs.SERVING if wl == "serving" else configs.LONG_CONTEXT
    w = base.scaled(batch=len(LENGTHS))
    cache, k, v, t16, tinvt = _setup(w, LENGTHS, STEPS)
    say(f"[ragged {w.name}] prefilled {LENGTHS}")
    _, stats = _check_cache(cache, w, k, v, t16)
    say(f"[ragged {w.name}] prefill cache parity {stats}")
    for step in range(STEPS):
        ks = torch.stack([k[b, :, n:n + 1] for b, n in enumerate(cache.seq_n)]).contiguous()
        vs = torch.stack([v[b, :, n:n + 1] for b, n in enumerate(cache.seq_n)]).contiguous()
        W.append_flush_ragged(cache, ks, vs, t16.cuda())
        q = gen.queries(w, 0, step, "cuda")
        if step % 2:
            out, qt = W.decode_attention_ragged(cache, q, t_inv_t=tinvt.cuda())
        else:
            qt = W.query_transform(tinvt.cuda(), q, w.num_kv_heads)
            out, _ = W.decode_attention_ragged(cache, q, q_t=qt)
        torch.cuda.synchronize()
        _check_decode(cache, w, k, v, t16, q, qt, out)
    _, stats = _check_cache(cache, w, k, v, t16)
    say(f"[ragged {w.name}] after {STEPS} steps: lengths {cache.seq_n}, cache parity {stats}")


def test_ragged_equal_lengths_is_the_uniform_path():
    """A ragged batch whose sequences all hold the same count gives the uniform path's
    cache and output bit for bit."""
    w = configs.SERVING.scaled(batch=3, context=1500)
    n0 = 1400
    k, v = gen.kv_tensors(w, 0, n0 + 40, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.cuda(), tinvt.cuda()
    a = W.KVCache(spec_of(w, capacity=n0 + 40), "cuda")
    b = W.KVCache(spec_of(w, capacity=n0 + 40), "cuda")
    W.append_flush(a, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous(), t16)
    W.append_flush(b, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous(), t16)
    b.seq_n = [n0] * 3
    for step in range(40):
        ks, vs = k[:, :, n0 + step:n0 + step + 1].contiguous(), v[:, :, n0 + step:n0 + step + 1].contiguous()
        W.append_flush(a, ks, vs, t16)
        W.append_flush_ragged(b, ks, vs, t16)
    q = gen.queries(w, 0, 0, "cuda")
    oa, qa = W.decode_attention_fused(a, q, tinvt)
    ob, qb = W.decode_attention_ragged(b, q, t_inv_t=tinvt)
    torch.cuda.synchronize()
    for p in W.PLANES:
        assert torch.equal(a.planes[p], b.planes[p]), p
    assert torch.equal(qa, qb) and torch.equal(oa, ob)
