"""wushkv_decode_attention_noalloc (the decode with its split-K partials in the library's
own fixed device array) against wushkv_decode_attention with a caller workspace, through
the C ABI: the outputs must be equal bit for bit (same kernels, same partial layout), on
two calls in a row whose second has a smaller input, plus a third on the plain fp32
kernel's shape.  A decode needing more partials than the array holds is rejected before
anything is enqueued."""
import ctypes

import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from tests.parity_util import Run, say

pytestmark = pytest.mark.gpu


def _both(r, n_splits):
    w = r.w
    q = gen.queries(w, 0, 0, "cuda")
    qt = W.query_transform(r.tinvt, q, w.num_kv_heads)
    P = W.decode_num_splits(r.cache, r.cache.n, w.num_q_heads, n_splits)
    need = W.lib().wushkv_decode_workspace_bytes(ctypes.byref(r.cache.desc), r.cache.n, w.num_q_heads, n_splits)
    ref = W.decode_attention(r.cache, q, qt, num_splits=n_splits)
    out = torch.full_like(ref, float("nan"))
    W.decode_attention_noalloc(r.cache, q, qt, num_splits=n_splits, out=out)
    torch.cuda.synchronize()
    say(f"[noalloc] {w.name} B={w.batch} Hq={w.num_q_heads} n={r.cache.n} splits={P} partials {need} bytes: "
        f"equal {torch.equal(ref, out)}")
    assert need <= W.NOALLOC_SCRATCH_BYTES
    assert torch.equal(ref, out)
    return need


def test_noalloc_equals_workspace_decode_on_consecutive_calls():
    # 1: the 8B-class layer at 8192 tokens: 64 partitions of the matrix-core decode and the
    #    merge kernel, all through the array
    w1 = configs.LAYER_8B.scaled(name="noalloc1", seed=51)
    r1 = Run(w1, n_total=w1.context + 1)
    r1.append(w1.context + 1)
    big = _both(r1, 0)
    # 2: a smaller input on the same array: a shorter context, fewer sequences' worth of
    #    partials, a split count of its own
    w2 = configs.LONG_CONTEXT.scaled(name="noalloc2", seed=52, batch=1, context=3000)
    r2 = Run(w2, n_total=w2.context + 1)
    r2.append(w2.context + 1)
    small = _both(r2, 17)
    assert small < big
    # 3: the plain fp32 kernel's shape (head_dim 64), smaller still
    w3 = configs.TINY.scaled(name="noalloc3", seed=53)
    r3 = Run(w3, n_total=700)
    r3.append(700)
    _both(r3, 5)


def test_noalloc_rejects_partials_beyond_the_array():
    w = configs.LONG_CONTEXT.scaled(name="noalloc_big", seed=54, batch=64, context=1000)
    spec = W.CacheSpec(batch=w.batch, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, capacity=w.context,
                       sink=w.sink, recent=w.recent, chunk=w.chunk, bits_k=2, bits_v=3, quant_k=W.Q_AFFINE,
                       quant_v=W.Q_AFFINE)
    cache = W.KVCache(spec, "cuda")
    cache.n = w.context
    need = W.lib().wushkv_decode_workspace_bytes(ctypes.byref(cache.desc), cache.n, w.num_q_heads, 128)
    assert need > W.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    qt = torch.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    out = torch.full_like(qt, 7.0)
    with pytest.raises(W.WushKVError) as e:
        W.decode_attention_noalloc(cache, q, qt, num_splits=128, out=out)
    assert e.value.status == W.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())          # nothing was enqueued
