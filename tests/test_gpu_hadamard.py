"""The fixed Hadamard key transform formed in registers (wushkv_append_flush_hadamard, a fast
Walsh-Hadamard transform instead of the d x d product) against the oracle's key transform
with T_K = fp16(H / sqrt(d)) (digest, "motivation" / "key experiments": Hadamard is the
fixed-transform baseline), and against the dense path given that same fp16 matrix: both
decide codes near a boundary and parameters near an fp16 midpoint from the exact x, so the
two caches agree bit for bit."""
import numpy as np
import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from synth import transforms as TR
from tests.parity_util import Run, say, spec_of

pytestmark = pytest.mark.gpu

CASES = {
    # name: workload (K/V distributions of the 8B layer or the serving shape)
    "quest2_d128_bf16": configs.LAYER_8B.scaled(name="had_q2", seed=61, context=3000, decode_steps=12),
    "affine2_d128_bf16": configs.SERVING.scaled(name="had_a2", seed=62, batch=2, context=2500, decode_steps=12),
    "quest4_d64_f32": configs.TINY.scaled(name="had_q4", seed=63, batch=2, num_kv_heads=2, num_q_heads=8, context=1500,
                                          decode_steps=12, bits_k=4, bits_v=3),
    "affine3_d128_f16in": configs.LONG_CONTEXT.scaled(name="had_a3", seed=64, batch=1, context=2000, decode_steps=12,
                                                      bits_k=3, bits_v=3, in_dtype="f16"),
}


def _hadamard_inputs(w):
    t16, tinvt = TR.as_inputs(TR.per_head(TR.hadamard(w.head_dim), w.num_kv_heads))
    scale = float(np.float16(1.0 / np.sqrt(w.head_dim)))
    assert np.all(np.abs(t16.numpy().astype(np.float64)) == scale)
    return t16, tinvt, scale


@pytest.mark.parametrize("case", sorted(CASES))
def test_hadamard_transform_matches_oracle_and_dense(case):
    w = CASES[case]
    t16, tinvt, scale = _hadamard_inputs(w)
    r = Run(w)                                   # the oracle side uses r.t16_cpu
    r.t16_cpu, r.t16, r.tinvt = t16, t16.cuda(), tinvt.cuda()
    dense = W.KVCache(spec_of(w, capacity=r.n_total), "cuda")
    n0 = w.context
    say(f"[hadamard {case}] prefill {n0}, {w.decode_steps} steps, scale {scale}")
    W.append_flush_hadamard(r.cache, r.k[:, :, :n0].contiguous(), r.v[:, :, :n0].contiguous(), scale)
    W.append_flush(dense, r.k[:, :, :n0].contiguous(), r.v[:, :, :n0].contiguous(), r.t16)
    _, stats = r.check_cache()
    say(f"[hadamard {case}] prefill vs oracle {stats}")
    for s in range(w.decode_steps):
        n = r.cache.n
        ks, vs = r.k[:, :, n:n + 1].contiguous(), r.v[:, :, n:n + 1].contiguous()
        W.append_flush_hadamard(r.cache, ks, vs, scale)
        W.append_flush(dense, ks, vs, r.t16)
    torch.cuda.synchronize()
    _, stats = r.check_cache()
    say(f"[hadamard {case}] after steps vs oracle {stats}")
    for p in W.PLANES:
        assert torch.equal(r.cache.planes[p], dense.planes[p]), p
    q, qt, out = r.decode(0)
    r.check_decode(q, qt, out)
