"""Fixed and data-adaptive key transforms through the GPU path, and the module-output
error they give, against the oracle.

T_K is an input of the path, so a fixed transform (identity, orthonormal Hadamard) or
a data-adaptive one (Gram whitening, built here from the library's own calibration sums
over held-out keys of the same heads) runs through the same kernels as any other.  For
each, two synthetic attention modules are prefilled on the GPU and decoded for several
queries; the decode is held to the oracle on the device's own cache (1e-4 relative L2),
and the module-output error computed from the GPU's outputs (relative Frobenius error
against full-precision attention over the unquantized keys and values) to the oracle's
own figure for the same module."""
import numpy as np
import pytest
import torch

import bit_kv_cache_amd as W
from oracle import wushkv_ref as R
from synth import configs, gen
from synth import transforms as TR
from tests.parity_util import device_head_cache, plane_arrays, rel_l2, say, spec_of

pytestmark = pytest.mark.gpu

N_TOKENS = 700
N_QUERIES = 4


def _transform(kind, w, layer):
    d, H = w.head_dim, w.num_kv_heads
    if kind == "identity":
        return TR.as_inputs(TR.per_head(np.eye(d), H))
    if kind == "hadamard":
        return TR.as_inputs(TR.per_head(TR.hadamard(d), H))
    if kind == "dense":
        return gen.key_transforms(w, layer)
    # whitening from the calibration sums of held-out rows (batch rows B .. 2B - 1)
    held = torch.stack([torch.stack([gen.kv_block(w, layer, w.batch + b, g, N_TOKENS, "cuda")[0]
                                     for g in range(H)]) for b in range(w.batch)])
    gram = W.calib_stats(held.contiguous(), 1).double().cpu().numpy()
    count = w.batch * N_TOKENS
    return TR.as_inputs(np.stack([TR.whitening(gram[g], count) for g in range(H)]))


@pytest.mark.parametrize("kind", ["identity", "hadamard", "dense", "whitening"])
@pytest.mark.parametrize("quant", ["affine", "quest"])
def test_transform_module_error_matches_oracle(kind, quant):
    base = configs.SERVING.scaled(batch=2, context=N_TOKENS)
    w = base if quant == "affine" else base.scaled(quant_k=configs.QUEST, quant_v=configs.QUEST)
    G, d = w.group, w.head_dim
    errs_gpu, errs_or = [], []
    for layer in range(2):
        t16, tinvt = _transform(kind, w, layer)
        k, v = gen.kv_tensors(w, layer, N_TOKENS, "cuda")
        cache = W.KVCache(spec_of(w, capacity=N_TOKENS), "cuda")
        W.append_flush(cache, k, v, t16.cuda())
        qs = [gen.queries(w, layer, s, "cuda") for s in range(N_QUERIES)]
        outs, qts = [], []
        for q in qs:
            o, qt = W.decode_attention_fused(cache, q, tinvt.cuda())
            outs.append(o)
            qts.append(qt)
        torch.cuda.synchronize()
        pa = plane_arrays(cache)
        got, dev_ref, or_out, fp_out = [], [], [], []
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                kk = k[b, g].float().cpu().numpy().astype(np.float64)
                vv = v[b, g].float().cpu().numpy().astype(np.float64)
                c_dev = device_head_cache(pa, cache.spec, b, g, N_TOKENS)
                c_or = R.build_head_cache(kk, vv, t16[g].numpy(), N_TOKENS, sink=w.sink, recent=w.recent,
                                          chunk=w.chunk, quant_k=w.quant_k, quant_v=w.quant_v, bits_k=w.bits_k,
                                          bits_v=w.bits_v, clip_mult=w.clip_mult, pct_lo=w.pct_lo,
                                          pct_hi=w.pct_hi)
                for s, q in enumerate(qs):
                    qn = q[b, g * G:(g + 1) * G].float().cpu().numpy().astype(np.float64)
                    qtn = qts[s][b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
                    fp_out.append(R.attention_fp(qn, kk, vv))
                    for hh in range(G):
                        got.append(outs[s][b, g * G + hh].cpu().numpy())
                        dev_ref.append(R.decode_head(c_dev, qn[hh], qtn[hh]))
                        or_out.append(R.decode_head(c_or, qn[hh], R.query_transform(t16[g].numpy(), qn[hh])))
        dev = rel_l2(got, dev_ref)
        assert dev <= 1e-4, (kind, quant, layer, dev)
        fp = np.concatenate(fp_out)
        errs_gpu.append(R.module_output_error(np.stack(got), fp))
        errs_or.append(R.module_output_error(np.stack(or_out), fp))
    gm_gpu, gm_or = R.geometric_mean(errs_gpu), R.geometric_mean(errs_or)
    say(f"[transform {kind:9s} {quant}] module-output error: GPU {gm_gpu:.4f}, oracle {gm_or:.4f}")
    assert abs(gm_gpu - gm_or) <= 5e-3 * max(gm_or, 1e-3) + 2e-4, (gm_gpu, gm_or)
