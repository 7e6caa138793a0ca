"""GPU parity of the calibration sums (wushkv_calib_stats) against the oracle's
float64 calib_stats.

Tolerance, from the arithmetic: every product of two bf16/f16 inputs is exact in fp32,
and an output element is a chain of fp32 additions -- a workgroup's run of rows (bpw
batch rows x the group's heads x T tokens, T rounded up to 64) on the matrix cores, then
the group's nparts partials in a fixed order.  Recursive fp32 summation of m terms errs
by at most (m - 1) u sum|terms| (u = 2^-24), so with m = bpw * group * T64 + nparts the
test allows 2 m u sum|x_i x_j| per element (the factor 2 leaves room for a truncating
adder).  nparts (one per batch block) and bpw follow from the workspace size the library
asks for."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_amd as W
from oracle import wushkv_ref as R
from synth import configs, gen
from tests.parity_util import say

pytestmark = pytest.mark.gpu


def _chain(B, H, T, group):
    nb = W.lib().wushkv_calib_workspace_bytes(B, H, T, 128, group) // (10 * 1024 * 4) // (H // group)
    bpw = math.ceil(B / nb)
    return bpw * group * 64 * math.ceil(T / 64) + nb


def _compare(got, xs, group, chain, label):
    """got: the GPU sums of the groups whose rows xs [B, k * group, T, d] (CPU) holds."""
    want = R.calib_stats(xs, group)
    bound = 2.0 * chain * 2.0 ** -24 * R.calib_sum_abs(xs, group)
    err = np.abs(got - want)
    worst = float((err / np.maximum(bound, 1e-30)).max())
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    say(f"[calib {label}] rows {xs.shape}, group {group}: rel Frobenius {rel:.2e}, worst error / bound {worst:.3f}")
    assert np.all(err <= bound), f"{label}: error exceeds the fp32 summation bound"
    for g in range(got.shape[0]):
        assert np.array_equal(got[g], got[g].T)


def _check(x, group, label):
    B, H, T, d = x.shape
    out = W.calib_stats(x, group)
    torch.cuda.synchronize()
    _compare(out.double().cpu().numpy(), x.float().cpu().numpy(), group, _chain(B, H, T, group),
             f"{label} {x.dtype}")


def _rows(B, H, T, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    scale = torch.exp(torch.randn(128, generator=g, device="cuda") * 1.5)
    x = torch.randn(B, H, T, 128, generator=g, device="cuda") * scale
    x[..., 5] *= 20.0                                # an outlier channel
    return x.to(dtype)


@pytest.mark.parametrize("B,H,T,group,dtype", [
    (1, 1, 64, 1, torch.bfloat16),      # one LDS step, one workgroup
    (1, 1, 1, 1, torch.bfloat16),       # a single row: x x^T
    (3, 8, 200, 4, torch.bfloat16),     # ragged tail, query-head groups
    (2, 6, 129, 3, torch.float16),      # fp16 input
    (5, 4, 1000, 2, torch.bfloat16),
    (40, 2, 70, 1, torch.bfloat16),     # several batch rows per workgroup
])
def test_calib_matches_oracle(B, H, T, group, dtype):
    _check(_rows(B, H, T, dtype, 1000 + B * 31 + T), group, f"random seed {1000 + B * 31 + T}")


def test_calib_deterministic_and_workspace_reuse():
    x = _rows(3, 8, 300, torch.bfloat16, 77)
    ws = W.calib_workspace(3, 8, 300, 128, 4)
    a = W.calib_stats(x, 4, workspace=ws).clone()
    W.calib_stats(_rows(2, 4, 50, torch.bfloat16, 78), 2, workspace=ws)   # smaller call in between
    b = W.calib_stats(x, 4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_calib_workload_full_size_sampled():
    """The calibration workload (128 sequences x 1024 tokens, 8 KV / 32 query heads): every
    group computed on the GPU in one call per statistic, two groups of each checked."""
    w = configs.CALIB
    T = w.context
    k, v = gen.kv_tensors(w, 0, T, "cuda")
    for name, x in (("keys", k), ("values", v)):
        out = W.calib_stats(x, 1)
        torch.cuda.synchronize()
        chain = _chain(w.batch, w.num_kv_heads, T, 1)
        for g in (0, 5):
            _compare(out[g:g + 1].double().cpu().numpy(), x[:, g:g + 1].float().cpu().numpy(), 1, chain,
                     f"{w.name} {name} head {g}")
    del k, v
    q = gen.calib_queries(w, 0, T, "cuda")
    out = W.calib_stats(q, w.group)
    torch.cuda.synchronize()
    chain = _chain(w.batch, w.num_q_heads, T, w.group)
    for g in (0, 7):
        xs = q[:, g * w.group:(g + 1) * w.group].float().cpu().numpy()
        _compare(out[g:g + 1].double().cpu().numpy(), xs, w.group, chain, f"{w.name} queries group {g}")
