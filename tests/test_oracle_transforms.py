"""Pins of the module-output-error metric (oracle) and of the key-transform inputs
(synth/transforms.py), CPU only.

* attention_fp equals torch's scaled_dot_product_attention in float64 (a library
  routine) and, for a zero query, the mean of the values (a closed form).
* module_output_error and geometric_mean against closed forms.
* hadamard(d) is orthonormal with entries +-1/sqrt(d) and equals scipy's Sylvester
  Hadamard matrix / sqrt(d); whitening() whitens the second moment it was built from,
  up to the stated scale, and keeps the identity's Frobenius norm.
* as_inputs: q~ . (T16 k) equals q . k for every transform.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import wushkv_ref as R
from synth import transforms as TR


def test_attention_fp_matches_sdpa():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 64))
    k = rng.standard_normal((40, 64)) * 3.0
    v = rng.standard_normal((40, 64))
    got = R.attention_fp(q, k, v)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_fp_zero_query_is_the_value_mean():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((17, 8))
    out = R.attention_fp(np.zeros((1, 8)), rng.standard_normal((17, 8)), v)
    assert np.allclose(out[0], v.mean(axis=0), rtol=1e-13, atol=1e-13)


def test_module_error_and_geometric_mean_closed_forms():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((3, 4, 8))
    assert R.module_output_error(ref, ref) == 0.0
    assert R.module_output_error(ref * 1.25, ref) == pytest.approx(0.25, rel=1e-13)
    d = rng.standard_normal(ref.shape)
    assert R.module_output_error(ref + d, ref) == pytest.approx(np.sqrt((d ** 2).sum() / (ref ** 2).sum()), rel=1e-13)
    assert R.geometric_mean([0.5, 0.125]) == pytest.approx(0.25, rel=1e-13)
    assert R.geometric_mean([0.3] * 7) == pytest.approx(0.3, rel=1e-13)


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_is_sylvester_and_orthonormal(d):
    h = TR.hadamard(d)
    assert np.allclose(h @ h.T, np.eye(d), atol=1e-13)
    assert np.allclose(np.abs(h), 1.0 / np.sqrt(d))
    assert np.array_equal(h * np.sqrt(d), scipy.linalg.hadamard(d).astype(np.float64))
    with pytest.raises(ValueError):
        TR.hadamard(d * 3 if d > 1 else 3)


def test_whitening_whitens_and_keeps_the_frobenius_norm():
    rng = np.random.default_rng(6)
    d, n = 16, 4000
    a = rng.standard_normal((d, d)) * (2.0 ** rng.uniform(-3, 3, d))[None, :]
    x = rng.standard_normal((n, d)) @ a.T
    gram = x.T @ x
    t = TR.whitening(gram, n)
    sigma = gram / n
    # T = c sigma^{-1/2} with c^2 = d / trace(sigma^{-1}): T sigma T^T = c^2 I
    c2 = d / np.trace(np.linalg.inv(sigma))
    assert np.allclose(t @ sigma @ t.T, c2 * np.eye(d), rtol=1e-9, atol=1e-9 * c2)
    assert np.linalg.norm(t) == pytest.approx(np.sqrt(d), rel=1e-12)
    assert np.allclose(t, t.T, atol=1e-12)
    # a diagonal second moment gives a diagonal transform, 1 / sqrt(sigma_i) up to c
    s = np.array([4.0, 1.0, 0.25, 9.0])
    td = TR.whitening(np.diag(s) * 10, 10)
    want = np.diag(1 / np.sqrt(s))
    assert np.allclose(td, want * (2.0 / np.linalg.norm(want)), atol=1e-13)


@pytest.mark.parametrize("kind", ["identity", "hadamard", "whitening"])
def test_as_inputs_preserves_scores(kind):
    rng = np.random.default_rng(7)
    d = 64
    if kind == "identity":
        t = np.eye(d)
    elif kind == "hadamard":
        t = TR.hadamard(d)
    else:
        x = rng.standard_normal((500, d)) * (2.0 ** rng.uniform(-2, 2, d))[None, :]
        t = TR.whitening(x.T @ x, 500)
    t16, tinvt = TR.as_inputs(TR.per_head(t, 2))
    assert t16.shape == (2, d, d) and tinvt.shape == (2, d, d)
    k = rng.standard_normal(d)
    q = rng.standard_normal(d)
    for g in range(2):
        kt = t16[g].double().numpy() @ k
        qt = tinvt[g].double().numpy() @ q
        assert qt @ kt == pytest.approx(q @ k, rel=1e-6, abs=1e-6)
