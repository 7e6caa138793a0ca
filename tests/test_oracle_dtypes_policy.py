"""Pins of the oracle's dtype helpers and cache policy (CPU only).

dtype helpers are checked against torch's own casts (a library routine); the
closed-form count of quantized tokens and the ring placement are checked
against a token-by-token simulation of the window policy (brute force)."""
import numpy as np
import pytest
import torch

from oracle import wushkv_ref as R


def _special_values():
    f16max = 65504.0
    vals = [0.0, -0.0, 1.0, -1.0, f16max, -f16max, 65519.99, 65520.0, 6.103515625e-05,
            5.960464477539063e-08, 2.9802322387695312e-08, 2.98023224e-08 * 1.5, 1e-9]
    # exact fp16 midpoints (ties) between consecutive fp16 values, both parities
    h = np.arange(0x3C00, 0x3C40, dtype=np.uint16).view(np.float16).astype(np.float64)
    vals += list((h[:-1] + h[1:]) / 2)
    return np.array(vals + [-v for v in vals])


def test_f16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(400_000) * 10.0 ** rng.uniform(-9, 4.8, 400_000),
        rng.uniform(-65504, 65504, 300_000),
        rng.standard_normal(300_000) * 1e-6,
        _special_values(),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).double().numpy()
    got = R.f16(x)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.array_equal(got, ref)


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(500_000) * 10.0 ** rng.uniform(-30, 30, 500_000),
        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.3895314e38], dtype=np.float64),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(R.bf16(x), ref)


def _simulate(n_total, sink, recent, chunk):
    """Append tokens one at a time: the first `sink` stay, the rest enter a
    ring of recent+chunk rows; when the ring is full its oldest `chunk`
    tokens are flushed.  Returns, after every append, (body count, ring
    token positions, slot of each ring token)."""
    body = 0
    ring = []  # positions, oldest first
    slots = {}
    next_slot = 0
    hist = []
    for p in range(n_total):
        if p >= sink:
            ring.append(p)
            slots[p] = next_slot
            next_slot = (next_slot + 1) % (recent + chunk)
            if len(ring) == recent + chunk:
                flushed, ring = ring[:chunk], ring[chunk:]
                assert flushed == list(range(sink + body, sink + body + chunk))
                body += chunk
        hist.append((body, list(ring), dict((q, slots[q]) for q in ring)))
    return hist


@pytest.mark.parametrize("sink,recent,chunk", [(64, 256, 8), (64, 256, 16), (0, 16, 4), (5, 7, 3), (5, 6, 3), (3, 0, 2), (0, 0, 1)])
def test_policy_matches_token_by_token_simulation(sink, recent, chunk):
    hist = _simulate(3000, sink, recent, chunk)
    for n in range(0, 3001):
        body, ring, slots = hist[n - 1] if n > 0 else (0, [], {})
        assert R.n_quantized(n, sink, recent, chunk) == body
        for p in range(n):
            want = "sink" if p < sink else ("body" if p < sink + body else "recent")
            if p < sink or n < 40 or p in (sink + body - 1, sink + body, n - 1):
                assert R.region(p, n, sink, recent, chunk) == want
        for p, s in slots.items():
            assert R.ring_slot(p, sink, recent, chunk) == s
        # live ring tokens occupy distinct slots and a flushed chunk never wraps
        assert len(set(slots.values())) == len(slots)
        if body and recent % chunk == 0:
            first = R.ring_slot(sink + body - chunk, sink, recent, chunk)
            assert first + chunk <= recent + chunk


def test_windows_hold_exact_fp16_values():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((700, 16)).astype(np.float32) * 3
    v = rng.standard_normal((700, 16)).astype(np.float32)
    t = np.eye(16, dtype=np.float16)
    for n in (1, 30, 64, 65, 319, 320, 328, 329, 700):
        c = R.build_head_cache(k, v, t, n, sink=64, recent=256, chunk=8,
                               quant_k="quest", quant_v="affine", bits_k=2, bits_v=3)
        ns, nb = c.sink_n, c.body_n
        assert ns == min(n, 64) and nb == R.n_quantized(n, 64, 256, 8)
        assert np.array_equal(c.sink_k, k[:ns].astype(np.float16).astype(np.float64))
        assert np.array_equal(c.sink_v, v[:ns].astype(np.float16).astype(np.float64))
        assert np.array_equal(c.recent_k, k[64 + nb:n].astype(np.float16).astype(np.float64))
        assert np.array_equal(c.recent_v, v[64 + nb:n].astype(np.float16).astype(np.float64))
        assert ns + nb + len(c.recent_k) == n
