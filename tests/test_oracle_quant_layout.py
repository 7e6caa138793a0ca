"""Pins of the oracle's quantizers, transforms and code layout (CPU only).

Pins used: hand-worked examples (tests/golden/*.txt), brute-force nearest
level search, the Gaussian MSE integral by quadrature, numpy.percentile,
numpy.linalg.inv, and invariants (code range, half-bin error bound)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import layout as LY
from oracle import wushkv_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _nums(s):
    return [float(t) for t in s.split()]


def _golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            parts = [p.strip() for p in line.split("|")]
            rows.setdefault(parts[0], []).append(parts[1:])
    return rows


# --------------------------------------------------------------------------- worked examples

def test_quest_worked_example():
    (row,) = _golden("quant_worked.txt")["quest2"]
    x = np.array(_nums(row[0]))
    step = float(row[1].split()[1])
    codes = [int(v) for v in row[2].split()[1:]]
    deq = _nums(row[3].split(" ", 1)[1])
    st = R.quest_params(x, 2, 2.5)
    assert st == step
    assert R.quest_codes(x[None], np.array([st]), 2)[0].tolist() == codes
    assert R.quest_dequant(np.array([codes]), np.array([st]), 2)[0].tolist() == deq


def test_affine_worked_example():
    (row,) = _golden("quant_worked.txt")["affine2"]
    x = np.array(_nums(row[0]))
    sc, zr = float(row[1].split()[1]), float(row[1].split()[3])
    codes = [int(v) for v in row[2].split()[1:]]
    deq = _nums(row[3].split(" ", 1)[1])
    s, z = R.affine_params(x, 2, 10.0, 90.0)
    assert (s, z) == (sc, zr)
    assert R.affine_codes(x[None], np.array([s]), np.array([z]), 2)[0].tolist() == codes
    assert R.affine_dequant(np.array([codes]), np.array([s]), np.array([z]))[0].tolist() == deq


def test_transform_worked_example_orientation():
    (row,) = _golden("quant_worked.txt")["transform"]
    t = np.array([float(v) for v in row[0].split()[1:]]).reshape(2, 2)
    k = np.array([float(v) for v in row[1].split()[1:]])
    tk = [float(v) for v in row[2].split()[1:]]
    q = np.array([float(v) for v in row[3].split()[1:]])
    qt = [float(v) for v in row[4].split()[1:]]
    assert R.key_transform(t.astype(np.float16), k[None])[0].tolist() == tk
    assert np.allclose(R.query_transform(t.astype(np.float16), q[None])[0], qt, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- QuEST

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quest_invariants_and_brute_force(bits):
    rng = np.random.default_rng(bits)
    L = 2 ** bits
    x = rng.standard_normal((4000, 128)) * rng.uniform(0.01, 50, (4000, 1))
    x[:50] = rng.standard_t(3, (50, 128)) * 10
    st = R.quest_params(x, bits, 2.5)
    codes = R.quest_codes(x, st, bits)
    assert codes.min() >= 0 and codes.max() <= L - 1
    xh = R.quest_dequant(codes, st, bits)
    inside = np.abs(x) <= st[:, None] * L / 2
    assert np.all(np.abs(x - xh)[inside] <= st[:, None].repeat(128, 1)[inside] / 2 * (1 + 1e-12))
    # brute force: nearest of the L reconstruction levels (ties excluded)
    levels = (np.arange(L) - (L - 1) / 2)[None, None, :] * st[:, None, None]
    dist = np.abs(x[..., None] - levels)
    srt = np.sort(dist, axis=-1)
    untied = srt[..., 1] - srt[..., 0] > 1e-9 * st[:, None]
    assert np.array_equal(np.argmin(dist, axis=-1)[untied], codes[untied])


def test_quest_rms_scaling_and_degenerate_rows():
    a = 0.7
    x = np.array([[a, -a] * 32])
    st = R.quest_params(x, 2, 2.5)
    assert st[0] == R.f16(2 * 2.5 * a / 4)
    z = np.zeros((1, 64))
    st0 = R.quest_params(z, 3, 2.5)
    assert st0[0] == 0.0
    assert R.quest_codes(z, st0, 3).tolist() == [[4] * 64]
    assert np.all(R.quest_dequant(R.quest_codes(z, st0, 3), st0, 3) == 0.0)
    # a row so small its step underflows fp16 behaves like the zero row
    tiny = np.full((1, 64), 1e-9)
    st1 = R.quest_params(tiny, 2, 2.5)
    assert st1[0] == 0.0 and R.quest_codes(tiny, st1, 2).tolist() == [[2] * 64]


@pytest.mark.parametrize("bits,expected", [(2, 0.1403), (3, 0.0382), (4, 0.0120)])
def test_quest_gaussian_mse_matches_quadrature(bits, expected):
    """With a fixed step 2*2.5*sigma/L on N(0, sigma^2), the mean squared
    reconstruction error equals the integral over the bins of (x - centre)^2
    weighted by the Gaussian density."""
    L = 2 ** bits
    sigma = 1.0
    step = 2 * 2.5 * sigma / L
    edges = [-np.inf] + [(k - L / 2) * step for k in range(1, L)] + [np.inf]
    centres = [(q - (L - 1) / 2) * step for q in range(L)]
    mse_quad = sum(integrate.quad(lambda t, c=c: (t - c) ** 2 * stats.norm.pdf(t), a, b, epsabs=1e-13)[0]
                   for a, b, c in zip(edges[:-1], edges[1:], centres))
    # integrate the oracle's quantizer itself on a fine grid
    t = np.linspace(-12, 12, 2_400_001)
    codes = R.quest_codes(t[None], np.array([step]), bits)[0]
    err2 = (t - R.quest_dequant(codes[None], np.array([step]), bits)[0]) ** 2
    mse_grid = integrate.trapezoid(err2 * stats.norm.pdf(t), t)
    assert abs(mse_grid - mse_quad) < 1e-6
    assert abs(mse_quad - expected) < 1e-4


# --------------------------------------------------------------------------- affine

@pytest.mark.parametrize("d,plo,phi", [(128, 0.5, 99.5), (64, 0.5, 99.5), (128, 1.0, 99.0), (128, 2.5, 97.5), (16, 10.0, 90.0)])
def test_affine_percentiles_match_numpy(d, plo, phi):
    rng = np.random.default_rng(d)
    x = rng.standard_t(3, (3000, d)) * rng.uniform(0.1, 20, (3000, 1))
    xs = np.sort(x, axis=-1)
    ref = np.percentile(x, [plo, phi], axis=-1)
    lo, hi = R.percentile_linear(xs, plo), R.percentile_linear(xs, phi)
    assert np.allclose(lo, ref[0], rtol=1e-12, atol=1e-12 * np.abs(x).max())
    assert np.allclose(hi, ref[1], rtol=1e-12, atol=1e-12 * np.abs(x).max())
    s, z = R.affine_params(x, 2, plo, phi)
    assert np.array_equal(z, R.f16(ref[0]))
    assert np.allclose(s, R.f16((ref[1] - ref[0]) / 3), rtol=1e-3, atol=0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_affine_invariants_and_brute_force(bits):
    rng = np.random.default_rng(10 + bits)
    L = 2 ** bits
    x = rng.standard_t(3, (4000, 128)) * rng.uniform(0.05, 30, (4000, 1))
    s, z = R.affine_params(x, bits, 0.5, 99.5)
    codes = R.affine_codes(x, s, z, bits)
    assert codes.min() >= 0 and codes.max() <= L - 1
    xh = R.affine_dequant(codes, s, z)
    inside = (x >= z[:, None]) & (x <= (z + (L - 1) * s)[:, None])
    half = np.broadcast_to(s[:, None] / 2, x.shape)
    assert np.all(np.abs(x - xh)[inside] <= half[inside] * (1 + 1e-12))
    levels = z[:, None, None] + np.arange(L)[None, None, :] * s[:, None, None]
    dist = np.abs(x[..., None] - levels)
    srt = np.sort(dist, axis=-1)
    untied = srt[..., 1] - srt[..., 0] > 1e-9 * s[:, None]
    assert np.array_equal(np.argmin(dist, axis=-1)[untied], codes[untied])
    # the codes change exactly at the listed decision boundaries
    par = np.stack([s, z], -1)
    b, _ = R.decision_boundaries("affine", bits, par)
    eps = 1e-7 * np.maximum(np.abs(b), s[:, None])
    up = R.codes_from_params(b + eps, "affine", bits, par)
    dn = R.codes_from_params(b - eps, "affine", bits, par)
    assert np.all(up - dn == 1)


def test_quest_decision_boundaries():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((500, 64))
    for bits in (2, 3, 4):
        st = R.quest_params(x, bits, 2.5)
        b, _ = R.decision_boundaries("quest", bits, st[:, None])
        eps = 1e-7 * st[:, None]
        up = R.codes_from_params(b + eps, "quest", bits, st[:, None])
        dn = R.codes_from_params(b - eps, "quest", bits, st[:, None])
        assert np.all(up - dn == 1)
        assert np.all(R.near_boundary(b, "quest", bits, st[:, None]))


def test_affine_degenerate_row():
    x = np.full((2, 32), 3.25)
    s, z = R.affine_params(x, 2, 0.5, 99.5)
    assert s.tolist() == [0.0, 0.0] and z.tolist() == [3.25, 3.25]
    c = R.affine_codes(x, s, z, 2)
    assert np.all(c == 0) and np.all(R.affine_dequant(c, s, z) == 3.25)


def test_fp16_midpoint_detector():
    h = np.float16(1.5).astype(np.float64)
    up = np.nextafter(np.float16(1.5), np.float16(2)).astype(np.float64)
    mid = (h + up) / 2
    assert R.fp16_midpoint_near(np.array([mid, mid * (1 + 5e-7)])).tolist() == [True, True]
    assert R.fp16_midpoint_near(np.array([h, mid * (1 + 5e-6)])).tolist() == [False, False]


# --------------------------------------------------------------------------- transforms

def test_transform_invariance_and_inverse():
    rng = np.random.default_rng(3)
    d = 128
    qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    s = 2.0 ** rng.uniform(-2, 2, d)
    t16 = (qm * s[None, :]).astype(np.float16)
    k = rng.standard_normal((50, d))
    q = rng.standard_normal((7, d))
    kt = R.key_transform(t16, k)
    qt = R.query_transform(t16, q)
    assert np.allclose(qt @ kt.T, q @ k.T, rtol=1e-10, atol=1e-10)
    # T = Q diag(s) before fp16 rounding has inverse-transpose Q diag(1/s)
    exact = qm * s[None, :]
    ti = np.linalg.inv(exact).T
    assert np.allclose(ti, qm / s[None, :], rtol=0, atol=1e-12)
    # identity and orthogonal T
    eye = np.eye(d, dtype=np.float16)
    assert np.array_equal(R.key_transform(eye, k), k)
    assert np.allclose(R.query_transform(eye, q), q, atol=0)
    o16 = qm.astype(np.float16)
    o = o16.astype(np.float64)
    assert np.allclose(R.query_transform(o16, q), q @ np.linalg.inv(o), atol=1e-12)


# --------------------------------------------------------------------------- layout

def _codes_k(d, rule):
    j = np.arange(d)
    return {"j%4": j % 4, "j%8": j % 8, "j": j, "4*(j//16)": 4 * (j // 16), "4*(j%2)": 4 * (j % 2)}[rule][None, :]


def test_pack_k_worked_words():
    for d, bits, rule, words in [(r[0].split()[0], r[0].split()[1], r[0].split()[2], r[1].split())
                                 for r in _golden("pack_worked.txt")["k"]]:
        d, bits = int(d), int(bits)
        raw = LY.pack_k(_codes_k(d, rule), bits)
        got = np.frombuffer(raw.tobytes(), dtype="<u4").tolist()
        assert got == [int(w, 16) for w in words]


def _codes_v(d, rule):
    u = np.arange(64)[:, None]
    j = np.arange(d)[None, :]
    f = {"u//16": u // 16 + 0 * j, "u%4": u % 4 + 0 * j, "(u//4)%4": (u // 4) % 4 + 0 * j,
         "j%4": j % 4 + 0 * u, "4+u%4": 4 + u % 4 + 0 * j, "4*(u%4)+u//16": 4 * (u % 4) + u // 16 + 0 * j,
         "4*(j//16)+j%4": 4 * (j // 16) + j % 4 + 0 * u}
    return f[rule]


def test_pack_v_worked_words():
    rows = _golden("pack_worked.txt")
    for spec, words in rows["v"]:
        d, bits, rule = spec.split()
        got = np.frombuffer(LY.pack_v(_codes_v(int(d), rule), int(bits)).tobytes(), dtype="<u4").tolist()
        kind, *vals = words.split()
        if kind == "all":
            want = [int(vals[0], 16)] * 64
        elif kind == "lanes":
            want = []
            for v in vals:
                w, n = v.split("x")
                want += [int(w, 16)] * int(n)
        else:  # cycle
            want = [int(vals[i % 4], 16) for i in range(64)]
        assert got == want, rule
    (spec, p0, p1), = rows["v3"]
    d, bits, rule = spec.split()
    raw = LY.pack_v(_codes_v(int(d), rule), int(bits))[0]
    assert np.frombuffer(raw[:256].tobytes(), "<u4").tolist() == [int(p0.split()[2], 16)] * 64
    assert np.frombuffer(raw[256:].tobytes(), "<u2").tolist() == [int(p1.split()[2], 16)] * 64


def test_pack_v_worked_words_4bit():
    # plane 1 of a 4-bit value set: its offset, shifts and word index, by hand
    for spec, p0, p1 in _golden("pack_worked.txt")["v4"]:
        d, bits, rule = spec.split()
        d = int(d)
        raw = LY.pack_v(_codes_v(d, rule), int(bits))[0]
        nw = 64 * d // 16
        for plane, text in ((0, p0), (1, p1)):
            name, kind, *vals = text.split()
            assert name == f"plane{plane}" and kind == "cycle"
            want = [int(vals[i % len(vals)], 16) for i in range(nw)]
            got = np.frombuffer(raw[4 * nw * plane:4 * nw * (plane + 1)].tobytes(), "<u4").tolist()
            assert got == want, (spec, plane)
        assert np.array_equal(LY.unpack_v(raw, int(bits), d, 64), _codes_v(d, rule))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_pack_roundtrip(bits, d):
    rng = np.random.default_rng(bits * d)
    assert LY.unpack_k(np.zeros(0, np.uint8), bits, d, 0).shape == (0, d)
    assert LY.unpack_v(np.zeros(0, np.uint8), bits, d, 0).shape == (0, d)
    for T in (1, 63, 64, 65, 200):
        c = rng.integers(0, 2 ** bits, (T, d))
        assert np.array_equal(LY.unpack_k(LY.pack_k(c, bits), bits, d, T), c)
        pv = LY.pack_v(c, bits)
        assert pv.shape == (-(-T // 64), LY.v_set_bytes(d, bits))
        assert np.array_equal(LY.unpack_v(pv, bits, d, T), c)
        assert LY.pack_k(c, bits).shape == (T, LY.k_row_bytes(d, bits))
