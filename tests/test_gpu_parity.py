"""GPU parity of the HIP path against the CPU oracle (run on an MI355X).

Each test names its workload, shape and seed in its printed lines.  Sizes are
chosen so the oracle finishes in seconds while spanning several 64-token sets,
flush boundaries and a ragged tail; the full-size workloads are checked on
sampled (batch row, KV head) pairs."""
import numpy as np
import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from synth import transforms as TR
from tests.parity_util import Run, say

pytestmark = pytest.mark.gpu


def test_c0_tiny_full():
    w = configs.TINY
    r = Run(w, n_total=w.capacity)
    r.append(w.context)
    r.check_cache()
    r.append(1)
    q, qt, out = r.decode(0)
    r.check_cache()
    r.check_decode(q, qt, out)


def test_c1_layer_decode_steps():
    """The 8B-class layer: 8192-token prefill, then 64 decode steps (8 flushes), each
    decode held to the oracle on all 8 KV heads (32 query heads)."""
    w = configs.LAYER_8B
    r = Run(w)
    r.append(w.context)
    _, stats = r.check_cache()
    say(f"[c1 prefill] {stats}")
    worst = 0.0
    for step in range(w.decode_steps):
        r.append(1)
        q, qt, out = r.decode(step)
        e2e, _ = r.check_decode(q, qt, out)
        worst = max(worst, e2e)
    _, stats = r.check_cache()
    say(f"[c1 after 64 steps] {stats}; worst end-to-end rel-L2 over the steps {worst:.3e}")


def test_c2_serving_scaled():
    w = configs.SERVING.scaled(batch=2, context=4000)
    r = Run(w)
    r.append(w.context)
    r.check_cache()
    r.append(1)
    q, qt, out = r.decode(0)
    r.check_decode(q, qt, out)


def test_c4_long_context_scaled_empty_partitions():
    # 128 partitions over fewer than 128 sets leaves some partitions empty
    w = configs.LONG_CONTEXT.scaled(batch=1, context=6000)
    r = Run(w)
    r.append(w.context)
    r.check_cache()
    r.append(1)
    q, qt, out = r.decode(0, num_splits=128)
    r.check_decode(q, qt, out)


def test_c4_partitions_beyond_resident_waves():
    """More KV partitions than the GPU holds resident decode waves per KV head (64 KV
    heads ask 128): the MFMA kernel has each wave walk consecutive logical partitions'
    tokens rather than run several rounds of workgroups, so the request equals the
    library's own count bit for bit, and is held to the oracle on sampled heads."""
    w = configs.LONG_CONTEXT.scaled(context=12000)
    r = Run(w)
    r.append(w.context)
    r.append(1)
    p_lib = W.decode_num_splits(r.cache, r.cache.n, w.num_q_heads, 0)
    q, qt, out128 = r.decode(0, num_splits=128)
    r.check_decode(q, qt, out128, heads=[(0, 0), (3, 5), (7, 7)])
    if p_lib < 128:
        _, _, out_lib = r.decode(0, num_splits=p_lib)
        torch.cuda.synchronize()
        assert torch.equal(out128, out_lib), p_lib


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_c3_bulk_flush_scaled(bits):
    w = configs.BULK_FLUSH.scaled(num_kv_heads=2, num_q_heads=8, context=4096 + 37, bits_k=bits, bits_v=bits)
    r = Run(w, n_total=w.context)
    r.append(w.context)
    _, stats = r.check_cache()
    say(f"[c3 bits={bits}] {stats}")


FUZZ = [
    # d, bits_k, bits_v, quant_k, quant_v, chunk, n_prefill, steps, G
    (64, 2, 2, "quest", "quest", 8, 10, 3, 4),
    (64, 3, 4, "affine", "quest", 16, 70, 5, 2),
    (128, 4, 3, "quest", "affine", 8, 319, 12, 1),
    (128, 2, 3, "affine", "affine", 16, 600, 20, 8),
    (64, 4, 4, "affine", "affine", 8, 1000, 9, 16),
    (128, 3, 2, "quest", "quest", 16, 333, 17, 4),
]


@pytest.mark.parametrize("case", FUZZ, ids=[f"d{c[0]}k{c[1]}v{c[2]}{c[3][0]}{c[4][0]}C{c[5]}n{c[6]}G{c[8]}" for c in FUZZ])
def test_fuzz_shapes_and_flush_boundaries(case):
    d, bk, bv, qk, qv, C, n0, steps, G = case
    w = configs.SERVING.scaled(name="fuzz", seed=100 + n0, batch=2, num_kv_heads=2, num_q_heads=2 * G, head_dim=d,
                               context=n0, decode_steps=steps, bits_k=bk, bits_v=bv, quant_k=qk, quant_v=qv,
                               chunk=C, k_dist="gauss", v_dist="t3")
    r = Run(w)
    r.append(n0)
    r.check_cache()
    for s in range(steps):
        r.append(1)
        q, qt, out = r.decode(s, num_splits=(s % 3))
        r.check_decode(q, qt, out)
    r.check_cache()


def test_token_by_token_equals_prefill():
    """A 420-token prefill and 420 single-token appends leave bitwise-equal live
    cache contents (ring slots of flushed tokens are stale and not compared)."""
    from oracle import layout as LY
    from oracle import wushkv_ref as R
    from tests.parity_util import plane_arrays
    w = configs.SERVING.scaled(name="tok", seed=7, batch=1, num_kv_heads=2, num_q_heads=8, context=420,
                               decode_steps=0, chunk=8)
    a = Run(w)
    a.append(420)
    b = Run(w)
    for _ in range(420):
        b.append(1)
    torch.cuda.synchronize()
    pa, pb = plane_arrays(a.cache), plane_arrays(b.cache)
    nb = R.n_quantized(420, 64, 256, 8)
    live = (np.arange(64 + nb, 420) - 64) % (256 + 8)
    for g in range(2):
        for p in ("sink_k", "sink_v"):
            assert np.array_equal(pa[p][0, g].view(np.uint16), pb[p][0, g].view(np.uint16)), p
        for p in ("ring_k", "ring_v"):
            assert np.array_equal(pa[p][0, g, live].view(np.uint16), pb[p][0, g, live].view(np.uint16)), p
        for p in ("par_k", "par_v"):
            assert np.array_equal(pa[p][0, g, :nb].view(np.uint16), pb[p][0, g, :nb].view(np.uint16)), p
        assert np.array_equal(LY.unpack_k(pa["codes_k"][0, g], 2, 128, nb), LY.unpack_k(pb["codes_k"][0, g], 2, 128, nb))
        assert np.array_equal(LY.unpack_v(pa["codes_v"][0, g], 2, 128, nb), LY.unpack_v(pb["codes_v"][0, g], 2, 128, nb))
    a.check_cache()
    b.check_cache()


def test_decode_deterministic_and_split_invariant():
    w = configs.SERVING.scaled(name="det", seed=9, batch=2, context=3000)
    r = Run(w)
    r.append(w.context)
    q, qt, o1 = r.decode(0, num_splits=5)
    _, _, o2 = r.decode(0, num_splits=5)
    assert torch.equal(o1, o2)
    for P in (1, 2, 17, 47):
        _, _, o3 = r.decode(0, num_splits=P)
        rel = float((o3 - o1).norm() / o1.norm())
        assert rel < 1e-5, (P, rel)


def test_decode_workspace_reuse():
    """One workspace serves decodes of different split counts: each call matches a
    call on a fresh workspace bit for bit."""
    w = configs.SERVING.scaled(name="wsreuse", seed=12, batch=3, context=4000)
    r = Run(w)
    r.append(w.context)
    r.append(1)
    q = r.decode(0)[0]
    qt = W.query_transform(r.tinvt, q, w.num_kv_heads)
    ws = W.decode_workspace(r.cache, r.cache.n, w.num_q_heads, 64)
    for P in (5, 1, 17, 64, 5, 0, 3):
        fresh = W.decode_attention(r.cache, q, qt, num_splits=P)
        reused = W.decode_attention(r.cache, q, qt, num_splits=P, workspace=ws)
        torch.cuda.synchronize()
        say(f"[workspace reuse] P={P}")
        assert torch.equal(fresh, reused), P
    r.check_decode(q, qt, reused)


def test_decode_large_batch_short_context():
    """A batch of 520 sequences at a short context: 4160 (batch row, KV head) grid rows,
    few body sets each."""
    w = configs.SERVING.scaled(name="manyheads", seed=13, batch=520, context=700)
    r = Run(w)
    r.append(w.context)
    r.append(1)
    q, qt, out = r.decode(0)
    r.check_decode(q, qt, out, heads=[(0, 0), (263, 4), (519, 7)])


@pytest.mark.parametrize("wl", ["whole", "split", "generic", "forced"])
def test_fused_query_transform_is_bitwise(wl):
    """The decode that forms q~ itself returns the same q~ and output, bit for bit, as
    the query transform followed by the plain decode: the 12-wave layout (n >= ~1800
    gives the library's 12 splits at 32 x 8 KV heads), the split layout, a shape only
    the generic kernel serves, and the generic kernel chosen by its own entry point."""
    w = {"whole": configs.SERVING.scaled(name="fw", seed=31, context=2000),
         "split": configs.LAYER_8B.scaled(name="fs", seed=32, context=3000),
         "generic": configs.TINY.scaled(name="fg", seed=33),
         "forced": configs.LAYER_8B.scaled(name="ff", seed=34, context=2000)}[wl]
    r = Run(w, n_total=w.context + 1)
    r.append(w.context)
    r.append(1)
    q = gen.queries(w, 0, 0, "cuda")
    qt = W.query_transform(r.tinvt, q, w.num_kv_heads)
    if wl == "whole":
        assert W.decode_num_splits(r.cache, r.cache.n, w.num_q_heads, 0) == 12
    if wl == "forced":
        ref, _ = W.decode_attention_generic(r.cache, q, q_t=qt)
        out, qt2 = W.decode_attention_generic(r.cache, q, t_inv_t=r.tinvt)
    else:
        ref = W.decode_attention(r.cache, q, qt)
        out, qt2 = W.decode_attention_fused(r.cache, q, r.tinvt)
    torch.cuda.synchronize()
    say(f"[fused] {wl}: q~ equal {torch.equal(qt, qt2)}, out equal {torch.equal(ref, out)}")
    assert torch.equal(qt, qt2)
    assert torch.equal(ref, out)


def test_snapshot_restore_continues_bitwise():
    w = configs.LAYER_8B.scaled(name="snap", context=1000, decode_steps=20)
    r = Run(w)
    r.append(1000)
    snap = r.cache.snapshot()
    outs = []
    for s in range(20):
        r.append(1)
        outs.append(r.decode(s)[2].clone())
    r.cache.restore(snap)
    for s in range(20):
        r.append(1)
        assert torch.equal(r.decode(s)[2], outs[s]), s


@pytest.mark.parametrize("wl,P", [("serving", 0), ("serving", 13), ("long", 128), ("layer", 0)])
def test_fast_decode_matches_generic_kernel(wl, P):
    """The MFMA decode and the generic decode agree on the same cache."""
    w = {"serving": configs.SERVING.scaled(batch=3, context=5000, seed=21),
         "long": configs.LONG_CONTEXT.scaled(batch=2, context=9000, seed=22),
         "layer": configs.LAYER_8B.scaled(context=3000, seed=23)}[wl]
    r = Run(w)
    r.append(w.context)
    r.append(1)
    q, qt, fast = r.decode(0, num_splits=P)
    gen_out, _ = W.decode_attention_generic(r.cache, q, q_t=qt, num_splits=P)
    torch.cuda.synchronize()
    rel = float((fast - gen_out).norm() / gen_out.norm())
    say(f"[fast vs generic] {wl} P={P} rel-L2 {rel:.3e}")
    assert rel < 1e-4
    r.check_decode(q, qt, fast)


WIDE = [
    # bits_k, bits_v, quant_k, quant_v, G
    (4, 2, "quest", "quest", 4),
    (2, 4, "affine", "affine", 4),
    (4, 4, "quest", "quest", 4),
    (4, 3, "affine", "affine", 8),
    (4, 4, "affine", "quest", 8),
    (2, 4, "quest", "affine", 8),
    (3, 2, "quest", "quest", 4),
    (3, 3, "affine", "affine", 4),
    (3, 4, "quest", "affine", 8),
    (3, 3, "quest", "quest", 8),
]


@pytest.mark.parametrize("bits_k,bits_v,quant_k,quant_v,G", WIDE)
def test_wide_codes_mfma_decode(bits_k, bits_v, quant_k, quant_v, G):
    """4-bit keys (two 2-bit planes on the same q~ digits, the high plane's products
    scaled by 4), 3-bit keys (the third-bit plane as a second fp4 operand of e2m1 value
    2 per set bit) and 4-bit values (a second B operand on the same W at four times the
    weight) on the MFMA decode: held to the oracle, and to the generic kernel on the same
    cache, with a ragged last set and several splits."""
    qk = configs.QUEST if quant_k == "quest" else configs.AFFINE
    qv = configs.QUEST if quant_v == "quest" else configs.AFFINE
    w = configs.SERVING.scaled(name=f"wide{bits_k}{bits_v}{G}", seed=40 + bits_k + 3 * bits_v + G, batch=3,
                               context=3000 + 37, num_q_heads=8 * G, num_kv_heads=8, bits_k=bits_k, bits_v=bits_v,
                               quant_k=qk, quant_v=qv)
    r = Run(w)
    r.append(w.context)
    r.check_cache(heads=[(0, 0), (2, 7)])
    r.append(1)
    for P in (0, 8):
        q, qt, fast = r.decode(0, num_splits=P)
        gen_out, _ = W.decode_attention_generic(r.cache, q, q_t=qt, num_splits=P if P else 8)
        torch.cuda.synchronize()
        rel = float((fast - gen_out).norm() / gen_out.norm())
        say(f"[wide {bits_k}/{bits_v} {quant_k}/{quant_v} G={G} P={P}] fast vs generic rel-L2 {rel:.3e}")
        assert rel < 1e-4
        r.check_decode(q, qt, fast, heads=[(0, 0), (1, 3), (2, 7)])


@pytest.mark.parametrize("bits_v", [2, 3])
def test_whole_workgroup_layout_matches_generic(bits_v):
    """At the serving batch (256 (batch row, KV head) pairs) with 12 splits (the
    library's choice for 2-bit values) each KV head's partitions share one workgroup,
    which writes the output itself."""
    w = configs.SERVING.scaled(name=f"whole{bits_v}", seed=24 + bits_v, context=2000, bits_v=bits_v)
    r = Run(w)
    r.append(w.context)
    r.append(1)
    if bits_v == 2:
        assert W.decode_num_splits(r.cache, r.cache.n, w.num_q_heads, 0) == 12
    q, qt, fast = r.decode(0, num_splits=12)
    gen_out, _ = W.decode_attention_generic(r.cache, q, q_t=qt, num_splits=12)
    torch.cuda.synchronize()
    rel = float((fast - gen_out).norm() / gen_out.norm())
    say(f"[whole vs generic] bits_v={bits_v} rel-L2 {rel:.3e}")
    assert rel < 1e-4
    r.check_decode(q, qt, fast, heads=[(0, 0), (17, 3), (31, 7)])


# ---- full-size workloads, in the launch configuration the benchmark times, checked on
# sampled (batch row, KV head) pairs (the oracle builds each sampled head's whole cache)

def test_c2_serving_full_size_sampled():
    w = configs.SERVING                       # B=32, n=32768, affine 2/2-bit, chunk 16
    r = Run(w)
    r.append(w.context)
    heads = [(0, 0), (13, 5), (31, 7)]
    _, stats = r.check_cache(heads)
    say(f"[c2 full] cache {stats}")
    r.append(1)
    q, qt, out = r.decode(0, num_splits=0)    # the library's split choice, as timed
    r.check_decode(q, qt, out, heads=heads)


def test_c4_long_context_full_size_sampled():
    w = configs.LONG_CONTEXT                  # B=8, n=131072, G=8, affine K 2-bit / V 3-bit
    r = Run(w)
    r.append(w.context)
    heads = [(0, 0), (7, 6)]
    _, stats = r.check_cache(heads)
    say(f"[c4 full] cache {stats}")
    r.append(1)
    q, qt, out = r.decode(0, num_splits=w.num_splits)
    r.check_decode(q, qt, out, heads=heads)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_c3_bulk_flush_full_size_sampled(bits):
    # one of the 36 layer calls: 8 KV heads x 65536 tokens, the timed launch
    w = configs.BULK_FLUSH.scaled(bits_k=bits, bits_v=bits)
    r = Run(w, layer=5, n_total=w.context)
    r.append(w.context)
    _, stats = r.check_cache([(0, 1), (0, 6)])
    say(f"[c3 full bits={bits}] {stats}")


def test_degenerate_rows():
    """All-zero rows (QuEST step 0 -> code L/2; affine scale 0 -> code 0) and
    constant rows (affine hi == lo) in both K and V, flushed and decoded."""
    for quant in ("quest", "affine"):
        w = configs.SERVING.scaled(name=f"degen_{quant}", seed=31, batch=1, num_kv_heads=2, num_q_heads=8,
                                   context=700, decode_steps=1, quant_k=quant, quant_v=quant, chunk=8)
        r = Run(w)
        k, v = r.k, r.v
        k[:, :, 100:140] = 0
        v[:, :, 120:160] = 0
        k[:, 1, 300:340] = 1.5
        v[:, 0, 310:350] = -0.75
        r.append(w.context)
        _, stats = r.check_cache()
        say(f"[degenerate {quant}] {stats}")
        r.append(1)
        q, qt, out = r.decode(0)
        r.check_decode(q, qt, out)


def test_value_rows_on_decision_boundaries():
    """Value rows whose elements sit exactly on the affine decision boundaries: with two
    channels at 0 and two at 3, the percentile range is [0, 3], so the 2-bit scale is 1
    and the zero 0, and the other channels take 0.5, 1.5 and 2.5 (exact in bf16).  Every
    such element is a tie, decided again in fp64 by the flush (round half to even: codes
    0, 2, 2), up to 124 per row and 32 per lane.  No mismatch is allowed, not even in the
    band the parity rule admits."""
    w = configs.SERVING.scaled(name="value_ties", seed=37, batch=1, num_kv_heads=2, num_q_heads=8,
                               context=700, decode_steps=1, chunk=16)
    r = Run(w)
    d = w.head_dim
    base = torch.tensor([0.0, 0.0, 3.0, 3.0] + [0.5, 1.5, 2.5] * ((d - 4) // 3) + [1.5] * ((d - 4) % 3))
    rows = torch.stack([torch.roll(base, 7 * i) for i in range(700)]).to(r.v.dtype).to(r.v.device)
    r.v[0, 0, 64:600] = rows[64:600]
    r.v[0, 1, 200:400] = rows[200:400]
    r.append(w.context)
    _, stats = r.check_cache()
    say(f"[value ties] {stats}")
    assert stats["code_mism"] == 0, stats
    r.append(1)
    q, qt, out = r.decode(0)
    r.check_decode(q, qt, out)


def test_key_rows_on_decision_boundaries():
    """The same ties on the key side.  With T_K the identity the contraction is exact
    (products k * 1 and k * 0), so key rows built like the value rows above land exactly
    on the boundaries, and every tie goes through the per-token fp64 dot product, one
    candidate per pass of the four lanes of a token (up to 124 passes per tile)."""
    w = configs.SERVING.scaled(name="key_ties", seed=41, batch=1, num_kv_heads=2, num_q_heads=8,
                               context=700, decode_steps=1, chunk=16)
    r = Run(w)
    d, H = w.head_dim, w.num_kv_heads
    t16, tinvt = TR.as_inputs(TR.per_head(np.eye(d), H))
    r.t16_cpu, r.t16, r.tinvt = t16, t16.to(r.k.device), tinvt.to(r.k.device)
    base = torch.tensor([0.0, 0.0, 3.0, 3.0] + [0.5, 1.5, 2.5] * ((d - 4) // 3) + [1.5] * ((d - 4) % 3))
    rows = torch.stack([torch.roll(base, 5 * i) for i in range(700)]).to(r.k.dtype).to(r.k.device)
    r.k[0, 0, 64:600] = rows[64:600]
    r.k[0, 1, 100:300] = rows[100:300]
    r.append(w.context)
    _, stats = r.check_cache()
    say(f"[key ties] {stats}")
    assert stats["code_mism"] == 0, stats
    r.append(1)
    q, qt, out = r.decode(0)
    r.check_decode(q, qt, out)


def test_wide_percentiles_exact_params():
    """Affine quantization at the 5th / 95th percentiles: eight order statistics from each
    end (the most the flush keeps), K and V, prefill and steps across flushes; parameters
    bit-exact, codes within the boundary rule, decode to the oracle."""
    w = configs.SERVING.scaled(name="pct5", seed=43, batch=2, num_kv_heads=4, num_q_heads=16, context=3000,
                               decode_steps=20, pct_lo=5.0, pct_hi=95.0, chunk=8)
    r = Run(w)
    r.append(w.context)
    _, stats = r.check_cache()
    say(f"[percentiles 5/95] prefill {stats}")
    for s in range(w.decode_steps):
        r.append(1)
    q, qt, out = r.decode(0)
    _, stats = r.check_cache()
    say(f"[percentiles 5/95] after {w.decode_steps} steps {stats}")
    r.check_decode(q, qt, out)
