"""Token counts in device memory (wushkv_append_flush_device, wushkv_decode_attention_device)
and the decode step captured as a graph.

The device-count path runs the same kernels as the host-count ragged path, with each
sequence's count read on the device instead of from the launch arguments, so with the
split count fixed the two give the same caches and outputs bit for bit.  The ragged path
is itself held to the oracle (test_gpu_ragged.py); here the device path is held to it
bitwise, step by step, and the graph-replayed step to both."""
import ctypes

import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from tests.parity_util import check_decode_lengths, plane_arrays, say, spec_of

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 320, 335, 1000, 2501]
STEPS = 20


def _twin_caches(w, lengths, steps):
    """Two caches holding the same ragged prefill, plus the token streams."""
    cap = max(lengths) + steps
    k, v = gen.kv_tensors(w, 0, cap, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    caches = []
    for _ in range(2):
        c = W.KVCache(spec_of(w, capacity=cap), "cuda")
        for b, n in enumerate(lengths):
            W.append_flush(c.sequence(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(),
                           t16.cuda(), n_before=0)
        c.seq_n = list(lengths)
        caches.append(c)
    return caches, k, v, t16.cuda(), tinvt.cuda(), cap


def _next_tokens(k, v, counts):
    ks = torch.stack([k[b, :, n:n + 1] for b, n in enumerate(counts)]).contiguous()
    vs = torch.stack([v[b, :, n:n + 1] for b, n in enumerate(counts)]).contiguous()
    return ks, vs


def _splits(cache, max_tokens, hq):
    return W.lib().wushkv_decode_num_splits(ctypes.byref(cache.desc), max_tokens, hq, 0)


def _quantized(n, w):
    """Body tokens once n are cached: whole chunks past the sink and recent windows."""
    return w.chunk * (max(0, n - w.sink - w.recent) // w.chunk)


def _same_planes(a, b):
    for p in W.PLANES:
        assert torch.equal(a.planes[p], b.planes[p]), p


@pytest.mark.parametrize("wl", ["serving", "long"])
def test_device_counts_match_host_counts(wl):
    base = configs.SERVING if wl == "serving" else configs.LONG_CONTEXT
    w = base.scaled(batch=len(LENGTHS))
    (ha, dv), k, v, t16, tinvt, cap = _twin_caches(w, LENGTHS, STEPS)
    counts = torch.tensor(LENGTHS, dtype=torch.int32, device="cuda")
    P = _splits(ha, cap, w.num_q_heads)
    say(f"[device counts {w.name}] lengths {LENGTHS}, capacity {cap}, {P} splits")
    for step in range(STEPS):
        ks, vs = _next_tokens(k, v, ha.seq_n)
        W.append_flush_ragged(ha, ks, vs, t16)
        W.append_flush_device(dv, counts, ks, vs, t16)
        q = gen.queries(w, 0, step, "cuda")
        oh, qh = W.decode_attention_ragged(ha, q, t_inv_t=tinvt, num_splits=P)
        od, qd = W.decode_attention_device(dv, counts, cap, q, t_inv_t=tinvt, num_splits=P)
        torch.cuda.synchronize()
        assert counts.tolist() == ha.seq_n, (step, counts.tolist(), ha.seq_n)
        assert torch.equal(qh, qd), step
        assert torch.equal(oh, od), step
    _same_planes(ha, dv)


def test_graph_replays_the_next_step():
    """One device-count step (append + flush + decode with the query transform) recorded
    into a graph and replayed STEPS times, new tokens and queries copied into its input
    buffers before each replay, with eager work (the host-count twin) and
    synchronizations between replays: every replay equals the eager step bitwise, and
    the replays cross flushes of different sequences."""
    w = configs.SERVING.scaled(batch=len(LENGTHS))
    (ha, dv), k, v, t16, tinvt, cap = _twin_caches(w, LENGTHS, STEPS + 1)
    counts = torch.tensor(LENGTHS, dtype=torch.int32, device="cuda")
    P = _splits(ha, cap, w.num_q_heads)
    B, Hkv, d, Hq = w.batch, w.num_kv_heads, w.head_dim, w.num_q_heads
    ks_buf = torch.empty((B, Hkv, 1, d), dtype=k.dtype, device="cuda")
    vs_buf = torch.empty_like(ks_buf)
    q_buf = torch.empty((B, Hq, d), dtype=gen.queries(w, 0, 0, "cuda").dtype, device="cuda")
    qt_buf = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    out_buf = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = W.decode_workspace(dv, cap, Hq, P)

    def fill(step, counts_now):
        ks, vs = _next_tokens(k, v, counts_now)
        ks_buf.copy_(ks)
        vs_buf.copy_(vs)
        q_buf.copy_(gen.queries(w, 0, step, "cuda"))
        return ks, vs

    def device_step():
        W.append_flush_device(dv, counts, ks_buf, vs_buf, t16)
        W.decode_attention_device(dv, counts, cap, q_buf, t_inv_t=tinvt, q_t=qt_buf, num_splits=P, workspace=ws,
                                  out=out_buf)

    # step 0 eagerly on both (it also primes the library's per-kernel queries)
    ks, vs = fill(0, ha.seq_n)
    device_step()
    W.append_flush_ragged(ha, ks, vs, t16)
    oh, _ = W.decode_attention_ragged(ha, q_buf, t_inv_t=tinvt, num_splits=P)
    torch.cuda.synchronize()
    assert torch.equal(oh, out_buf)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):             # records on torch's capture stream
        device_step()
    torch.cuda.synchronize()
    assert counts.tolist() == ha.seq_n      # recording ran nothing
    flushes = 0
    for step in range(1, STEPS + 1):
        ks, vs = fill(step, ha.seq_n)
        before = [_quantized(n, w) for n in ha.seq_n]
        g.replay()
        W.append_flush_ragged(ha, ks, vs, t16)
        oh, qh = W.decode_attention_ragged(ha, q_buf, t_inv_t=tinvt, num_splits=P)
        torch.cuda.synchronize()
        flushes += sum(_quantized(n, w) > q for n, q in zip(ha.seq_n, before))
        assert counts.tolist() == ha.seq_n, step
        assert torch.equal(qh, qt_buf), step
        assert torch.equal(oh, out_buf), step
    _same_planes(ha, dv)
    say(f"[graph replay] {STEPS} replays over lengths {LENGTHS} -> {ha.seq_n}, {flushes} sequence flushes")
    assert flushes >= len(LENGTHS) - 2


def test_device_counts_out_of_range():
    """A device count outside the valid range leaves that sequence's cache and count
    alone (append) or gives NaN rows for it (decode); the other sequences are unaffected."""
    w = configs.SERVING.scaled(batch=4)
    lengths = [300, 700, 700, 1200]
    (ha, dv), k, v, t16, tinvt, cap = _twin_caches(w, lengths, 4)
    bad = [300, -1, cap, 1200]          # sequence 1 negative, sequence 2 full
    counts = torch.tensor(bad, dtype=torch.int32, device="cuda")
    ks, vs = _next_tokens(k, v, [300, 700, 700, 1200])
    W.append_flush_device(dv, counts, ks, vs, t16)
    torch.cuda.synchronize()
    assert counts.tolist() == [301, -1, cap, 1201]
    for b in (1, 2):                     # untouched, byte for byte (ha is the prefill as it was)
        for p in W.PLANES:
            assert torch.equal(dv.sequence(b).planes[p], ha.sequence(b).planes[p]), (b, p)
    q = gen.queries(w, 0, 0, "cuda")
    dcounts = torch.tensor([301, 0, cap + 5, 1201], dtype=torch.int32, device="cuda")
    P = _splits(ha, cap, w.num_q_heads)
    od, _ = W.decode_attention_device(dv, dcounts, cap, q, t_inv_t=tinvt, num_splits=P)
    W.append_flush_ragged(ha.sequence(0), ks[0:1], vs[0:1], t16, n_before=[300])
    W.append_flush_ragged(ha.sequence(3), ks[3:4], vs[3:4], t16, n_before=[1200])
    oh, _ = W.decode_attention_ragged(ha, q, t_inv_t=tinvt, n_tokens=[301, 700, 700, 1201], num_splits=P)
    torch.cuda.synchronize()
    assert torch.isnan(od[1]).all() and torch.isnan(od[2]).all()
    assert torch.equal(od[0], oh[0]) and torch.equal(od[3], oh[3])


@pytest.mark.parametrize("layout", ["split", "whole"])
def test_device_step_matches_host_counts(layout):
    """wushkv_decode_step_device (flush, decode with the append fused, count update)
    against the host-count ragged calls, bitwise, over steps that cross flushes; the
    whole layout (one 12-wave workgroup per KV head) needs 32 x 8 KV heads."""
    if layout == "split":
        w, lengths = configs.SERVING.scaled(batch=len(LENGTHS)), LENGTHS
    else:
        w = configs.SERVING.scaled(batch=32)
        lengths = [1900 + 7 * b for b in range(32)]
    (ha, dv), k, v, t16, tinvt, cap = _twin_caches(w, lengths, STEPS)
    counts = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    P = _splits(ha, cap, w.num_q_heads)
    if layout == "whole":
        assert P == 12, P
    t16_cpu = gen.key_transforms(w, 0)[0]
    heads = [(0, 0), (len(lengths) // 2, 3), (len(lengths) - 1, 7)]
    for step in range(STEPS):
        ks, vs = _next_tokens(k, v, ha.seq_n)
        q = gen.queries(w, 0, step, "cuda")
        W.append_flush_ragged(ha, ks, vs, t16)
        oh, qh = W.decode_attention_ragged(ha, q, t_inv_t=tinvt, num_splits=P)
        od, qd = W.decode_step_device(dv, counts, cap, ks, vs, t16, q, tinvt, num_splits=P)
        torch.cuda.synchronize()
        assert counts.tolist() == ha.seq_n, step
        assert torch.equal(qh, qd), step
        assert torch.equal(oh, od), (step, float((oh - od).abs().max()))
        if step in (0, STEPS - 1):
            # the device-count step against the oracle itself, on its own cache
            check_decode_lengths(plane_arrays(dv), dv.spec, w, k, v, t16_cpu, counts.tolist(), q, qd, od,
                                 heads=heads, what=f"device step {layout}, step {step}")
    _same_planes(ha, dv)
    say(f"[device step {layout}] {P} splits, {STEPS} steps: equal to the host-count calls")


def test_graph_replays_the_fused_device_step():
    """One wushkv_decode_step_device call recorded into a graph and replayed STEPS
    times, as the graph test above, against the host-count calls."""
    w = configs.SERVING.scaled(batch=len(LENGTHS))
    (ha, dv), k, v, t16, tinvt, cap = _twin_caches(w, LENGTHS, STEPS + 1)
    counts = torch.tensor(LENGTHS, dtype=torch.int32, device="cuda")
    P = _splits(ha, cap, w.num_q_heads)
    B, Hkv, d, Hq = w.batch, w.num_kv_heads, w.head_dim, w.num_q_heads
    ks_buf = torch.empty((B, Hkv, 1, d), dtype=k.dtype, device="cuda")
    vs_buf = torch.empty_like(ks_buf)
    q_buf = torch.empty((B, Hq, d), dtype=gen.queries(w, 0, 0, "cuda").dtype, device="cuda")
    qt_buf = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    out_buf = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = W.decode_workspace(dv, cap, Hq, P)

    def fill(step):
        ks, vs = _next_tokens(k, v, ha.seq_n)
        ks_buf.copy_(ks)
        vs_buf.copy_(vs)
        q_buf.copy_(gen.queries(w, 0, step, "cuda"))
        return ks, vs

    def device_step():
        W.decode_step_device(dv, counts, cap, ks_buf, vs_buf, t16, q_buf, tinvt, q_t=qt_buf, num_splits=P,
                             workspace=ws, out=out_buf)

    def host_step(ks, vs):
        W.append_flush_ragged(ha, ks, vs, t16)
        return W.decode_attention_ragged(ha, q_buf, t_inv_t=tinvt, num_splits=P)

    ks, vs = fill(0)
    device_step()                            # eager first step (primes the library)
    oh, _ = host_step(ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(oh, out_buf)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device_step()
    torch.cuda.synchronize()
    for step in range(1, STEPS + 1):
        ks, vs = fill(step)
        g.replay()
        oh, qh = host_step(ks, vs)
        torch.cuda.synchronize()
        assert counts.tolist() == ha.seq_n, step
        assert torch.equal(qh, qt_buf), step
        assert torch.equal(oh, out_buf), step
    # the last replay against the oracle, on the graph-stepped cache itself
    check_decode_lengths(plane_arrays(dv), dv.spec, w, k, v, gen.key_transforms(w, 0)[0], counts.tolist(), q_buf,
                         qt_buf, out_buf, what=f"graph-replayed fused step {STEPS}")
    _same_planes(ha, dv)
