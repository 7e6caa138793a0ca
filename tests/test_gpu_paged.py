"""Paged body (wushkv_append_flush_paged, wushkv_decode_attention_paged) against the
oracle and against the contiguous ragged cache.

Paging only moves where each body row lives: every row keeps its layout, the kernels'
arithmetic is unchanged.  So a paged cache whose sequences map their logical pages to
physical pages in a shuffled order holds, page by page, exactly the rows of the
contiguous cache, and decodes to the same outputs bit for bit.  The paged cache itself
is also held to the oracle: its rows gathered through the page table pass the cache
parity rule for every (sequence, KV head), and its decode is checked end to end and on
its own contents.  Covered: the fast decode's split layout (serving shape), its
3-bit-value path (long-context shape) and the generic kernel (d = 64)."""
import numpy as np
import pytest
import torch

import bit_kv_cache_amd as W
from synth import configs, gen
from tests.parity_util import check_decode_lengths, check_head, paged_plane_arrays, say, spec_of

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 320, 335, 1000, 2501]
STEPS = 20
PAGE = 256


def _workload(name):
    if name == "serving":
        return configs.SERVING.scaled(batch=len(LENGTHS))
    if name == "long":
        return configs.LONG_CONTEXT.scaled(batch=len(LENGTHS))
    return configs.TINY.scaled(batch=len(LENGTHS), num_q_heads=8, num_kv_heads=2)


def _row_bytes(spec):
    """Bytes per body row of each pooled plane (value codes: a set's bytes / 64)."""
    d = spec.head_dim
    return {"codes_k": d * spec.bits_k // 8, "codes_v": d * spec.bits_v // 8,
            "par_k": 2 * (1 if spec.quant_k == W.Q_QUEST else 2), "par_v": 2 * (1 if spec.quant_v == W.Q_QUEST else 2)}


@pytest.mark.parametrize("wl", ["serving", "long", "generic"])
def test_paged_matches_contiguous(wl):
    w = _workload(wl)
    cap = max(LENGTHS) + STEPS
    k, v = gen.kv_tensors(w, 0, cap, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.cuda(), tinvt.cuda()
    spec = spec_of(w, capacity=cap)
    ca = W.KVCache(spec, "cuda")
    body = -(-(cap - w.sink) // 64) * 64
    mp = -(-body // PAGE)
    npages = w.batch * mp + 3                     # a few pages nobody uses
    pc = W.PagedKVCache(spec, PAGE, npages, max_pages=mp)
    perm = np.random.default_rng(11).permutation(npages)[: w.batch * mp].reshape(w.batch, mp)
    pc.table.copy_(torch.from_numpy(perm.astype(np.int32)))
    for b, n in enumerate(LENGTHS):
        W.append_flush(ca.sequence(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(), t16,
                       n_before=0)
        W.append_flush_paged(pc.sequence(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(), t16,
                             n_before=[0])
    ca.seq_n = list(LENGTHS)
    pc.seq_n = list(LENGTHS)
    P = W.decode_num_splits(ca, cap, w.num_q_heads, 0)
    say(f"[paged {w.name}] lengths {LENGTHS}, {PAGE}-token pages, {mp} per sequence, {npages} in the pool, {P} splits")
    for step in range(STEPS):
        ks = torch.stack([k[b, :, n:n + 1] for b, n in enumerate(ca.seq_n)]).contiguous()
        vs = torch.stack([v[b, :, n:n + 1] for b, n in enumerate(ca.seq_n)]).contiguous()
        W.append_flush_ragged(ca, ks, vs, t16)
        W.append_flush_paged(pc, ks, vs, t16)
        q = gen.queries(w, 0, step, "cuda")
        oa, qa = W.decode_attention_ragged(ca, q, t_inv_t=tinvt, num_splits=P)
        op, qp = W.decode_attention_paged(pc, q, t_inv_t=tinvt, num_splits=P)
        torch.cuda.synchronize()
        assert torch.equal(qa, qp), step
        assert torch.equal(oa, op), (step, float((oa - op).abs().max()))
    # the paged cache itself against the oracle: every (sequence, KV head), then the last
    # step's decode end to end and on the paged cache's own contents
    pa = paged_plane_arrays(pc)
    stats = {}
    t16_cpu = gen.key_transforms(w, 0)[0]
    for b, n in enumerate(pc.seq_n):
        for g in range(w.num_kv_heads):
            check_head(pa, spec, b, g, k[b, g].float().cpu().numpy().astype(np.float64),
                       v[b, g].float().cpu().numpy().astype(np.float64), t16_cpu[g].numpy(), n, stats)
    if stats.get("code_total"):
        assert stats["code_mism"] <= 1e-5 * stats["code_total"], stats
    say(f"[paged {w.name}] paged cache vs oracle after {STEPS} steps: {stats}")
    check_decode_lengths(pa, spec, w, k, v, t16_cpu, pc.seq_n, q, qp, op, what=f"paged {w.name}")
    # windows as they are; body rows page by page
    for p in W.PagedKVCache.WINDOWS:
        assert torch.equal(ca.planes[p], pc.planes[p]), p
    rb = _row_bytes(spec)
    H = w.num_kv_heads
    for p, r in rb.items():
        cont = ca.planes[p].cpu().numpy()[: w.batch * H * body * r].reshape(w.batch, H, body, r)
        pool = pc.planes[p].cpu().numpy()[: npages * H * PAGE * r].reshape(npages, H, PAGE, r)
        for b in range(w.batch):
            for lp in range(mp):
                rows = min(PAGE, body - lp * PAGE)
                got = pool[perm[b, lp], :, :rows]
                want = cont[b, :, lp * PAGE:lp * PAGE + rows]
                assert np.array_equal(got, want), (p, b, lp)
    say(f"[paged {w.name}] {STEPS} steps: outputs and every page equal to the contiguous cache")


def test_paged_invalid_entries_stay_inside_the_pools():
    """Table entries outside [0, num_pages) are never written through and read as page
    0: a sequence whose entries are all invalid leaves every pool page untouched, and
    the other sequences still equal the contiguous cache bit for bit."""
    w = configs.SERVING.scaled(batch=3)
    lengths = [900, 1300, 700]
    cap = max(lengths) + 4
    k, v = gen.kv_tensors(w, 0, cap, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.cuda(), tinvt.cuda()
    spec = spec_of(w, capacity=cap)
    ca = W.KVCache(spec, "cuda")
    body = -(-(cap - w.sink) // 64) * 64
    mp = -(-body // PAGE)
    npages = 2 * mp + 1                       # page 0 is nobody's; sequences 0 and 2 own the rest
    pc = W.PagedKVCache(spec, PAGE, npages, max_pages=mp)
    table = np.zeros((3, mp), dtype=np.int32)
    table[0] = 1 + np.arange(mp)
    table[1, ::2], table[1, 1::2] = -1, npages + 5          # all invalid
    table[2] = 1 + mp + np.arange(mp)
    pc.table.copy_(torch.from_numpy(table))
    for b, n in enumerate(lengths):
        W.append_flush(ca.sequence(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(), t16,
                       n_before=0)
        W.append_flush_paged(pc.sequence(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous(), t16,
                             n_before=[0])
    ca.seq_n, pc.seq_n = list(lengths), list(lengths)
    P = W.decode_num_splits(ca, cap, w.num_q_heads, 0)
    ks = torch.stack([k[b, :, n:n + 1] for b, n in enumerate(lengths)]).contiguous()
    vs = torch.stack([v[b, :, n:n + 1] for b, n in enumerate(lengths)]).contiguous()
    W.append_flush_ragged(ca, ks, vs, t16)
    W.append_flush_paged(pc, ks, vs, t16)
    q = gen.queries(w, 0, 0, "cuda")
    oa, _ = W.decode_attention_ragged(ca, q, t_inv_t=tinvt, num_splits=P)
    op, _ = W.decode_attention_paged(pc, q, t_inv_t=tinvt, num_splits=P)
    torch.cuda.synchronize()
    assert torch.equal(oa[0], op[0]) and torch.equal(oa[2], op[2])
    assert torch.isfinite(op[1]).all()                      # read from page 0: defined, just not this sequence's
    H, rb = w.num_kv_heads, _row_bytes(spec)
    for p, r in rb.items():
        pool = pc.planes[p].cpu().numpy()[: npages * H * PAGE * r].reshape(npages, H, PAGE, r)
        assert not pool[0].any(), p                          # nothing was written through an invalid entry
