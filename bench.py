"""Benchmark of the WUSH-KV online path on one MI355X.

A step is one decode step of the batched-serving workload (32 sequences of
32768 tokens, 32 query / 8 KV heads, head_dim 128, 2-bit percentile-clipped
affine K and V, sink 64 / recent 256 / chunk 16): append one token to every
sequence (flushing 16 tokens every 16th step), then GQA decode attention over the
whole cache with the query transform folded into its prologue.  The headline value is decode
attention GB/s: algorithmic bytes the decode must move (codes, parameters, FP16
windows, q, q~, out) per step over the step time.  Before the warm-up steps the
decode is launched untimed for a fraction of a second so that the timed steps run at
the chip's steady clocks.  Further legs time the bulk prefill flush (36 layers x 8 KV
heads x 65536 tokens) at 2, 3 and 4 bits, the long-context decode (8 sequences of
131072 tokens, 64 query / 8 KV heads, 2-bit K / 3-bit V), the calibration sums of one
layer (128 sequences of 1024 tokens), and the CPU oracle on a bounded sample of the
decode step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-flush] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)




# kernel sources each counter summary depends on
COUNTER_SOURCES = {
    "decode": ("decode_fast.hip", "decode_generic.hip", "wushkv_internal.h"),
    "flush": ("append_flush.hip", "wushkv_internal.h"),
    "calib": ("calib.hip", "wushkv_internal.h"),
}


def kernel_source_hash(files):
    """Hash of the named kernel sources, to tell whether a committed counter summary
    was taken on the kernels as they are now."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_kv_cache_amd", "csrc")
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def decode_bytes(w, n):
    """Algorithmic bytes of one decode over n cached tokens."""
    from synth.configs import QUEST
    S, R, C, d = w.sink, w.recent, w.chunk, w.head_dim
    nq = C * (max(0, n - S - R) // C)
    pk = 1 if w.quant_k == QUEST else 2
    pv = 1 if w.quant_v == QUEST else 2
    heads = w.batch * w.num_kv_heads
    body = nq * (d * w.bits_k // 8 + d * w.bits_v // 8 + 2 * pk + 2 * pv)
    window = (n - nq) * d * 2 * 2
    qio = w.batch * w.num_q_heads * d * (2 + 4 + 4)  # q bf16, q~ f32, out f32
    return heads * (body + window) + qio


def flush_bytes(w, bits, n):
    """Algorithmic bytes of one bulk prefill flush call (one layer)."""
    S, R, C, d = w.sink, w.recent, w.chunk, w.head_dim
    nq = C * (max(0, n - S - R) // C)
    heads = w.batch * w.num_kv_heads
    read = n * d * 2 * 2
    write = nq * (2 * d * bits // 8 + 2 * 2) + (n - nq) * d * 2 * 2
    return heads * (read + write) + w.num_kv_heads * d * d * 2


def traffic_from_profile(name, kernels):
    """Measured HBM bytes per launch of `kernels` (summed) from a committed counter
    summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", name)
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    files = rec.get("source_files")
    if not files or rec.get("source_hash") != kernel_source_hash(files):
        return None
    try:
        return sum(rec["kernels"][k]["bytes_per_dispatch"] for k in kernels)
    except KeyError:
        return None


def run_decode_leg(args):
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen

    w = configs.SERVING
    dev = "cuda"
    n0 = w.context
    n_breakdown = args.steps
    total = n0 + args.warmup + args.steps + n_breakdown
    log(f"[bench] decode workload {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} n={n0}")
    k, v = gen.kv_tensors(w, 0, total, dev)
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.to(dev), tinvt.to(dev)
    spec = W.CacheSpec(batch=w.batch, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, capacity=total,
                       sink=w.sink, recent=w.recent, chunk=w.chunk, bits_k=w.bits_k, bits_v=w.bits_v,
                       quant_k=W.Q_AFFINE, quant_v=W.Q_AFFINE, pct_lo=w.pct_lo, pct_hi=w.pct_hi)
    cache = W.KVCache(spec, dev)
    W.append_flush(cache, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous(), t16)
    nsteps = args.warmup + args.steps + n_breakdown
    steps_k = [k[:, :, n0 + i:n0 + i + 1].contiguous() for i in range(nsteps)]
    steps_v = [v[:, :, n0 + i:n0 + i + 1].contiguous() for i in range(nsteps)]
    del k, v
    qs = [gen.queries(w, 0, i, dev) for i in range(nsteps)]
    qt = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    out = torch.empty_like(qt)
    P = W.decode_num_splits(cache, total, w.num_q_heads, 0)
    ws = W.decode_workspace(cache, total, w.num_q_heads, P)
    torch.cuda.synchronize()
    log(f"[bench] prefill done; splits={P}")

    def step(i):
        # one decode step in one call: append (fused into the decode kernel), flush when
        # due, decode with the query transform
        W.decode_step(cache, steps_k[i], steps_v[i], t16, qs[i], tinvt, q_t=qt, num_splits=P, workspace=ws, out=out)


    # Settle: after idle the chip runs the first few dozen decodes fast, then slower for
    # ~150 launches while its power management adjusts, then steadily.  Decode-only
    # launches (the cache does not grow) for at least settle_s seconds before the
    # warm-up steps put the timed region in the steady state.
    t_settle = time.perf_counter()
    n_settle = 0
    while n_settle < 300 or time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            W.decode_attention_fused(cache, qs[n_settle % nsteps], tinvt, num_splits=P, workspace=ws, out=out, q_t=qt)
        n_settle += 50
        torch.cuda.synchronize()
    log(f"[bench] settle: {n_settle} decode launches in {time.perf_counter() - t_settle:.2f} s")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K whole steps, wall clock between two synchronizations (no events
    # inside: each event record costs the GPU a few microseconds)
    n_start = cache.n
    t0 = time.perf_counter()
    for j in range(args.steps):
        step(args.warmup + j)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    nbytes = sum(decode_bytes(w, n_start + j + 1) for j in range(args.steps)) / args.steps
    # K further steps with HIP events (on the library's stream, torch's current one)
    # around each call.  A step with no flush due is one launch, the decode kernel with
    # the append fused: its average is the kernel's launch duration for the roofline.
    # Steps with a flush due add the flush kernel.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_breakdown)]
    n_ev = cache.n
    for j in range(n_breakdown):
        evs[j][0].record()
        step(args.warmup + args.steps + j)
        evs[j][1].record()
    torch.cuda.synchronize()

    def q_of(nn):
        return w.chunk * (max(0, nn - w.sink - w.recent) // w.chunk)

    flush_due = [q_of(n_ev + j + 1) > q_of(n_ev + j) for j in range(n_breakdown)]
    plain = [e[0].elapsed_time(e[1]) for e, f in zip(evs, flush_due) if not f]
    with_flush = [e[0].elapsed_time(e[1]) for e, f in zip(evs, flush_due) if f]
    dec_ms = sum(plain) / len(plain)
    flush_ms = sum(with_flush) / len(with_flush) if with_flush else float("nan")
    kern_bytes = sum(decode_bytes(w, n_ev + j + 1) for j, f in enumerate(flush_due) if not f) / len(plain)
    log(f"[bench] step {ms_step:.4f} ms; with events around each call: {dec_ms:.4f} ms with no flush due "
        f"({len(plain)} steps, {kern_bytes / (dec_ms * 1e-3) / 1e9:.0f} GB/s), {flush_ms:.4f} ms with one "
        f"({len(with_flush)} steps); decode bytes {nbytes / 1e6:.1f} MB")
    return dict(workload=w, ms_step=ms_step, dec_ms=dec_ms, flush_step_ms=flush_ms, n_flush=len(with_flush),
                n_plain=len(plain), bytes=nbytes, splits=P, n=n_start, cache=cache, kern_ms=dec_ms,
                kern_bytes=kern_bytes)


def run_flush_leg(args):
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen

    w = configs.BULK_FLUSH
    dev = "cuda"
    n = w.context
    layers = w.layers
    log(f"[bench] bulk flush workload {w.name}: {layers} layers x Hkv={w.num_kv_heads} x {n} tokens")
    kv = [gen.kv_tensors(w, l, n, dev) for l in range(layers)]
    tks = [gen.key_transforms(w, l)[0].to(dev) for l in range(layers)]
    res = {}
    bits_list = [int(b) for b in args.flush_bits.split(",")] if args.flush_bits else list(w.flush_bits)
    had_res = None
    for bits in bits_list:
        spec = W.CacheSpec(batch=1, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, capacity=n,
                           sink=w.sink, recent=w.recent, chunk=w.chunk, bits_k=bits, bits_v=bits,
                           quant_k=W.Q_QUEST, quant_v=W.Q_QUEST)
        caches = [W.KVCache(spec, dev) for _ in range(layers)]
        for rep in range(2):  # first pass warms up
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(layers):
                W.append_flush(caches[l], kv[l][0], kv[l][1], tks[l], n_before=0)
            e1.record()
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        nbytes = layers * flush_bytes(w, bits, n)
        # the T_K contraction: 2 d^2 flop per flushed key row, on fp16 MFMA (dense peak 2.5 PFLOP/s)
        rows = layers * w.num_kv_heads * (w.chunk * (max(0, n - w.sink - w.recent) // w.chunk))
        tflops = 2 * w.head_dim ** 2 * rows / (ms * 1e-3) / 1e12
        res[bits] = dict(ms=ms, tokens_per_s=n / (ms * 1e-3), gbs=nbytes / (ms * 1e-3) / 1e9,
                         bytes=nbytes, bytes_layer=flush_bytes(w, bits, n), mfma_tflops=tflops)
        log(f"[bench] flush {bits}-bit: {ms:.3f} ms for {layers} layers -> {n / (ms * 1e-3):.3e} tokens/s, "
            f"{nbytes / (ms * 1e-3) / 1e9:.1f} GB/s")
        if bits == 2 and args.hadamard:
            # the fixed Hadamard key transform: in-register butterflies vs the same matrix,
            # fp16(H / sqrt(d)), through the dense contraction
            import numpy as np

            from synth import transforms as TR
            th = TR.as_inputs(TR.per_head(TR.hadamard(w.head_dim), w.num_kv_heads))[0].to(dev)
            scale = float(np.float16(1.0 / np.sqrt(w.head_dim)))
            hms = {}
            for name, f in (("fwht", lambda c, l: W.append_flush_hadamard(c, kv[l][0], kv[l][1], scale, n_before=0)),
                            ("dense_hadamard", lambda c, l: W.append_flush(c, kv[l][0], kv[l][1], th, n_before=0))):
                for rep in range(2):
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for l in range(layers):
                        f(caches[l], l)
                    e1.record()
                    torch.cuda.synchronize()
                hms[name] = e0.elapsed_time(e1)
            res["hadamard"] = hms
            log(f"[bench] flush 2-bit with the Hadamard key transform: in-register FWHT {hms['fwht']:.3f} ms, "
                f"the same matrix through the contraction {hms['dense_hadamard']:.3f} ms for {layers} layers")
        had_res = res.pop("hadamard", had_res)
        del caches
    del kv
    torch.cuda.empty_cache()
    if had_res:
        res["hadamard"] = had_res
    return res


def configs_name(attr):
    from synth import configs
    return getattr(configs, attr).name


def run_long_leg(args):
    """Decode calls on the long-context workload (8 sequences of 131072 tokens, 64 query /
    8 KV heads, affine 2-bit K / 3-bit V), launched back to back: at 128 splits, the
    configuration's own count, and at the count the library picks."""
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen

    w = configs.LONG_CONTEXT
    dev = "cuda"
    n = w.context + 1
    log(f"[bench] long-context workload {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} n={n}")
    k, v = gen.kv_tensors(w, 0, n, dev)
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.to(dev), tinvt.to(dev)
    spec = W.CacheSpec(batch=w.batch, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, capacity=n,
                       sink=w.sink, recent=w.recent, chunk=w.chunk, bits_k=w.bits_k, bits_v=w.bits_v,
                       quant_k=W.Q_AFFINE, quant_v=W.Q_AFFINE, pct_lo=w.pct_lo, pct_hi=w.pct_hi)
    cache = W.KVCache(spec, dev)
    W.append_flush(cache, k[:, :, :n - 1].contiguous(), v[:, :, :n - 1].contiguous(), t16)
    W.append_flush(cache, k[:, :, n - 1:].contiguous(), v[:, :, n - 1:].contiguous(), t16)
    del k, v
    q = gen.queries(w, 0, 0, dev)
    nbytes = decode_bytes(w, cache.n)
    out = {}
    for label, P in (("splits_128", 128), ("library_splits", 0)):
        splits = W.decode_num_splits(cache, cache.n, w.num_q_heads, P)
        ws = W.decode_workspace(cache, cache.n, w.num_q_heads, P)
        o = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        qt = torch.empty_like(o)
        f = lambda: W.decode_attention_fused(cache, q, tinvt, num_splits=P, workspace=ws, out=o, q_t=qt)
        t0 = time.perf_counter()   # settle, as in the decode leg
        while time.perf_counter() - t0 < args.settle_s:
            for _ in range(20):
                f()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        out[label] = {"splits": splits, "us_per_call": round(us, 2), "GB_per_s": round(gbs, 1),
                      "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"[bench] long-context decode, {splits} splits: {us:.1f} us per call ({gbs:.0f} GB/s)")
    out["bytes_per_call"] = int(nbytes)
    out["note"] = ("splits = KV partitions requested; on the MFMA path a request above the resident decode "
                   "waves per KV head (32 here) has each wave walk consecutive logical partitions' tokens "
                   "instead of running extra rounds of workgroups (the same attention, coarser partials)")
    del cache
    torch.cuda.empty_cache()
    return out


def run_graph_leg(args):
    """The launch-bound decode step of one sequence of an 8B-class layer (32 query / 8 KV
    heads, 8192 cached tokens, QuEST 2-bit K and V, chunk 8): append + flush + decode with
    the query transform, per step, launched eagerly with host-side counts, eagerly with
    device-resident counts, and as one recorded graph replayed once per step."""
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen

    w = configs.LAYER_8B
    dev = "cuda"
    n0, warm, steps = w.context, 16, 256
    cap = n0 + 6 * (warm + steps) + 1
    k, v = gen.kv_tensors(w, 0, n0 + 1, dev)
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.to(dev), tinvt.to(dev)
    spec = W.CacheSpec(batch=1, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, capacity=cap, sink=w.sink,
                       recent=w.recent, chunk=w.chunk, bits_k=w.bits_k, bits_v=w.bits_v, quant_k=W.Q_QUEST,
                       quant_v=W.Q_QUEST, clip_mult=w.clip_mult)
    cache = W.KVCache(spec, dev)
    W.append_flush(cache, k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous(), t16)
    ks, vs = k[:, :, n0:n0 + 1].contiguous(), v[:, :, n0:n0 + 1].contiguous()
    q = gen.queries(w, 0, 0, dev)
    Hq = w.num_q_heads
    P = W.decode_num_splits(cache, cap, Hq, 0)
    ws = W.decode_workspace(cache, cap, Hq, P)
    o = torch.empty(1, Hq, w.head_dim, dtype=torch.float32, device=dev)
    qt = torch.empty_like(o)
    counts = torch.tensor([n0], dtype=torch.int32, device=dev)

    def host_step():
        W.append_flush(cache, ks, vs, t16)
        W.decode_attention_fused(cache, q, tinvt, num_splits=P, workspace=ws, out=o, q_t=qt)

    def device_step():
        W.append_flush_device(cache, counts, ks, vs, t16)
        W.decode_attention_device(cache, counts, cap, q, t_inv_t=tinvt, q_t=qt, num_splits=P, workspace=ws, out=o)

    def fused_host_step():
        W.decode_step(cache, ks, vs, t16, q, tinvt, q_t=qt, num_splits=P, workspace=ws, out=o)

    def fused_device_step():
        W.decode_step_device(cache, counts, cap, ks, vs, t16, q, tinvt, q_t=qt, num_splits=P, workspace=ws, out=o)

    def timed(f):
        for _ in range(warm):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    host_us = timed(host_step)
    fused_us = timed(fused_host_step)
    counts.fill_(cache.n)
    dev_us = timed(device_step)
    fdev_us = timed(fused_device_step)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device_step()
    graph_us = timed(g.replay)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        fused_device_step()
    graph_fused_us = timed(g2.replay)
    n_end = int(counts.item())
    log(f"[bench] 8B-layer decode step ({w.name}, n {n0} -> {n_end}): eager {host_us:.1f} us (fused step "
        f"{fused_us:.1f}), eager with device counts {dev_us:.1f} us (fused {fdev_us:.1f}), graph replay "
        f"{graph_us:.1f} us (fused {graph_fused_us:.1f})")
    out = {"workload": w.name, "context_start": n0, "steps_timed": steps, "splits": P,
           "eager_host_counts_us": round(host_us, 2), "eager_fused_step_us": round(fused_us, 2),
           "eager_device_counts_us": round(dev_us, 2), "eager_fused_device_step_us": round(fdev_us, 2),
           "graph_replay_us": round(graph_us, 2), "graph_replay_fused_us": round(graph_fused_us, 2),
           "bytes_per_decode": int(decode_bytes(w, n0)),
           "note": "append + flush (when due) + decode with the query transform, per step: as separate calls "
                   "(append_flush then decode) or one fused call (decode_step / decode_step_device); 6 x (16 + "
                   "256) steps past the prefill"}
    del cache
    torch.cuda.empty_cache()
    return out


def run_paged_leg(args):
    """The batched-serving decode (32 sequences x 32768 tokens, 32/8 heads, affine 2/2)
    on a paged body beside the contiguous cache: 256-token pages, each sequence's pages
    scattered over the pool in a seeded random order.  The two are timed alternately
    (fused decode with the library's split count), and their outputs must be equal."""
    import numpy as np
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen

    w = configs.SERVING
    n, page = w.context, 256
    k, v = gen.kv_tensors(w, 0, n, "cuda")
    t16, tinvt = gen.key_transforms(w, 0)
    t16, tinvt = t16.cuda(), tinvt.cuda()
    spec = W.CacheSpec(batch=w.batch, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, capacity=n, sink=w.sink,
                       recent=w.recent, chunk=w.chunk, bits_k=w.bits_k, bits_v=w.bits_v, quant_k=W.Q_AFFINE,
                       quant_v=W.Q_AFFINE, pct_lo=w.pct_lo, pct_hi=w.pct_hi)
    ca = W.KVCache(spec, "cuda")
    W.append_flush(ca, k, v, t16)
    body = -(-(n - w.sink) // 64) * 64
    mp = -(-body // page)
    pc = W.PagedKVCache(spec, page, w.batch * mp, max_pages=mp)
    perm = np.random.default_rng(7).permutation(w.batch * mp).reshape(w.batch, mp).astype(np.int32)
    pc.table.copy_(torch.from_numpy(perm))
    W.append_flush_paged(pc, k, v, t16, n_before=[0] * w.batch)
    del k, v
    q = gen.queries(w, 0, 0, "cuda")
    Hq = w.num_q_heads
    P = W.decode_num_splits(ca, n, Hq, 0)
    ws = W.decode_workspace(ca, n, Hq, P)
    oc = torch.empty(w.batch, Hq, w.head_dim, dtype=torch.float32, device="cuda")
    op, qc, qp = torch.empty_like(oc), torch.empty_like(oc), torch.empty_like(oc)
    lens = [n] * w.batch
    fc = lambda: W.decode_attention_ragged(ca, q, q_t=qc, t_inv_t=tinvt, n_tokens=lens, num_splits=P, workspace=ws,
                                           out=oc)
    fp = lambda: W.decode_attention_paged(pc, q, q_t=qp, t_inv_t=tinvt, n_tokens=lens, num_splits=P, workspace=ws,
                                          out=op)
    fc()
    fp()
    torch.cuda.synchronize()
    same = bool(torch.equal(oc, op))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(10):
            fc()
            fp()
        torch.cuda.synchronize()
    res = {"contiguous": [], "paged": []}
    for _ in range(6):
        for name, f in (("contiguous", fc), ("paged", fp)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                f()
            e1.record()
            torch.cuda.synchronize()
            res[name].append(e0.elapsed_time(e1) / 20 * 1e3)
    med = {k2: float(np.median(v2)) for k2, v2 in res.items()}
    log(f"[bench] paged serving decode ({page}-token pages, {mp} per sequence, scattered): paged "
        f"{med['paged']:.1f} us, contiguous {med['contiguous']:.1f} us per call (medians), outputs equal: {same}")
    del ca, pc
    torch.cuda.empty_cache()
    return {"page_tokens": page, "pages_per_sequence": mp, "splits": P, "outputs_equal": same,
            "paged_us_per_call": round(med["paged"], 2), "contiguous_us_per_call": round(med["contiguous"], 2),
            "note": "ragged-call decode with the query transform fused, alternated 6 x 20 calls, medians"}


def run_transform_leg(args):
    """Module-output error of the path under different key transforms, on synthetic
    attention modules: 8 modules (layers) of 4 sequences x 1024 tokens, 32 query / 8 KV
    heads, d = 128, bf16 keys with outlier channels under per-head covariance.  Each
    module is prefilled through the library with T_K = identity, the orthonormal
    Hadamard matrix, the workloads' random dense transform, or Gram whitening (from the
    library's calibration sums over held-out keys of the same heads), then decoded for 16
    queries per sequence.  The error is the relative Frobenius error of the attention
    outputs against full-precision attention over the unquantized keys and values (fp32
    on the GPU), summarized over the modules by a geometric mean.  Synthetic data: the
    figures show the transforms' effect on such data, not on a trained model."""
    import numpy as np
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen
    from synth import transforms as TR

    base = configs.SERVING.scaled(batch=4, context=1024)
    n, nq, modules = 1024, 16, 8
    d, H, G = base.head_dim, base.num_kv_heads, base.group
    settings = [("affine", 2), ("quest", 2), ("quest", 3), ("quest", 4)]
    kinds = ["identity", "hadamard", "dense", "whitening"]
    errs = {(k, s): [] for k in kinds for s in settings}
    t0 = time.perf_counter()
    for layer in range(modules):
        k, v = gen.kv_tensors(base, layer, n, "cuda")
        qs = torch.stack([gen.queries(base, layer, s, "cuda") for s in range(nq)])       # [nq, B, Hq, d]
        # full-precision reference: per KV head its G query heads over all n tokens
        qg = qs.float().reshape(nq, base.batch, H, G, d).permute(1, 2, 0, 3, 4).reshape(base.batch, H, nq * G, d)
        kf, vf = k.float(), v.float()
        sc = torch.matmul(qg, kf.transpose(-1, -2).contiguous()) / np.sqrt(d)
        ref = torch.matmul(torch.softmax(sc, dim=-1), vf)                                  # [B, H, nq*G, d]
        ref = ref.reshape(base.batch, H, nq, G, d).permute(2, 0, 1, 3, 4).reshape(nq, base.batch, H * G, d)
        held = torch.stack([torch.stack([gen.kv_block(base, layer, base.batch + b, g, n, "cuda")[0]
                                         for g in range(H)]) for b in range(base.batch)]).contiguous()
        gram = W.calib_stats(held, 1).double().cpu().numpy()
        trans = {"identity": TR.as_inputs(TR.per_head(np.eye(d), H)),
                 "hadamard": TR.as_inputs(TR.per_head(TR.hadamard(d), H)),
                 "dense": gen.key_transforms(base, layer),
                 "whitening": TR.as_inputs(np.stack([TR.whitening(gram[g], base.batch * n) for g in range(H)]))}
        for kind in kinds:
            t16, tinvt = trans[kind][0].cuda(), trans[kind][1].cuda()
            for quant, bits in settings:
                qc = W.Q_AFFINE if quant == "affine" else W.Q_QUEST
                spec = W.CacheSpec(batch=base.batch, num_kv_heads=H, head_dim=d, capacity=n, sink=base.sink,
                                   recent=base.recent, chunk=base.chunk, bits_k=bits, bits_v=bits, quant_k=qc,
                                   quant_v=qc, clip_mult=base.clip_mult, pct_lo=base.pct_lo, pct_hi=base.pct_hi)
                cache = W.KVCache(spec, "cuda")
                W.append_flush(cache, k, v, t16)
                out = torch.stack([W.decode_attention_fused(cache, qs[s], tinvt)[0] for s in range(nq)])
                e = float(torch.linalg.vector_norm((out - ref).double()) / torch.linalg.vector_norm(ref.double()))
                errs[(kind, (quant, bits))].append(e)
    res = {}
    for (kind, (quant, bits)), e in errs.items():
        res.setdefault(f"{quant}_{bits}bit", {})[kind] = round(float(np.exp(np.mean(np.log(e)))), 4)
    log(f"[bench] module-output error (geometric mean over {modules} synthetic modules, "
        f"{time.perf_counter() - t0:.1f} s): " + "; ".join(f"{s}: " + ", ".join(f"{k} {v:.3f}" for k, v in r.items())
                                                      for s, r in res.items()))
    res["note"] = ("synthetic modules: 4 sequences x 1024 tokens, 8 KV heads, 16 decode queries each; relative "
                   "Frobenius error of the attention outputs vs full precision, geometric mean over 8 modules; "
                   "whitening = (key second moment)^(-1/2) from held-out keys, Frobenius-normalized (not the "
                   "pages' WUSH construction)")
    return res


def run_calib_leg(args):
    """Calibration sums of one layer of the calibration workload (128 sequences x 1024
    tokens, 8 KV / 32 query heads): key Gram, value Gram and the key Hessian (query heads
    grouped by KV head), each timed over back-to-back calls after a settle."""
    import torch

    import bit_kv_cache_amd as W
    from synth import configs, gen

    w = configs.CALIB
    dev = "cuda"
    T = w.context
    log(f"[bench] calibration workload {w.name}: {w.batch} sequences x {T} tokens, Hkv={w.num_kv_heads} Hq={w.num_q_heads}")
    k, v = gen.kv_tensors(w, 0, T, dev)
    q = gen.calib_queries(w, 0, T, dev)
    res = {}
    total_bytes, total_flop, total_us = 0, 0, 0.0
    legs = [(name, x, group) for name, x, group in (("key_gram", k, 1), ("value_gram", v, 1),
                                                     ("key_hessian", q, w.group))
            if name in args.calib_legs.split(",")]
    for name, x, group in legs:
        B, H, _, d = x.shape
        ws = W.calib_workspace(B, H, T, d, group, dev)
        out = torch.empty((H // group, d, d), dtype=torch.float32, device=dev)
        f = lambda: W.calib_stats(x, group, workspace=ws, out=out)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle_s:
            for _ in range(10):
                f()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 30
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        nbytes = x.numel() * x.element_size() + out.numel() * 4
        flop = 2 * B * H * T * d * d
        res[name] = {"us_per_call": round(us, 2), "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "TFLOP_per_s": round(flop / (us * 1e-6) / 1e12, 1), "bytes": int(nbytes), "flop": int(flop)}
        total_bytes += nbytes
        total_flop += flop
        total_us += us
        log(f"[bench] calib {name}: {us:.1f} us ({nbytes / (us * 1e-6) / 1e9:.0f} GB/s, "
            f"{flop / (us * 1e-6) / 1e12:.0f} TFLOP/s)")
    res["layer"] = {"us": round(total_us, 2), "GB_per_s": round(total_bytes / (total_us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(total_bytes / (total_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "TFLOP_per_s": round(total_flop / (total_us * 1e-6) / 1e12, 1)}
    kg = res.get("key_gram")
    if kg is not None:
        achieved = kg["bytes"] / (kg["us_per_call"] * 1e-6) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": traffic_from_profile("calib_key_gram_counters.json",
                                                           ["calib_partial_kernel<true>", "calib_reduce_kernel"]),
                           "kernel": "calib_partial_kernel<true> + calib_reduce_kernel on the key Gram (bf16 "
                                     "keys, group 1): bytes = keys read + fp32 output written, per call"}
    del k, v, q
    torch.cuda.empty_cache()
    return res


def summarize_counters(fetch_csv, write_csv, copy_mib):
    """Per-dispatch HBM bytes of the library's kernels from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the fp32 -> fp64 copy of --copy-check (its bytes are known)."""
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            if "wushkv" in name:
                acc[name.replace("void ", "").replace("wushkv::(anonymous namespace)::", "").split("(")[0]].append(val)
            elif "copy" in name and "double" in name:
                copy.append(val)
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}, copy

    fetch, nf, cf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw, cw = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib << 20          # read by the fp32 -> fp64 copy; it writes twice that
    if not cf or not cw:
        raise SystemExit("no fp32 -> fp64 copy-check dispatches in the counter files (run with --copy-check)")
    ff = copy_bytes / (sum(cf) / len(cf) * 1024)
    wf = 2 * copy_bytes / (sum(cw) / len(cw) * 1024)
    kernels = {}
    for k in sorted(fetch):
        kernels[k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write.get(k, 0.0), 1),
                      "dispatches": nf[k],
                      "bytes_per_dispatch": int(fetch[k] * 1024 * ff + write.get(k, 0.0) * 1024 * wf)}
    return {"calibration": {"copy_read_bytes": copy_bytes, "copy_write_bytes": 2 * copy_bytes,
                            "copy_fetch_kib": round(sum(cf) / len(cf), 1),
                            "copy_write_kib": round(sum(cw) / len(cw), 1), "fetch_factor": round(ff, 5),
                            "write_factor": round(wf, 5), "copy_dispatches": len(cf)},
            "kernels": kernels}


def summarize_pmc(csv_path):
    """Every counter of a rocprofv3 --pmc counter_collection.csv, averaged per dispatch of
    each of the library's kernels (grouped by kernel and grid), as a text table; with the
    SQ_* counters also the derived per-wave instruction counts and busy fractions."""
    import csv
    import collections

    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"]
        if "wushkv" not in name:
            continue
        name = name.replace("void ", "").replace("wushkv::(anonymous namespace)::", "").split("(")[0]
        acc[(name, r["Grid_Size"], r["Workgroup_Size"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = []
    for (name, grid, wg), cs in sorted(acc.items()):
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        lines.append(f"{name}  grid {grid}  workgroup {wg}  ({n} dispatches)")
        for c in sorted(mean):
            lines.append(f"    {c:28s} {mean[c]:16.1f}")
        waves = mean.get("SQ_WAVES")
        if waves:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
                if c in mean:
                    lines.append(f"    {c + ' per wave':28s} {mean[c] / waves:16.1f}")
        if mean.get("SQ_BUSY_CYCLES") and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            lines.append(f"    {'MFMA busy / SQ busy':28s} {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / mean['SQ_BUSY_CYCLES']:16.4f}")
        if mean.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in mean:
            lines.append(f"    {'LDS conflict cycles / LDS op':28s} "
                         f"{mean['SQ_LDS_BANK_CONFLICT'] / mean['SQ_INSTS_LDS']:16.3f}")
    return "\n".join(lines)


def summarize_trace(trace_csv):
    """Library kernels of a rocprofv3 kernel-trace CSV grouped by (kernel, grid, workgroup
    size): the legs of this bench launch distinct grids.  Durations in microseconds."""
    import csv
    import collections
    import statistics

    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        if "wushkv" not in name:
            continue
        name = name.replace("void ", "").replace("wushkv::(anonymous namespace)::", "").replace("wushkv::", "")
        key = (name.split("(")[0], f'{r["Grid_Size_X"]},{r["Grid_Size_Y"]},{r["Grid_Size_Z"]}', r["Workgroup_Size_X"])
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = [f"{'kernel':34s} {'grid x,y,z':>22s} {'wg':>5s} {'calls':>6s} {'avg':>9s} {'median':>9s} {'min':>9s}"]
    for key in sorted(groups, key=lambda k: -sum(groups[k])):
        v = groups[key]
        lines.append(f"{key[0]:34s} {key[1]:>22s} {key[2]:>5s} {len(v):6d} {sum(v) / len(v):9.2f} "
                     f"{statistics.median(v):9.2f} {min(v):9.2f}")
    return "\n".join(lines)


def _cpu_flush_worker_init(barrier):
    global _CPU_BARRIER
    _CPU_BARRIER = barrier


def _cpu_flush_worker(job):
    """One (layer, KV head) block of the bulk flush through the oracle, single-threaded:
    the key transform, quantization and packing of its 65216 body rows (plus its FP16
    windows).  Inputs are generated first, untimed; all workers start timing together."""
    layer, head, bits = job
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import layout as LY
    from oracle import wushkv_ref as R
    from synth import configs, gen
    w = configs.BULK_FLUSH
    k, v = gen.kv_block(w, layer, 0, head, w.context, "cpu")
    k = k.float().numpy().astype(np.float64)
    v = v.float().numpy().astype(np.float64)
    t16 = gen.key_transforms(w, layer)[0][head].numpy()
    with threadpool_limits(limits=1):
        _CPU_BARRIER.wait()
        t0 = time.perf_counter()
        c = R.build_head_cache(k, v, t16, w.context, sink=w.sink, recent=w.recent, chunk=w.chunk, quant_k="quest",
                               quant_v="quest", bits_k=bits, bits_v=bits, clip_mult=w.clip_mult)
        LY.pack_k(c.codes_k, bits)
        LY.pack_v(c.codes_v, bits)
        t1 = time.perf_counter()
    return t0, t1


def _cpu_decode_worker(job):
    """The oracle's decode step for the G query heads of one (batch row, KV head) pair of
    the batched-serving workload, single-threaded: its cache is built first (untimed), then
    query transform + decode are repeated for `seconds`; returns (reps, seconds)."""
    b, g, n, seconds = job
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import wushkv_ref as R
    from synth import configs, gen
    w = configs.SERVING
    t16 = gen.key_transforms(w, 0)[0][g].numpy()
    kb, vb = gen.kv_block(w, 0, b, g, n, "cpu")
    kb, vb = kb.float().numpy().astype(np.float64), vb.float().numpy().astype(np.float64)
    c = R.build_head_cache(kb, vb, t16, n, sink=w.sink, recent=w.recent, chunk=w.chunk, quant_k=w.quant_k,
                           quant_v=w.quant_v, bits_k=w.bits_k, bits_v=w.bits_v, pct_lo=w.pct_lo, pct_hi=w.pct_hi)
    q = gen.queries(w, 0, 0, "cpu").float().numpy().astype(np.float64)
    with threadpool_limits(limits=1):
        _CPU_BARRIER.wait()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < seconds:
            for h in range(g * w.group, (g + 1) * w.group):
                R.decode_head(c, q[b, h], R.query_transform(t16, q[b, h]))
            reps += 1
        return reps, time.perf_counter() - t0


def run_cpu_decode_leg(cores, n, seconds=8.0):
    """The oracle's decode of the batched-serving step on `cores` (batch row, KV head) pairs
    at once, one single-threaded process per core; the step time of all 256 pairs is the
    mean time per pair scaled by 256 / cores (the pairs are independent)."""
    import multiprocessing as mp

    from synth import configs
    w = configs.SERVING
    pairs = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    jobs = [(b, g, n, seconds) for b, g in pairs[:: len(pairs) // cores][:cores]]
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(len(jobs))
    with ctx.Pool(len(jobs), initializer=_cpu_flush_worker_init, initargs=(barrier,)) as pool:
        res = pool.map(_cpu_decode_worker, jobs)
    per_pair = sum(el / reps for reps, el in res) / len(res)
    step_s = per_pair * len(pairs) / len(jobs)
    return step_s, per_pair, len(jobs), sum(r for r, _ in res)


def run_cpu_flush_leg(cores, bits=2):
    """The oracle's bulk flush on `cores` (layer, KV head) blocks at once, one process per
    core (spawned, single-threaded), timed from a common start to the last finish; the full
    pass (36 layers x 8 KV heads) is that wall time scaled by 288 / blocks."""
    import multiprocessing as mp

    from synth import configs
    w = configs.BULK_FLUSH
    nb = cores
    jobs = [(l % w.layers, (3 * l) % w.num_kv_heads, bits) for l in range(nb)]
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(nb)
    with ctx.Pool(nb, initializer=_cpu_flush_worker_init, initargs=(barrier,)) as pool:
        spans = pool.map(_cpu_flush_worker, jobs)
    wall = max(t1 for _, t1 in spans) - min(t0 for t0, _ in spans)
    per_block = sum(t1 - t0 for t0, t1 in spans) / nb
    blocks = w.layers * w.num_kv_heads
    pass_s = wall * blocks / nb
    return {"value": round(w.context / pass_s, 1), "unit": "tokens/s", "cores": nb, "kind": "oracle",
            "sample": f"{nb} of {blocks} (layer, KV head) blocks of the bulk flush at {bits} bits (65536 tokens each: "
                      f"key transform, QuEST quantization and packing of 65216 body rows), one single-threaded process "
                      f"per core, {wall:.2f} s wall; the 36-layer pass scaled to {pass_s:.1f} s",
            "single_core_tokens_per_s": round(w.context / (per_block * blocks), 1),
            "single_core_note": f"one block per core in {per_block:.2f} s on average; a full pass on one core would "
                                f"take {per_block * blocks:.0f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg (profiling the flush alone)")
    ap.add_argument("--flush-bits", type=str, default="", help="comma-separated bit widths of the flush leg")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context decode leg")
    ap.add_argument("--no-hadamard", dest="hadamard", action="store_false",
                    help="skip the Hadamard key-transform timing of the flush leg")
    ap.add_argument("--no-calib", action="store_true", help="skip the calibration-statistics leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the launch-bound decode-step leg")
    ap.add_argument("--no-transforms", action="store_true", help="skip the key-transform module-error leg")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-body decode leg")
    ap.add_argument("--calib-legs", type=str, default="key_gram,value_gram,key_hessian",
                    help="comma-separated sums the calibration leg times")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed decode-only launches before the warm-up steps")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="first copy a MIB-sized device buffer three times: a plain copy of known size, whose "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the decode kernel's traffic figures")
    ap.add_argument("--counters-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: summarize two rocprofv3 counter_collection.csv files (runs made with "
                         "--copy-check MIB) as JSON on stdout")
    ap.add_argument("--counters-kernels", choices=sorted(COUNTER_SOURCES), default="decode",
                    help="which kernels' sources the counter summary is tied to")
    ap.add_argument("--pmc-summary", metavar="COUNTER_CSV",
                    help="no GPU work: average every counter of a rocprofv3 --pmc counter_collection.csv per "
                         "dispatch of each library kernel and print it")
    ap.add_argument("--trace-summary", metavar="TRACE_CSV",
                    help="no GPU work: group a rocprofv3 kernel_trace.csv by kernel and grid and print it")
    args = ap.parse_args()
    if args.pmc_summary:
        print(summarize_pmc(args.pmc_summary))
        return
    if args.trace_summary:
        print(summarize_trace(args.trace_summary))
        return
    if args.counters_summary:
        rec = summarize_counters(*args.counters_summary, args.copy_check or 1024)
        rec["source_files"] = list(COUNTER_SOURCES[args.counters_kernels])
        rec["source_hash"] = kernel_source_hash(rec["source_files"])
        print(json.dumps(rec, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every workload runs on a single MI355X); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    # the oracle's flush baseline runs first, in worker processes started before this
    # process touches the GPU (one per core of the job's share, at most 16)
    cpu_flush = cpu_decode = None
    if not args.no_cpu and not args.no_decode:
        from synth import configs as _cfg
        ncores = min(16, len(os.sched_getaffinity(0)))
        n_cpu = _cfg.SERVING.context + args.warmup + args.steps + 1   # the decode leg's context at its timed steps
        cpu_decode = run_cpu_decode_leg(ncores, n_cpu)
        log(f"[bench] cpu decode baseline: {cpu_decode[0]:.2f} s per step ({cpu_decode[2]} processes)")
        if not args.no_flush:
            cpu_flush = run_cpu_flush_leg(ncores)
            log(f"[bench] cpu flush baseline: {cpu_flush['value']} tokens/s ({cpu_flush['cores']} processes)")
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_check > 0:
        # an fp32 -> fp64 conversion copy: MIB read, 2 MIB written, by a kernel no
        # workload launches (a same-dtype copy goes through the runtime's blit path)
        n = args.copy_check << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty(n // 4, dtype=torch.float64, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy check: 3 fp32 -> fp64 copies of {n} bytes")
        del src, dst

    if args.no_decode:
        rec = {}
        if not args.no_flush:
            rec["flush"] = {f"{b}bit": r for b, r in run_flush_leg(args).items()}
        if not args.no_calib:
            rec["calibration"] = run_calib_leg(args)
        print(json.dumps(rec), flush=True)
        return
    dl = run_decode_leg(args)
    w = dl["workload"]
    fl = {} if args.no_flush else run_flush_leg(args)
    lc = {} if args.no_long else run_long_leg(args)
    cl = {} if args.no_calib else run_calib_leg(args)
    gl = {} if args.no_graph else run_graph_leg(args)
    tl = {} if args.no_transforms else run_transform_leg(args)
    pl = {} if args.no_paged else run_paged_leg(args)
    achieved = dl["kern_bytes"] / (dl["kern_ms"] * 1e-3) / 1e9
    traffic = traffic_from_profile("decode_batched_serving_counters.json", ["decode_fast_kernel<4, 2, 2, 12, false, true>"])
    value = dl["bytes"] / (dl["ms_step"] * 1e-3) / 1e9
    line = {
        "metric": "2-bit GQA decode-attention HBM GB/s (% of peak); flush tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dl["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": ("scores, softmax and accumulation in fp32; the body's q~ . c runs on fp4 x fp4 matrix cores "
                       "as exact digit products of q~ on a 22-bit fixed-point grid, and p * s_V enters the fp16 PV "
                       "product as an fp16 hi + lo pair (~22 bits); cache codes are 2-bit, windows and "
                       "parameters fp16"),
        "data": "synthetic (seeded Student-t K/V under per-head covariance, random per-head T_K)",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "context": dl["n"],
                   "quant": "percentile-clipped affine 2-bit K and V", "sink": w.sink, "recent": w.recent,
                   "chunk": w.chunk, "splits": dl["splits"], "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_breakdown_ms": {"step_no_flush": round(dl["dec_ms"], 5), "step_with_flush": round(dl["flush_step_ms"], 5),
                              "steps_no_flush": dl["n_plain"], "steps_with_flush": dl["n_flush"],
                              "note": "a step is one wushkv_decode_step call: the new token's append fused into "
                                      "the decode kernel, plus the flush kernel when a chunk is due; HIP-event "
                                      "intervals around each call over K further steps"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_fast_kernel<4,2,2,12>: GQA decode with the query transform in its "
                               "prologue and the new token's append fused, one 12-wave workgroup per KV head "
                               "(12 splits, merged in LDS); duration from the steps with no flush due",
                     "bytes_per_launch": int(dl["kern_bytes"]), "us_per_launch": round(dl["kern_ms"] * 1e3, 2)},
    }
    had = fl.pop("hadamard", None) if fl else None
    w_flush_tokens = 65536
    if fl:
        line["flush"] = {f"{b}bit": {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_36_layers": round(r["ms"], 3),
                                     "GB_per_s": round(r["gbs"], 1), "frac_hbm": round(r["gbs"] / HBM_PEAK_GBS, 4),
                                     "key_transform_TFLOP_per_s": round(r["mfma_tflops"], 1),
                                     "key_transform_mfma_util": round(r["mfma_tflops"] / MFMA_F16_PEAK_TFLOPS, 4)}
                         for b, r in fl.items()}
        if 2 in fl:
            # HBM bytes per append_flush call (one layer) from the committed counter summary,
            # beside the call's algorithmic bytes
            # (one launch per layer: the same flush kernel also writes the window rows)
            ft = traffic_from_profile("flush_bulk_counters.json", ["flush_kernel<128, 2, 0, false, false, true>"])
            line["flush"]["2bit"]["algorithmic_bytes_per_layer"] = fl[2]["bytes_layer"]
            line["flush"]["2bit"]["traffic_bytes_per_layer"] = ft
        if had:
            line["flush"]["hadamard_2bit"] = {
                "fwht_ms_36_layers": round(had["fwht"], 3), "dense_ms_36_layers": round(had["dense_hadamard"], 3),
                "fwht_tokens_per_s": round(w_flush_tokens / (had["fwht"] * 1e-3), 1),
                "note": "T_K = fp16(H/sqrt(d)): in-register fast Walsh-Hadamard transform "
                        "(wushkv_append_flush_hadamard) vs the same matrix through the dense matrix-core contraction; "
                        "bit-identical caches"}
        line["flush"]["note"] = ("36 x append_flush(n_before=0, n_new=65536) of 8 KV heads, QuEST K and V; the key "
                                 "transform T_K k on v_mfma_f32_16x16x32_f16, 2 d^2 flop per body row, against the "
                                 "2.5 PFLOP/s dense fp16 peak (the flush is HBM-bound; at its HBM roofline the "
                                 "matrix cores would be ~18% busy)")
    if lc:
        line["long_context"] = dict(lc, workload=configs_name("LONG_CONTEXT"),
                                    quant="percentile-clipped affine 2-bit K / 3-bit V")
    if gl:
        line["decode_step_graph"] = gl
    if tl:
        line["transform_module_error"] = tl
    if pl:
        line["paged_decode"] = pl
    if cl:
        line["calibration"] = dict(cl, workload=configs_name("CALIB"),
                                   note="bf16 rows; out[g] = sum of x x^T; flop counted as 2 N d^2 per head")
    if not args.no_cpu:
        step_s, per_pair, nproc, reps = cpu_decode
        cb = {"value": round(dl["bytes"] / step_s / 1e9, 4), "unit": "GB/s", "cores": nproc, "kind": "oracle",
              "sample": f"{nproc} of {w.batch * w.num_kv_heads} (batch row, KV head) pairs x {w.group} query heads "
                        f"at the decode leg's context, one single-threaded process per core, query transform + "
                        f"decode repeated for 8 s each ({reps} pair-steps, {per_pair * 1e3:.1f} ms per pair); the "
                        f"step over all pairs scaled to {step_s:.3f} s",
              "single_core": {"value": round(dl["bytes"] / (per_pair * w.batch * w.num_kv_heads) / 1e9, 4),
                              "unit": "GB/s", "cores": 1,
                              "note": "the same pairs' mean time per pair, as if one core decoded all 256"}}
        if cpu_flush:
            cb["flush"] = cpu_flush
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
