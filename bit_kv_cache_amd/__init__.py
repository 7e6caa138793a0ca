"""Python binding of libwushkv, the MI355X (gfx950) WUSH-KV online path.

Argument marshalling only: torch provides device memory and the stream, and
every step of the path (append, flush with the key transform and quantization,
query transform, split-K GQA decode with its merge) runs in the library's HIP
kernels through the C ABI declared in include/wushkv.h.  There is no CPU
fallback: without the built library every call raises.
"""
import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwushkv.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP = range(8)
DT_F32, DT_BF16, DT_F16 = 0, 1, 2
Q_QUEST, Q_AFFINE = 0, 1
PLANES = ("sink_k", "sink_v", "ring_k", "ring_v", "codes_k", "codes_v", "par_k", "par_v")
EXPORTS = ("wushkv_status_string", "wushkv_abi_version", "wushkv_cache_check", "wushkv_plane_bytes",
           "wushkv_decode_num_splits", "wushkv_decode_workspace_bytes", "wushkv_append_flush",
           "wushkv_query_transform", "wushkv_decode_attention", "wushkv_decode_attention_fused",
           "wushkv_calib_stats", "wushkv_calib_workspace_bytes", "wushkv_append_flush_ragged",
           "wushkv_decode_attention_ragged", "wushkv_append_flush_device", "wushkv_decode_attention_device",
           "wushkv_pool_bytes", "wushkv_append_flush_paged", "wushkv_decode_attention_paged", "wushkv_decode_step",
           "wushkv_decode_step_device", "wushkv_decode_attention_generic", "wushkv_decode_attention_noalloc",
           "wushkv_append_flush_hadamard")


class WushKVError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class CacheDesc(ctypes.Structure):
    """Mirror of wushkv_cache (include/wushkv.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("sink", ctypes.c_int32), ("recent", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("bits_k", ctypes.c_int32), ("bits_v", ctypes.c_int32),
        ("quant_k", ctypes.c_int32), ("quant_v", ctypes.c_int32),
        ("clip_mult", ctypes.c_float), ("pct_lo", ctypes.c_float), ("pct_hi", ctypes.c_float),
    ] + [(p, ctypes.c_void_p) for p in PLANES]


_lib = None


def lib():
    """The loaded libwushkv (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_kv_cache_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(CacheDesc)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "wushkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "wushkv_abi_version": (ctypes.c_int, []),
            "wushkv_cache_check": (ctypes.c_int, [P]),
            "wushkv_plane_bytes": (sz, [P, ctypes.c_int]),
            "wushkv_decode_num_splits": (i32, [P, i64, i32, i32]),
            "wushkv_decode_workspace_bytes": (sz, [P, i64, i32, i32]),
            "wushkv_append_flush": (ctypes.c_int, [P, i64, i32, vp, vp, i32, vp, vp]),
            "wushkv_query_transform": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, i32, vp, vp]),
            "wushkv_decode_attention": (ctypes.c_int, [P, i64, vp, i32, vp, i32, i32, vp, sz, vp, vp]),
            "wushkv_decode_attention_fused": (ctypes.c_int, [P, i64, vp, i32, vp, vp, i32, i32, vp, sz, vp, vp]),
            "wushkv_calib_stats": (ctypes.c_int, [vp, i32, i32, i32, i64, i32, i32, vp, sz, vp, vp]),
            "wushkv_append_flush_ragged": (ctypes.c_int, [P, ctypes.POINTER(i64), i32, vp, vp, i32, vp, vp]),
            "wushkv_decode_attention_ragged": (ctypes.c_int, [P, ctypes.POINTER(i64), vp, i32, vp, vp, i32, i32, vp, sz,
                                                              vp, vp]),
            "wushkv_calib_workspace_bytes": (sz, [i32, i32, i64, i32, i32]),
            "wushkv_append_flush_device": (ctypes.c_int, [P, vp, i32, vp, vp, i32, vp, vp]),
            "wushkv_pool_bytes": (sz, [P, ctypes.POINTER(PagesDesc), ctypes.c_int]),
            "wushkv_decode_step": (ctypes.c_int, [P, i64, vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, vp, sz, vp, vp]),
            "wushkv_decode_step_device": (ctypes.c_int, [P, vp, i64, vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, vp, sz,
                                                         vp, vp]),
            "wushkv_append_flush_paged": (ctypes.c_int, [P, ctypes.POINTER(PagesDesc), ctypes.POINTER(i64), i32, vp, vp,
                                                         i32, vp, vp]),
            "wushkv_append_flush_hadamard": (ctypes.c_int, [P, i64, i32, vp, vp, i32, ctypes.c_float, vp]),
            "wushkv_decode_attention_noalloc": (ctypes.c_int, [P, i64, vp, i32, vp, i32, i32, vp, vp]),
            "wushkv_decode_attention_generic": (ctypes.c_int, [P, ctypes.POINTER(i64), vp, i32, vp, vp, i32, i32, vp,
                                                               sz, vp, vp]),
            "wushkv_decode_attention_paged": (ctypes.c_int, [P, ctypes.POINTER(PagesDesc), ctypes.POINTER(i64), vp, i32,
                                                             vp, vp, i32, i32, vp, sz, vp, vp]),
            "wushkv_decode_attention_device": (ctypes.c_int, [P, vp, i64, vp, i32, vp, vp, i32, i32, vp, sz, vp,
                                                              vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name, None)   # an older build may lack later entry points
            if fn is not None:
                fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(status):
    return lib().wushkv_status_string(int(status)).decode()


def _check(status, what):
    if status != OK:
        raise WushKVError(status, what)


_DTYPES = None


def _dtype_code(t):
    global _DTYPES
    if _DTYPES is None:
        import torch
        _DTYPES = {torch.float32: DT_F32, torch.bfloat16: DT_BF16, torch.float16: DT_F16}
    return _DTYPES[t.dtype]


def _stream(stream, device):
    """Raw HIP stream handle: the given torch stream, else torch's current stream on device."""
    if stream is not None:
        return stream.cuda_stream
    import torch
    index = device.index if device.index is not None else torch.cuda.current_device()
    return torch._C._cuda_getCurrentRawStream(index)


def _ptr(t):
    if not t.is_contiguous():
        raise ValueError("tensors passed to libwushkv must be contiguous")
    return t.data_ptr()


class PagesDesc(ctypes.Structure):
    """wushkv_pages: device page table [batch][max_pages] int32 and the page geometry."""
    _fields_ = [("table", ctypes.c_void_p), ("page_tokens", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


@dataclass
class CacheSpec:
    batch: int
    num_kv_heads: int
    head_dim: int
    capacity: int
    sink: int = 64
    recent: int = 256
    chunk: int = 8
    bits_k: int = 2
    bits_v: int = 2
    quant_k: int = Q_QUEST
    quant_v: int = Q_QUEST
    clip_mult: float = 2.5
    pct_lo: float = 0.5
    pct_hi: float = 99.5

    def desc(self, planes=None):
        d = CacheDesc(self.batch, self.num_kv_heads, self.head_dim, self.sink, self.recent, self.chunk,
                      self.capacity, self.bits_k, self.bits_v, self.quant_k, self.quant_v,
                      self.clip_mult, self.pct_lo, self.pct_hi)
        if planes:
            for p in PLANES:
                setattr(d, p, planes[p].data_ptr())
        return d

    def plane_bytes(self):
        d = self.desc()
        out = {p: int(lib().wushkv_plane_bytes(ctypes.byref(d), i)) for i, p in enumerate(PLANES)}
        if any(v == 0 and not p.startswith("sink") for p, v in out.items()):
            _check(lib().wushkv_cache_check(ctypes.byref(d)), "cache descriptor")
        return out


class KVCache:
    """Caller-owned cache planes (torch device memory) plus the token count."""

    def __init__(self, spec: CacheSpec, device="cuda"):
        import torch
        self.spec = spec
        self.planes = {p: torch.zeros(max(n, 16), dtype=torch.uint8, device=device)
                       for p, n in spec.plane_bytes().items()}
        self.desc = spec.desc(self.planes)
        self.n = 0
        self.seq_n = None   # per-sequence token counts of a ragged batch

    def sequence(self, b):
        """Batch row b as a one-sequence cache sharing this cache's memory (planes are
        [batch][...], so a row's block is contiguous): the uniform entry points then
        serve one sequence of a ragged batch, e.g. to prefill it."""
        import copy
        s = copy.copy(self.spec)
        s.batch = 1
        sub = KVCache.__new__(KVCache)
        sub.spec = s
        full = self.spec.plane_bytes()
        sub.planes = {p: self.planes[p][b * (full[p] // self.spec.batch):(b + 1) * (full[p] // self.spec.batch)]
                      for p in PLANES}
        sub.desc = s.desc(sub.planes)
        sub.n = self.seq_n[b] if self.seq_n is not None else self.n
        sub.seq_n = None
        return sub

    def view(self, plane, dtype=None):
        import torch
        t = self.planes[plane]
        return t.view(dtype) if dtype is not None else t

    def snapshot(self):
        return {p: t.clone() for p, t in self.planes.items()}, self.n

    def restore(self, snap):
        planes, n = snap
        for p, t in planes.items():
            self.planes[p].copy_(t)
        self.n = n


def append_flush(cache: KVCache, k_new, v_new, t_k16, n_before=None, stream=None):
    """Append [B, Hkv, n_new, d] keys/values (f32/bf16/f16) and run due flushes."""
    import torch
    n_before = cache.n if n_before is None else n_before
    n_new = k_new.shape[2]
    if k_new.dtype != v_new.dtype or t_k16.dtype != torch.float16:
        raise ValueError("k_new/v_new must share a dtype and t_k16 must be float16")
    _check(lib().wushkv_append_flush(ctypes.byref(cache.desc), n_before, n_new, _ptr(k_new), _ptr(v_new),
                                     _dtype_code(k_new), _ptr(t_k16), _stream(stream, k_new.device)),
           "append_flush")
    cache.n = n_before + n_new


def append_flush_hadamard(cache: KVCache, k_new, v_new, scale=None, n_before=None, stream=None):
    """append_flush with the fixed key transform T_K = scale * H (Sylvester-Hadamard of order
    head_dim), formed by an in-register fast Walsh-Hadamard transform.  scale defaults to
    fp16(1/sqrt(head_dim)), the orthonormal transform."""
    import numpy as np
    d = k_new.shape[-1]
    if scale is None:
        scale = float(np.float16(1.0 / np.sqrt(d)))
    n_before = cache.n if n_before is None else n_before
    n_new = k_new.shape[2]
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new/v_new must share a dtype")
    _check(lib().wushkv_append_flush_hadamard(ctypes.byref(cache.desc), n_before, n_new, _ptr(k_new), _ptr(v_new),
                                              _dtype_code(k_new), float(scale), _stream(stream, k_new.device)),
           "append_flush_hadamard")
    cache.n = n_before + n_new


def query_transform(t_inv_t, q, num_kv_heads, out=None, stream=None):
    """q~ = T^{-T} q: t_inv_t fp32 [Hkv, d, d], q [B, Hq, d] -> fp32 [B, Hq, d]."""
    import torch
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_query_transform(_ptr(t_inv_t), _ptr(q), _dtype_code(q), B, Hq, num_kv_heads, d,
                                        _ptr(out), _stream(stream, q.device)), "query_transform")
    return out


def decode_num_splits(cache: KVCache, n_tokens, num_q_heads, num_splits=0):
    return int(lib().wushkv_decode_num_splits(ctypes.byref(cache.desc), n_tokens, num_q_heads, num_splits))


def decode_workspace(cache: KVCache, n_tokens, num_q_heads, num_splits=0):
    """A zero-filled workspace large enough for this decode (counters start at zero)."""
    import torch
    n = lib().wushkv_decode_workspace_bytes(ctypes.byref(cache.desc), n_tokens, num_q_heads, num_splits)
    if n == 0:
        raise WushKVError(ERR_SHAPE, "decode_workspace")
    return torch.zeros(n, dtype=torch.uint8, device=cache.planes["sink_k"].device)


def decode_attention(cache: KVCache, q, q_t, n_tokens=None, num_splits=0, workspace=None, out=None, stream=None):
    """GQA decode over the cache's first n_tokens tokens -> fp32 [B, Hq, d]."""
    import torch
    n_tokens = cache.n if n_tokens is None else n_tokens
    B, Hq, d = q.shape
    if workspace is None:
        workspace = decode_workspace(cache, n_tokens, Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention(ctypes.byref(cache.desc), n_tokens, _ptr(q), _dtype_code(q), _ptr(q_t),
                                         Hq, num_splits, _ptr(workspace), workspace.numel(), _ptr(out),
                                         _stream(stream, q.device)), "decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # WUSHKV_NOALLOC_SCRATCH_BYTES


def decode_attention_noalloc(cache: KVCache, q, q_t, n_tokens=None, num_splits=0, out=None, stream=None):
    """decode_attention with the split-K partials in the library's own fixed device array
    (no workspace; the call allocates nothing).  Calls overlapping on one GPU race."""
    import torch
    n_tokens = cache.n if n_tokens is None else n_tokens
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention_noalloc(ctypes.byref(cache.desc), n_tokens, _ptr(q), _dtype_code(q), _ptr(q_t),
                                                 Hq, num_splits, _ptr(out), _stream(stream, q.device)),
           "decode_attention_noalloc")
    return out


def decode_attention_fused(cache: KVCache, q, t_inv_t, n_tokens=None, num_splits=0, workspace=None, out=None,
                           q_t=None, stream=None):
    """decode_attention with the query transform folded in: forms q~ = T^{-T} q itself
    (written to q_t, fp32 [B, Hq, d]) -> (out, q_t)."""
    import torch
    n_tokens = cache.n if n_tokens is None else n_tokens
    B, Hq, d = q.shape
    if workspace is None:
        workspace = decode_workspace(cache, n_tokens, Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention_fused(ctypes.byref(cache.desc), n_tokens, _ptr(q), _dtype_code(q),
                                               _ptr(t_inv_t), _ptr(q_t), Hq, num_splits, _ptr(workspace),
                                               workspace.numel(), _ptr(out), _stream(stream, q.device)),
           "decode_attention_fused")
    return out, q_t


def calib_workspace(batch, num_heads, tokens, head_dim=128, group=1, device="cuda"):
    """A workspace for calib_stats of these sizes."""
    import torch
    n = lib().wushkv_calib_workspace_bytes(batch, num_heads, tokens, head_dim, group)
    if n == 0:
        raise WushKVError(ERR_SHAPE, "calib_workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def calib_stats(x, group=1, workspace=None, out=None, stream=None):
    """Second-order calibration sums: x [B, H, T, d] bf16/f16 -> fp32 [H / group, d, d],
    out[g] = sum of x x^T over the rows of heads g*group .. g*group + group - 1."""
    import torch
    B, H, T, d = x.shape
    if workspace is None:
        workspace = calib_workspace(B, H, T, d, group, x.device)
    if out is None:
        out = torch.empty((H // group, d, d), dtype=torch.float32, device=x.device)
    _check(lib().wushkv_calib_stats(_ptr(x), _dtype_code(x), B, H, T, d, group, _ptr(workspace), workspace.numel(),
                                    _ptr(out), _stream(stream, x.device)), "calib_stats")
    return out


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * len(vals))(*vals)


def append_flush_ragged(cache: KVCache, k_new, v_new, t_k16, n_before=None, stream=None):
    """Append [B, Hkv, n_new, d] keys/values to a ragged batch: sequence b holds
    n_before[b] tokens (default: cache.seq_n) and receives its n_new tokens."""
    import torch
    n_before = list(cache.seq_n if n_before is None else n_before)
    n_new = k_new.shape[2]
    if k_new.dtype != v_new.dtype or t_k16.dtype != torch.float16:
        raise ValueError("k_new/v_new must share a dtype and t_k16 must be float16")
    _check(lib().wushkv_append_flush_ragged(ctypes.byref(cache.desc), _i64_array(n_before), n_new, _ptr(k_new),
                                            _ptr(v_new), _dtype_code(k_new), _ptr(t_k16),
                                            _stream(stream, k_new.device)), "append_flush_ragged")
    cache.seq_n = [n + n_new for n in n_before]


def decode_attention_ragged(cache: KVCache, q, q_t=None, t_inv_t=None, n_tokens=None, num_splits=0, workspace=None,
                            out=None, stream=None):
    """GQA decode of a ragged batch: sequence b attends n_tokens[b] tokens (default:
    cache.seq_n).  With t_inv_t the decode forms q~ itself into q_t (returned);
    otherwise q_t is the caller's q~.  -> (out, q_t)."""
    import torch
    n_tokens = list(cache.seq_n if n_tokens is None else n_tokens)
    B, Hq, d = q.shape
    if workspace is None:
        workspace = decode_workspace(cache, max(n_tokens), Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        if t_inv_t is None:
            raise ValueError("decode_attention_ragged needs q_t or t_inv_t")
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention_ragged(ctypes.byref(cache.desc), _i64_array(n_tokens), _ptr(q),
                                                _dtype_code(q), None if t_inv_t is None else _ptr(t_inv_t),
                                                _ptr(q_t), Hq, num_splits, _ptr(workspace), workspace.numel(),
                                                _ptr(out), _stream(stream, q.device)), "decode_attention_ragged")
    return out, q_t


def decode_attention_generic(cache: KVCache, q, q_t=None, t_inv_t=None, n_tokens=None, num_splits=0, workspace=None,
                             out=None, stream=None):
    """decode_attention_ragged on the library's plain fp32 decode kernel (every shape,
    no matrix cores): an independent second decode of the same cache for cross-checks.
    n_tokens defaults to cache.seq_n, else cache.n for every sequence.  -> (out, q_t)."""
    import torch
    B, Hq, d = q.shape
    if n_tokens is None:
        n_tokens = cache.seq_n if cache.seq_n is not None else [cache.n] * B
    n_tokens = list(n_tokens)
    if workspace is None:
        workspace = decode_workspace(cache, max(n_tokens), Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        if t_inv_t is None:
            raise ValueError("decode_attention_generic needs q_t or t_inv_t")
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention_generic(ctypes.byref(cache.desc), _i64_array(n_tokens), _ptr(q),
                                                 _dtype_code(q), None if t_inv_t is None else _ptr(t_inv_t),
                                                 _ptr(q_t), Hq, num_splits, _ptr(workspace), workspace.numel(),
                                                 _ptr(out), _stream(stream, q.device)), "decode_attention_generic")
    return out, q_t


def _device_counts(seq_n, batch, device):
    import torch
    if seq_n.dtype != torch.int32 or seq_n.shape != (batch,) or seq_n.device != device:
        raise ValueError("seq_n must be an int32 tensor [batch] on the cache's device")
    return _ptr(seq_n)


def append_flush_device(cache: KVCache, seq_n, k_new, v_new, t_k16, stream=None):
    """Append [B, Hkv, n_new, d] keys/values with the token counts in device memory:
    sequence b holds seq_n[b] tokens (int32 tensor [B] on the GPU), and the call adds
    n_new to each count on the stream.  Nothing here reads the counts on the host, so
    the call can be recorded into a CUDA/HIP graph and replayed as later steps.
    cache.seq_n (the host-side view) is not updated."""
    import torch
    if k_new.dtype != v_new.dtype or t_k16.dtype != torch.float16:
        raise ValueError("k_new/v_new must share a dtype and t_k16 must be float16")
    _check(lib().wushkv_append_flush_device(ctypes.byref(cache.desc), _device_counts(seq_n, cache.spec.batch,
                                                                                     k_new.device),
                                            k_new.shape[2], _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                            _ptr(t_k16), _stream(stream, k_new.device)), "append_flush_device")


def decode_attention_device(cache: KVCache, seq_n, max_tokens, q, t_inv_t=None, q_t=None, num_splits=0,
                            workspace=None, out=None, stream=None):
    """GQA decode with sequence b attending seq_n[b] tokens, read on the device
    (int32 tensor [B]); max_tokens bounds the counts and sizes the split count and
    workspace.  With t_inv_t the decode forms q~ itself into q_t.  -> (out, q_t)."""
    import torch
    B, Hq, d = q.shape
    if workspace is None:
        workspace = decode_workspace(cache, max_tokens, Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        if t_inv_t is None:
            raise ValueError("decode_attention_device needs q_t or t_inv_t")
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention_device(ctypes.byref(cache.desc), _device_counts(seq_n, B, q.device),
                                                int(max_tokens), _ptr(q), _dtype_code(q),
                                                None if t_inv_t is None else _ptr(t_inv_t), _ptr(q_t), Hq,
                                                num_splits, _ptr(workspace), workspace.numel(), _ptr(out),
                                                _stream(stream, q.device)), "decode_attention_device")
    return out, q_t


class PagedKVCache:
    """A cache whose quantized body lives in page pools: the window planes are
    [batch][...] as in KVCache, the code and parameter planes are pools of num_pages
    pages of page_tokens rows per KV head, and table (int32 [batch][max_pages], on the
    device) maps each sequence's logical body page to a physical page.  The caller
    fills the table; unused entries may hold anything."""

    def __init__(self, spec: CacheSpec, page_tokens, num_pages, max_pages=None, device="cuda"):
        import torch
        self.spec = spec
        body = max(0, spec.capacity - spec.sink)
        self.max_pages = max_pages or max(1, -(-body // page_tokens))
        self.table = torch.zeros((spec.batch, self.max_pages), dtype=torch.int32, device=device)
        self.pages = PagesDesc(self.table.data_ptr(), page_tokens, self.max_pages, num_pages)
        d = spec.desc()
        sizes = {p: int(lib().wushkv_pool_bytes(ctypes.byref(d), ctypes.byref(self.pages), i))
                 for i, p in enumerate(PLANES)}
        if any(v == 0 and not p.startswith("sink") for p, v in sizes.items()):
            raise WushKVError(ERR_SHAPE, "paged cache geometry")
        self.planes = {p: torch.zeros(max(n, 16), dtype=torch.uint8, device=device) for p, n in sizes.items()}
        self.desc = spec.desc(self.planes)
        self.seq_n = [0] * spec.batch

    WINDOWS = ("sink_k", "sink_v", "ring_k", "ring_v")

    def sequence(self, b):
        """Sequence b as a one-sequence paged cache: its own window rows and table row,
        the shared pools."""
        import copy
        s = copy.copy(self.spec)
        s.batch = 1
        sub = PagedKVCache.__new__(PagedKVCache)
        sub.spec, sub.max_pages = s, self.max_pages
        sub.table = self.table[b:b + 1]
        sub.pages = PagesDesc(sub.table.data_ptr(), self.pages.page_tokens, self.max_pages, self.pages.num_pages)
        sub.planes = dict(self.planes)
        for p in self.WINDOWS:
            per = self.planes[p].numel() // self.spec.batch
            sub.planes[p] = self.planes[p][b * per:(b + 1) * per]
        sub.desc = s.desc(sub.planes)
        sub.seq_n = [self.seq_n[b]]
        return sub


def append_flush_paged(cache: PagedKVCache, k_new, v_new, t_k16, n_before=None, stream=None):
    """append_flush_ragged on a paged cache (sequence b holds n_before[b] tokens,
    default cache.seq_n)."""
    import torch
    n_before = list(cache.seq_n if n_before is None else n_before)
    n_new = k_new.shape[2]
    if k_new.dtype != v_new.dtype or t_k16.dtype != torch.float16:
        raise ValueError("k_new/v_new must share a dtype and t_k16 must be float16")
    _check(lib().wushkv_append_flush_paged(ctypes.byref(cache.desc), ctypes.byref(cache.pages), _i64_array(n_before),
                                           n_new, _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(t_k16),
                                           _stream(stream, k_new.device)), "append_flush_paged")
    cache.seq_n = [n + n_new for n in n_before]


def decode_attention_paged(cache: PagedKVCache, q, q_t=None, t_inv_t=None, n_tokens=None, num_splits=0,
                           workspace=None, out=None, stream=None):
    """decode_attention_ragged on a paged cache.  -> (out, q_t)."""
    import torch
    n_tokens = list(cache.seq_n if n_tokens is None else n_tokens)
    B, Hq, d = q.shape
    if workspace is None:
        workspace = decode_workspace(cache, max(n_tokens), Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        if t_inv_t is None:
            raise ValueError("decode_attention_paged needs q_t or t_inv_t")
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_attention_paged(ctypes.byref(cache.desc), ctypes.byref(cache.pages),
                                               _i64_array(n_tokens), _ptr(q), _dtype_code(q),
                                               None if t_inv_t is None else _ptr(t_inv_t), _ptr(q_t), Hq, num_splits,
                                               _ptr(workspace), workspace.numel(), _ptr(out),
                                               _stream(stream, q.device)), "decode_attention_paged")
    return out, q_t


def decode_step(cache: KVCache, k_new, v_new, t_k16, q, t_inv_t, q_t=None, num_splits=0, workspace=None, out=None,
                n_before=None, stream=None):
    """One decode step in one call: append one token per sequence (k_new / v_new
    [B, Hkv, 1, d]), flush if due, and decode with the query transform fused; the same
    result as append_flush + decode_attention_fused.  -> (out, q_t)."""
    import torch
    n_before = cache.n if n_before is None else n_before
    B, Hq, d = q.shape
    if k_new.dtype != v_new.dtype or t_k16.dtype != torch.float16 or k_new.shape[2] != 1:
        raise ValueError("one new token per sequence, k_new/v_new of one dtype, t_k16 float16")
    if workspace is None:
        workspace = decode_workspace(cache, n_before + 1, Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_step(ctypes.byref(cache.desc), n_before, _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                    _ptr(t_k16), _ptr(q), _dtype_code(q), _ptr(t_inv_t), _ptr(q_t), Hq, num_splits,
                                    _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream, q.device)),
           "decode_step")
    cache.n = n_before + 1
    return out, q_t


def decode_step_device(cache: KVCache, seq_n, max_tokens, k_new, v_new, t_k16, q, t_inv_t, q_t=None, num_splits=0,
                       workspace=None, out=None, stream=None):
    """decode_step with the counts in device memory (int32 tensor [B]): sequence b
    holds seq_n[b] tokens, receives one, attends seq_n[b] + 1, and seq_n[b] is advanced
    on the stream.  Nothing is read on the host, so the call can be recorded into a
    graph and replayed as each following step.  -> (out, q_t)."""
    import torch
    B, Hq, d = q.shape
    if k_new.dtype != v_new.dtype or t_k16.dtype != torch.float16 or k_new.shape[2] != 1:
        raise ValueError("one new token per sequence, k_new/v_new of one dtype, t_k16 float16")
    if workspace is None:
        workspace = decode_workspace(cache, max_tokens, Hq, num_splits)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if q_t is None:
        q_t = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check(lib().wushkv_decode_step_device(ctypes.byref(cache.desc), _device_counts(seq_n, B, q.device),
                                           int(max_tokens), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(t_k16),
                                           _ptr(q), _dtype_code(q), _ptr(t_inv_t), _ptr(q_t), Hq, num_splits,
                                           _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream, q.device)),
           "decode_step_device")
    return out, q_t
