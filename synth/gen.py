"""Seeded input generators shared by the oracle tests, the GPU tests and the bench.

They produce what the cache receives from the model side of the path --
post-RoPE keys and values, decode queries, and each KV head's invertible key
transform T_K (with its inverse-transpose, which the caller hands the query
transform) -- and nothing of the method's own arithmetic.

Recipe (per layer l and KV head g; "stream" separates independent draws):

* U: Haar-orthogonal d x d (QR of a standard normal matrix, column signs fixed
  by sign(diag R)); lambda_i = 10**Uniform(-2, 2) (log-uniform on [1e-2, 1e2]).
* K rows k = U diag(sqrt(lambda)) z, with z ~ N(0, I) ("gauss") or iid
  t_3 / sqrt(3) ("t3", unit variance).  With k_outliers > 0, that many
  distinct channels of every K row are multiplied by 20.
* V rows: z ~ N(0, I) ("gauss_iso"), or the t_3 construction under its own
  per-head U and lambda ("t3").
* T_K = Q diag(s), Q Haar-orthogonal, s_i = 2**Uniform(-2, 2) (log-uniform on
  [0.25, 4]), rounded to fp16.  T^{-T} is the float64 inverse-transpose of
  that fp16 matrix, handed over in fp32.
* Queries q ~ N(0, I).  Calibration queries (a sequence of rows per query head):
  q = U_h diag(sqrt(lambda_h)) z under each query head's own U_h and lambda_h.
* Everything is rounded to bf16 (round-to-nearest-even) unless the workload's
  input dtype is fp32.

K/V rows are drawn with a torch.Generator on the target device, one seeded
block per (layer, batch row, KV head), so a caller can regenerate exactly the
blocks it needs.  The same (workload, device type) always gives the same
tensors; CPU and GPU draws differ from each other, so checks that compare a GPU
result against the oracle copy the GPU-resident inputs to the host.
"""
import numpy as np
import torch

from .configs import Workload

STREAM_K_STATS, STREAM_V_STATS, STREAM_T = 0, 1, 2
STREAM_K_ROWS, STREAM_V_ROWS = 10, 11
STREAM_Q = 20
STREAM_QC_STATS, STREAM_QC_ROWS = 30, 31


def _seed(*key) -> int:
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, dtype=np.uint64)[0] >> 1)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def head_mixing(w: Workload, layer: int, head: int, stream: int):
    """(U, lambda, outlier channel list) of one KV head, float64 numpy."""
    rng = _rng(w.seed, layer, head, stream)
    d = w.head_dim
    u = haar_orthogonal(rng, d)
    lam = 10.0 ** rng.uniform(-2.0, 2.0, size=d)
    outl = []
    if stream == STREAM_K_STATS and w.k_outliers:
        outl = sorted(rng.choice(d, size=w.k_outliers, replace=False).tolist())
    return u, lam, outl


def key_transforms(w: Workload, layer: int):
    """(T_K fp16 [Hkv,d,d], T^{-T} fp32 [Hkv,d,d]) as CPU tensors."""
    d = w.head_dim
    t16 = np.empty((w.num_kv_heads, d, d), dtype=np.float16)
    tinvt = np.empty((w.num_kv_heads, d, d), dtype=np.float32)
    for g in range(w.num_kv_heads):
        rng = _rng(w.seed, layer, g, STREAM_T)
        q = haar_orthogonal(rng, d)
        s = 2.0 ** rng.uniform(-2.0, 2.0, size=d)
        t = (q * s[None, :]).astype(np.float16)
        t16[g] = t
        tinvt[g] = np.linalg.inv(t.astype(np.float64)).T.astype(np.float32)
    return torch.from_numpy(t16), torch.from_numpy(tinvt)


def _rows(n: int, d: int, dist: str, gen: torch.Generator, device) -> torch.Tensor:
    z = torch.randn(n, d, generator=gen, device=device, dtype=torch.float32)
    if dist in ("t3",):
        chi = torch.randn(3, n, d, generator=gen, device=device, dtype=torch.float32).square_().sum(0)
        z = z / torch.sqrt(chi / 3.0) / np.sqrt(3.0)
    return z


def kv_block(w: Workload, layer: int, b: int, g: int, n: int, device="cpu"):
    """K and V rows [n, d] (input dtype) of batch row b, KV head g."""
    d = w.head_dim
    dt = torch_dtype(w.in_dtype)
    gen_k = torch.Generator(device=device).manual_seed(_seed(w.seed, layer, g, b, STREAM_K_ROWS))
    gen_v = torch.Generator(device=device).manual_seed(_seed(w.seed, layer, g, b, STREAM_V_ROWS))
    u, lam, outl = head_mixing(w, layer, g, STREAM_K_STATS)
    mix = torch.from_numpy((u * np.sqrt(lam)[None, :]).T.astype(np.float32)).to(device)
    k = _rows(n, d, w.k_dist, gen_k, device) @ mix
    if outl:
        k[:, outl] *= 20.0
    zv = _rows(n, d, w.v_dist, gen_v, device)
    if w.v_dist == "t3":
        uv, lamv, _ = head_mixing(w, layer, g, STREAM_V_STATS)
        mixv = torch.from_numpy((uv * np.sqrt(lamv)[None, :]).T.astype(np.float32)).to(device)
        v = zv @ mixv
    else:
        v = zv
    return k.to(dt), v.to(dt)


def kv_tensors(w: Workload, layer: int, n: int, device="cpu"):
    """K, V [B, Hkv, n, d] in the workload's input dtype."""
    dt = torch_dtype(w.in_dtype)
    shape = (w.batch, w.num_kv_heads, n, w.head_dim)
    k = torch.empty(shape, dtype=dt, device=device)
    v = torch.empty(shape, dtype=dt, device=device)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            k[b, g], v[b, g] = kv_block(w, layer, b, g, n, device)
    return k, v


def queries(w: Workload, layer: int, step: int, device="cpu") -> torch.Tensor:
    """Decode queries [B, Hq, d] for decode step `step`."""
    rng = _rng(w.seed, layer, STREAM_Q, step)
    q = rng.standard_normal((w.batch, w.num_q_heads, w.head_dim)).astype(np.float32)
    return torch.from_numpy(q).to(torch_dtype(w.in_dtype)).to(device)


def _calib_query_mix(w: Workload, layer: int, h: int, device) -> torch.Tensor:
    rng = _rng(w.seed, layer, h, STREAM_QC_STATS)
    u = haar_orthogonal(rng, w.head_dim)
    lam = 10.0 ** rng.uniform(-2.0, 2.0, size=w.head_dim)
    return torch.from_numpy((u * np.sqrt(lam)[None, :]).T.astype(np.float32)).to(device)


def calib_query_block(w: Workload, layer: int, b: int, h: int, n: int, device="cpu", mix=None) -> torch.Tensor:
    """Calibration query rows [n, d] (input dtype) of batch row b, query head h."""
    mix = _calib_query_mix(w, layer, h, device) if mix is None else mix
    gen = torch.Generator(device=device).manual_seed(_seed(w.seed, layer, h, b, STREAM_QC_ROWS))
    return (_rows(n, w.head_dim, "gauss", gen, device) @ mix).to(torch_dtype(w.in_dtype))


def calib_queries(w: Workload, layer: int, n: int, device="cpu", heads=None) -> torch.Tensor:
    """Calibration queries [B, len(heads), n, d] (all query heads by default)."""
    heads = list(range(w.num_q_heads)) if heads is None else list(heads)
    q = torch.empty((w.batch, len(heads), n, w.head_dim), dtype=torch_dtype(w.in_dtype), device=device)
    for i, h in enumerate(heads):
        mix = _calib_query_mix(w, layer, h, device)
        for b in range(w.batch):
            q[b, i] = calib_query_block(w, layer, b, h, n, device, mix)
    return q
