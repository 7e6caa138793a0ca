"""Key transforms T_K used as inputs of the path: fixed ones (identity, Hadamard) and a
data-adaptive one built from calibration statistics (Gram whitening).

The WUSH-KV pages compare their data-adaptive transforms with fixed orthogonal ones,
Hadamard among them, and note that an orthogonal transform cannot scale directions
unevenly (WUSH-KV digest, "takeaways" and "key experiments").  These builders supply
such transforms as T_K inputs; the library applies whatever T_K it is given.  Gram
whitening is one data-adaptive, non-orthogonal transform (the inverse square root of the
keys' second moment, scaled to the identity's Frobenius norm).  It is not the pages'
WUSH construction, whose formula the pages do not give.

Like the rest of synth/, this holds input generators only: no step of the quantizer,
the cache or the attention."""
import numpy as np
import torch


def hadamard(d: int) -> np.ndarray:
    """Orthonormal Sylvester-Hadamard matrix of order d (a power of two), float64."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def whitening(gram: np.ndarray, count: int) -> np.ndarray:
    """T = c (gram / count)^{-1/2} with c such that ||T||_F = sqrt(d): whitens rows whose
    second moment is gram / count, up to one overall scale."""
    sigma = np.asarray(gram, dtype=np.float64) / count
    sigma = 0.5 * (sigma + sigma.T)
    lam, u = np.linalg.eigh(sigma)
    lam = np.maximum(lam, lam.max() * 1e-8)
    t = (u / np.sqrt(lam)[None, :]) @ u.T
    return t * (np.sqrt(sigma.shape[0]) / np.linalg.norm(t))


def as_inputs(t: np.ndarray):
    """(T_K fp16 [..., d, d], T^{-T} fp32) as CPU tensors; the inverse-transpose is taken
    of the fp16-rounded matrix, so that q~ . (T16 k) = q . k exactly up to rounding."""
    t = np.asarray(t)
    t16 = t.astype(np.float16)
    tinvt = np.linalg.inv(t16.astype(np.float64)).swapaxes(-1, -2).astype(np.float32)
    return torch.from_numpy(t16), torch.from_numpy(np.ascontiguousarray(tinvt))


def per_head(t: np.ndarray, heads: int) -> np.ndarray:
    """The same d x d transform for every KV head: [heads, d, d]."""
    return np.broadcast_to(np.asarray(t), (heads,) + np.asarray(t).shape).copy()
