"""The five seeded synthetic workloads of the WUSH-KV online path.

Each workload stands in for what the pages evaluate on real models (Qwen3-8B
attention modules, 36 of them, GQA with 32 query and 8 KV heads and head_dim
128; WUSH-KV paper digest, "key experiments").  No model weights or datasets
are used: K/V rows are drawn from anisotropic Gaussian or Student-t
distributions and each KV head gets a synthetic invertible key transform.

This module holds sizes and names only -- none of the method's arithmetic.
"""
from dataclasses import dataclass, field, replace
from typing import Optional

QUEST = "quest"
AFFINE = "affine"


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int                 # tokens per sequence before decoding starts
    in_dtype: str                # "f32" or "bf16"
    quant_k: str
    quant_v: str
    bits_k: int
    bits_v: int
    sink: int = 64
    recent: int = 256
    chunk: int = 8
    clip_mult: float = 2.5
    pct_lo: float = 0.5
    pct_hi: float = 99.5
    decode_steps: int = 1
    num_splits: int = 0          # 0 = let the library choose
    k_dist: str = "gauss"        # "gauss" | "t3"
    v_dist: str = "gauss_iso"    # "gauss_iso" | "t3"
    k_outliers: int = 0          # outlier channels per head, scaled by 20
    flush_bits: tuple = ()       # bulk flush: bit-widths run as separate passes

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def capacity(self) -> int:
        return self.context + self.decode_steps

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="c0_tiny", seed=0, layers=1, batch=1, num_q_heads=4, num_kv_heads=1,
    head_dim=64, context=512, in_dtype="f32", quant_k=QUEST, quant_v=QUEST,
    bits_k=2, bits_v=2, chunk=8, decode_steps=1, k_dist="gauss", v_dist="gauss_iso")

LAYER_8B = Workload(
    name="c1_8b_layer_decode", seed=1, layers=1, batch=1, num_q_heads=32, num_kv_heads=8,
    head_dim=128, context=8192, in_dtype="bf16", quant_k=QUEST, quant_v=QUEST,
    bits_k=2, bits_v=2, chunk=8, decode_steps=64, k_dist="gauss", v_dist="gauss_iso",
    k_outliers=4)

SERVING = Workload(
    name="c2_batched_serving_decode", seed=2, layers=1, batch=32, num_q_heads=32, num_kv_heads=8,
    head_dim=128, context=32768, in_dtype="bf16", quant_k=AFFINE, quant_v=AFFINE,
    bits_k=2, bits_v=2, chunk=16, decode_steps=1, k_dist="t3", v_dist="t3")

BULK_FLUSH = Workload(
    name="c3_bulk_prefill_flush", seed=3, layers=36, batch=1, num_q_heads=32, num_kv_heads=8,
    head_dim=128, context=65536, in_dtype="bf16", quant_k=QUEST, quant_v=QUEST,
    bits_k=2, bits_v=2, chunk=8, decode_steps=0, k_dist="gauss", v_dist="gauss_iso",
    k_outliers=4, flush_bits=(2, 3, 4))

LONG_CONTEXT = Workload(
    name="c4_long_context_decode", seed=4, layers=1, batch=8, num_q_heads=64, num_kv_heads=8,
    head_dim=128, context=131072, in_dtype="bf16", quant_k=AFFINE, quant_v=AFFINE,
    bits_k=2, bits_v=3, chunk=8, decode_steps=1, num_splits=128, k_dist="t3", v_dist="t3")

ALL = [TINY, LAYER_8B, SERVING, BULK_FLUSH, LONG_CONTEXT]

# Calibration statistics (outside the decode/flush configurations above): one
# attention layer of the 8B geometry over 128 calibration sequences of 1024 tokens
# (digest, key experiments: 128 calibration sequences; the length 1024 stated for the
# evaluation sequences is taken for them too).  Keys as in the 8B layer workload.
CALIB = Workload(
    name="c5_calibration_stats", seed=5, layers=1, batch=128, num_q_heads=32, num_kv_heads=8,
    head_dim=128, context=1024, in_dtype="bf16", quant_k=QUEST, quant_v=QUEST,
    bits_k=2, bits_v=2, chunk=8, decode_steps=0, k_dist="gauss", v_dist="gauss_iso",
    k_outliers=4)
BY_NAME = {w.name: w for w in ALL}
