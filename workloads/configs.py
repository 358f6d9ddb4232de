"""The DSA workload shapes.

Hot-path dimensions follow the DeepSeek-V3.2 configuration defaults on the
DeepSeek-V3.2 model documentation page (index_topk 2048, index_head_dim 128,
index_n_heads 64, num_attention_heads 128, kv_lora_rank 512, qk_rope_head_dim
64, qk_nope_head_dim 128): the absorbed latent row is 512 + 64 = 576 wide, the
value is its first 512 columns, and the softmax scale is 1/sqrt(128 + 64), the
scale of the un-absorbed q/k width it must reproduce.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int          # B sequences
    n_q: int            # T queries per sequence (the last T tokens)
    max_kv: int         # L_max cache capacity
    kv_len: int         # L context length of every sequence
    idx_heads: int      # index_n_heads
    idx_dim: int        # index_head_dim
    topk: int           # index_topk
    heads: int          # MLA query heads
    qk_dim: int         # kv_lora_rank + qk_rope_head_dim
    v_dim: int          # kv_lora_rank
    sm_scale: float
    idx_dtype: str      # "f32" | "bf16" | "fp8"
    mla_dtype: str      # "f32" | "bf16" | "fp8" (e4m3 latent cache and queries, bf16 output)
    heavy_frac: float = 0.0       # share of key positions whose index-key and kv rows are scaled by 4
    lognormal_sigma: float = 0.0  # per-token row scale exp(sigma * z)
    seed: int = 0
    description: str = ""

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def rows(self) -> int:
        return self.batch * self.n_q


V32 = dict(idx_heads=64, idx_dim=128, topk=2048, heads=128, qk_dim=576, v_dim=512,
           sm_scale=1.0 / math.sqrt(128 + 64))

WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", batch=1, n_q=256, max_kv=256, kv_len=256, idx_heads=4, idx_dim=32, topk=64,
        heads=4, qk_dim=80, v_dim=64, sm_scale=1.0 / math.sqrt(80), idx_dtype="f32", mla_dtype="f32",
        description="tiny fp32 prefill L=256, 4 index heads x 32, top-64, 4-head MLA 80/64"),
    "prefill_4k": Workload(
        name="prefill_4k", batch=1, n_q=4096, max_kv=4096, kv_len=4096, idx_dtype="bf16", mla_dtype="bf16",
        description="single-layer bf16 prefill, L=4096", **V32),
    "decode_32k": Workload(
        name="decode_32k", batch=64, n_q=1, max_kv=32768, kv_len=32768, idx_dtype="bf16", mla_dtype="bf16",
        description="single-layer bf16 decode, 64 sequences x 1 query, context 32768", **V32),
    "prefill_32k": Workload(
        name="prefill_32k", batch=1, n_q=32768, max_kv=32768, kv_len=32768, idx_dtype="bf16",
        mla_dtype="bf16", heavy_frac=0.05,
        description="single-layer bf16 prefill, L=32768, 5% heavy-hitter keys x4", **V32),
    "decode_128k_fp8": Workload(
        name="decode_128k_fp8", batch=16, n_q=1, max_kv=131072, kv_len=131072, idx_dtype="fp8",
        mla_dtype="bf16", lognormal_sigma=0.5,
        description="decode, fp8 e4m3 indexer behind a Hadamard rotation, bf16 MLA, 16 x context 131072",
        **V32),
    "decode_128k_fp8_mla": Workload(
        name="decode_128k_fp8_mla", batch=16, n_q=1, max_kv=131072, kv_len=131072, idx_dtype="fp8",
        mla_dtype="fp8", lognormal_sigma=0.5,
        description="decode, fp8 indexer and fp8 e4m3 latent cache for the MLA, 16 x context 131072",
        **V32),
}

ORDER = ["tiny_f32", "prefill_4k", "decode_32k", "prefill_32k", "decode_128k_fp8", "decode_128k_fp8_mla"]


def get(name: str) -> Workload:
    return WORKLOADS[name]
