"""Workload descriptions (sizes, dtypes, distributions, seeds)."""

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional


@dataclass(frozen=True)
class Config:
    name: str
    cid: int                      # seed base: tensor seed = 1000*cid + id
    num_reqs: int
    q_len: int                    # query tokens per request
    seq_len: Optional[int]        # fixed context length, or None = varlen
    seq_len_range: Optional[tuple] = None   # (lo, hi) inclusive, varlen
    causal_prefill: bool = False  # q_len == seq_len, queries at 0..T-1
    n_idx_heads: int = 32
    d_idx: int = 128
    topk: int = 2048
    idx_dtype: str = "bf16"       # dtype of indexer q and new keys
    idx_cache_dtype: str = "bf16"
    idx_q_fp8: bool = False       # queries and keys rotated and quantised to e4m3
    idx_values: str = "normal"    # "normal" or "int3" (uniform ints -3..3)
    w_values: str = "normal_over_sqrt_heads"   # or "normal", "one_two"
    n_heads: int = 64
    kv_lora_rank: int = 512
    rope_dim: int = 64
    mla_dtype: str = "bf16"
    block_size: int = 64
    indexer_types: Optional[List[str]] = None  # None = one full layer
    # indexer prologue (the projections that produce q, k and w)
    hidden_dim: int = 6144
    q_lora_rank: int = 2048
    idx_rope_dim: int = 64
    norm_eps: float = 1e-5

    @property
    def n_layers(self):
        return 1 if self.indexer_types is None else len(self.indexer_types)

    @property
    def d_latent(self):
        return self.kv_lora_rank + self.rope_dim

    @property
    def softmax_scale(self):
        return 1.0 / math.sqrt(self.kv_lora_rank + self.rope_dim)

    def scaled(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "tiny_prefill": Config(
        name="tiny_prefill", cid=1, num_reqs=1, q_len=256, seq_len=256,
        causal_prefill=True, n_idx_heads=4, d_idx=32, topk=16,
        idx_dtype="f32", idx_cache_dtype="f32", idx_values="int3",
        w_values="one_two", n_heads=4, kv_lora_rank=64, rope_dim=16,
        mla_dtype="f32"),
    "decode_32k_mtp": Config(
        name="decode_32k_mtp", cid=2, num_reqs=64, q_len=2, seq_len=32768),
    "prefill_16k": Config(
        name="prefill_16k", cid=3, num_reqs=1, q_len=16384, seq_len=16384,
        causal_prefill=True, w_values="normal"),
    "fp8_decode_varlen": Config(
        name="fp8_decode_varlen", cid=4, num_reqs=128, q_len=1, seq_len=None,
        seq_len_range=(1024, 131072), idx_cache_dtype="fp8"),
    "fp8q_decode_32k_mtp": Config(
        name="fp8q_decode_32k_mtp", cid=6, num_reqs=64, q_len=2, seq_len=32768,
        idx_cache_dtype="fp8", idx_q_fp8=True),
    "indexshare_8layer": Config(
        name="indexshare_8layer", cid=5, num_reqs=64, q_len=1, seq_len=32768,
        indexer_types=["full", "shared", "shared", "shared",
                       "full", "shared", "shared", "shared"]),
}


def get_config(name):
    return CONFIGS[name]
