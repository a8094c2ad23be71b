"""Seeded synthetic inputs for the indexer + top-k + sparse-MLA path.

This module only draws random numbers and lays them out; it holds none of
the path's arithmetic (no scoring, selection, quantisation or attention).
The tests and the benchmark hand the same tensors to the HIP library and to
the CPU oracle.

Workloads (shapes and value distributions as given for the path):
  tiny_prefill      1 request, T = S = 256 causal; indexer 4 heads x 32 dims,
                    top-k 16; q, k integers uniform in [-3, 3] stored as f32,
                    w uniform in {1, 2}; MLA 4 heads, latent 64 + rope 16, f32
                    N(0,1) latent rows and queries.
  decode_32k_mtp    64 requests x 32768 cached tokens, 2 query tokens each
                    (one plus one MTP draft); indexer 32 heads x 128, bf16
                    q, k ~ N(0,1), w ~ N(0,1)/sqrt(32), top-k 2048; MLA 64
                    heads, latent 512 + rope 64, bf16 N(0,1).
  prefill_16k       1 request, 16384 tokens causal; indexer 32 x 128 bf16,
                    top-k 2048; MLA 64 x (512 + 64) bf16; all values N(0,1).
  fp8_decode_varlen 128 requests, lengths uniform in [1024, 131072], one
                    query each; indexer keys N(0,1) -> bf16 -> e4m3 + fp32
                    scale (quantised by the cache write), bf16 q,
                    w ~ N(0,1)/sqrt(32); MLA as decode_32k_mtp.
  fp8q_decode_32k_mtp  decode_32k_mtp with the FP8 indexer path: bf16
                    queries and keys rotated and quantised to e4m3 by the
                    library (per head / per token scales).
  indexshare_8layer 8 layers [full, shared, shared, shared] x 2, 64 requests
                    x 32768, one query each, per-layer bf16 indexer q, k, w
                    and latent rows.
Paged caches use 64-token blocks; each request's blocks are a seeded random
permutation of the physical blocks.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (Batch, LayerInputs, PrologueInputs, make_batch, make_layer,  # noqa: F401
                  make_prologue, make_random_indices, torch_gen)
