"""Seeded generators.  Random draws and memory layout only."""

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# tensor ids inside a config's seed space (seed = 1000 * cid + id + 100*layer)
_ID_LENS, _ID_BLOCKS, _ID_Q, _ID_W, _ID_K, _ID_QM, _ID_KV, _ID_IDX = range(8)
_ID_HID, _ID_QA, _ID_WQB, _ID_WK, _ID_WP, _ID_KNW = range(8, 14)


def torch_gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, dtype, seed, device, scale=1.0, chunk_elems=1 << 27):
    """N(0, scale^2) values drawn in fp32 and rounded to `dtype`."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    g = torch_gen(seed, device)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[s:e] = x.to(dtype)
    return out


def _ints(shape, lo, hi, seed, device):
    """Integers uniform in [lo, hi], stored as fp32."""
    g = torch_gen(seed, device)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device,
                         dtype=torch.int64).to(torch.float32)


@dataclass
class Batch:
    """Ragged batch + paged-cache geometry (host lists and device tensors)."""
    seq_lens: List[int]
    q_lens: List[int]
    block_size: int
    max_blocks: int
    num_slots: int
    block_table_host: np.ndarray         # [B, max_blocks] int32
    seq_lens_t: torch.Tensor             # [B] int32
    cu_q_t: torch.Tensor                 # [B+1] int32
    block_table_t: torch.Tensor          # [B, max_blocks] int32
    slot_mapping_t: torch.Tensor         # [N] int64, slots of the queries
    cu_q_host: np.ndarray

    @property
    def num_reqs(self):
        return len(self.seq_lens)

    @property
    def num_q_tokens(self):
        return int(sum(self.q_lens))

    @property
    def max_seq_len(self):
        return int(max(self.seq_lens))

    @property
    def max_q_len(self):
        return int(max(self.q_lens))


def make_batch(cfg, device, seq_lens=None, q_lens=None):
    """Lengths, block tables and query slots for a workload.

    seq_lens / q_lens override the config (used for small parity cases).
    """
    B = cfg.num_reqs
    if seq_lens is None:
        if cfg.seq_len is not None:
            seq_lens = [cfg.seq_len] * B
        else:
            lo, hi = cfg.seq_len_range
            rng = np.random.Generator(np.random.PCG64(1000 * cfg.cid + _ID_LENS))
            seq_lens = [int(x) for x in rng.integers(lo, hi + 1, size=B)]
    seq_lens = [int(x) for x in seq_lens]
    if q_lens is None:
        q_lens = [cfg.q_len if not cfg.causal_prefill else s for s in seq_lens]
    q_lens = [int(x) for x in q_lens]
    assert all(0 <= q <= s for q, s in zip(q_lens, seq_lens))
    bs = cfg.block_size
    nblk = [max(1, -(-s // bs)) for s in seq_lens]
    max_blocks = max(nblk)
    total = sum(nblk)
    rng = np.random.Generator(np.random.PCG64(1000 * cfg.cid + _ID_BLOCKS))
    perm = rng.permutation(total).astype(np.int32)
    bt = np.zeros((B, max_blocks), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    # slots of the query tokens (positions seq_len - q_len .. seq_len - 1)
    slots = []
    for b in range(B):
        for i in range(q_lens[b]):
            p = seq_lens[b] - q_lens[b] + i
            slots.append(int(bt[b, p // bs]) * bs + p % bs)
    return Batch(
        seq_lens=seq_lens, q_lens=q_lens, block_size=bs, max_blocks=max_blocks,
        num_slots=total * bs, block_table_host=bt,
        seq_lens_t=torch.tensor(seq_lens, dtype=torch.int32, device=device),
        cu_q_t=torch.tensor(cu, dtype=torch.int32, device=device),
        block_table_t=torch.from_numpy(bt).to(device),
        slot_mapping_t=torch.tensor(slots, dtype=torch.int64, device=device),
        cu_q_host=cu)


@dataclass
class LayerInputs:
    q_idx: Optional[torch.Tensor]      # [N, H_I, d_I]  f32 / bf16
    w: Optional[torch.Tensor]          # [N, H_I] f32
    k_src: Optional[torch.Tensor]      # [num_slots, d_I] key values (f32/bf16)
    q_mla: torch.Tensor                # [N, H, R+P]
    kv_cache: torch.Tensor             # [num_slots, R+P]


def make_layer(cfg, batch, device, layer=0, with_indexer=True):
    """One layer's tensors.  Keys are given in slot layout (every slot of the
    paged cache gets a value); for an FP8 cache they are the bf16 values that
    the cache write quantises."""
    base = 1000 * cfg.cid + 100 * layer
    N = batch.num_q_tokens
    S = batch.num_slots
    q_idx = w = k_src = None
    if with_indexer:
        key_dtype = _TORCH_DTYPES[cfg.idx_dtype]
        if cfg.idx_values == "int3":
            q_idx = _ints((N, cfg.n_idx_heads, cfg.d_idx), -3, 3, base + _ID_Q,
                          device).to(key_dtype)
            k_src = _ints((S, cfg.d_idx), -3, 3, base + _ID_K, device).to(key_dtype)
        else:
            q_idx = _normal((N, cfg.n_idx_heads, cfg.d_idx), key_dtype,
                            base + _ID_Q, device)
            k_src = _normal((S, cfg.d_idx), key_dtype, base + _ID_K, device)
        if cfg.w_values == "one_two":
            w = _ints((N, cfg.n_idx_heads), 1, 2, base + _ID_W, device)
        elif cfg.w_values == "normal":
            w = _normal((N, cfg.n_idx_heads), torch.float32, base + _ID_W, device)
        else:
            w = _normal((N, cfg.n_idx_heads), torch.float32, base + _ID_W, device,
                        scale=1.0 / math.sqrt(cfg.n_idx_heads))
    mdt = _TORCH_DTYPES[cfg.mla_dtype]
    q_mla = _normal((N, cfg.n_heads, cfg.d_latent), mdt, base + _ID_QM, device)
    kv = _normal((S, cfg.d_latent), mdt, base + _ID_KV, device)
    return LayerInputs(q_idx=q_idx, w=w, k_src=k_src, q_mla=q_mla, kv_cache=kv)


def make_random_indices(batch, topk, seed, device):
    """Synthetic index lists for testing attention on its own: for each query
    token, min(topk, pos+1) distinct positions drawn uniformly from 0..pos,
    ascending, then -1 up to width topk."""
    rows = []
    g = torch_gen(seed, device)
    for b in range(batch.num_reqs):
        L, ql = batch.seq_lens[b], batch.q_lens[b]
        for i in range(ql):
            pos = L - ql + i
            n = min(topk, pos + 1)
            r = torch.rand(pos + 1, generator=g, device=device)
            pick = torch.topk(r, n, largest=False).indices.to(torch.int32)
            pick, _ = torch.sort(pick)
            row = torch.full((topk,), -1, dtype=torch.int32, device=device)
            row[:n] = pick
            rows.append(row)
    if not rows:
        return torch.empty((0, topk), dtype=torch.int32, device=device)
    return torch.stack(rows)


@dataclass
class PrologueInputs:
    hidden: torch.Tensor        # [N, hidden_dim] bf16
    qa_normed: torch.Tensor     # [N, q_lora_rank] bf16
    cos: torch.Tensor           # [N, R/2] fp32
    sin: torch.Tensor
    wq_b: torch.Tensor          # [H * D, q_lora_rank] bf16
    wk: torch.Tensor            # [D, hidden_dim] bf16
    weights_proj: torch.Tensor  # [H, hidden_dim] bf16
    k_norm_weight: torch.Tensor  # [D] fp32


def make_prologue(cfg, batch, device, layer=0, n_tokens=None):
    """Synthetic inputs of the indexer prologue for the batch's query tokens:
    activations N(0,1), weights N(0, 1/fan_in) (linear-layer layout), k_norm
    weight 1 + N(0, 0.1^2), RoPE angles pos * 10000^(-2j/R) at each token's
    position."""
    base = 1000 * cfg.cid + 100 * layer
    N = batch.num_q_tokens if n_tokens is None else n_tokens
    H, D, R = cfg.n_idx_heads, cfg.d_idx, cfg.idx_rope_dim
    bf = torch.bfloat16
    hidden = _normal((N, cfg.hidden_dim), bf, base + _ID_HID, device)
    qa = _normal((N, cfg.q_lora_rank), bf, base + _ID_QA, device)
    wq_b = _normal((H * D, cfg.q_lora_rank), bf, base + _ID_WQB, device,
                   scale=1.0 / math.sqrt(cfg.q_lora_rank))
    wk = _normal((D, cfg.hidden_dim), bf, base + _ID_WK, device,
                 scale=1.0 / math.sqrt(cfg.hidden_dim))
    wp = _normal((H, cfg.hidden_dim), bf, base + _ID_WP, device,
                 scale=1.0 / math.sqrt(cfg.hidden_dim))
    knw = 1.0 + _normal((D,), torch.float32, base + _ID_KNW, device, scale=0.1)
    pos = []
    for b in range(batch.num_reqs):
        L, ql = batch.seq_lens[b], batch.q_lens[b]
        pos += [L - ql + i for i in range(ql)]
    pos = (pos + [0] * N)[:N]
    j = torch.arange(R // 2, dtype=torch.float64)
    ang = torch.tensor(pos, dtype=torch.float64)[:, None] * torch.pow(10000.0, -2.0 * j / R)
    return PrologueInputs(hidden=hidden, qa_normed=qa,
                          cos=torch.cos(ang).to(torch.float32).to(device),
                          sin=torch.sin(ang).to(torch.float32).to(device),
                          wq_b=wq_b, wk=wk, weights_proj=wp, k_norm_weight=knw)
