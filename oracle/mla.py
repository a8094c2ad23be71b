"""Oracle for absorbed sparse MLA over the selected latent rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: page "GLM5 TensorCast 适配设计" (GLM5 TensorCast adaptation
design), section "DSA Indexer fused semantic op": the indexer hands
topk_limit and topk_indices to the MLA backend, which limits attention to the
selected positions; section "Performance model design": the sparse attention
length is the width of topk_indices (or topk_limit).  Page "GLM5 full-stack
LoRA", section 2.2: absorbed MLA, where queries are projected into the latent
space so attention runs directly over the cached latent rows.

Readings fixed here:
  * a latent row holds kv_lora_rank latent dims followed by rope dims; the
    key is the whole row, the value is its first kv_lora_rank dims, and the
    output stays in latent space (the up-projection is outside the path);
  * z[h, j] = softmax_scale * q[h, :] . kv[j, :], p = softmax_j z,
    out[h, :] = sum_j p[h, j] kv[j, :R], lse[h] = log sum_j exp z[h, j];
  * index -1 means "no key"; a token with no valid index has out = 0 and
    lse = -inf.
"""

import numpy as np


def attend(q_t, kv_sel, kv_lora_rank, softmax_scale):
    """One token, all heads, over the given latent rows.

    q_t [H, D], kv_sel [n, D] float64 -> (out [H, R], lse [H])
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    kv_sel = np.asarray(kv_sel, dtype=np.float64)
    H = q_t.shape[0]
    R = kv_lora_rank
    if kv_sel.shape[0] == 0:
        return np.zeros((H, R)), np.full(H, -np.inf)
    z = softmax_scale * (q_t @ kv_sel.T)                  # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    p = e / s
    out = p @ kv_sel[:, :R]
    lse = (m + np.log(s))[:, 0]
    return out, lse


def sparse_mla(seq_lens, cu_q, block_table, block_size, q, kv_values,
               topk_idx, kv_lora_rank, softmax_scale, tokens=None):
    """Sparse MLA for every query token (or only the listed ones).

    q [N, H, D] float64; kv_values(slots) -> float64 rows [len(slots), D];
    topk_idx [N, k] logical positions (-1 = none).
    Returns out [N, H, R] and lse [N, H] (unrequested rows are NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    N, H, _ = q.shape
    out = np.full((N, H, kv_lora_rank), np.nan)
    lse = np.full((N, H), np.nan)
    want = range(N) if tokens is None else tokens
    for t in want:
        b = request_of_token(cu_q, t)
        idx = np.asarray(topk_idx[t])
        idx = idx[idx >= 0]
        out[t], lse[t] = attend(q[t], kv_values(slots_of(block_table, b, idx, block_size)),
                                kv_lora_rank, softmax_scale)
    return out, lse


def request_of_token(cu_q, t):
    """The request that owns query token t: the last b with cu_q[b] <= t."""
    return int(np.searchsorted(np.asarray(cu_q), t, side="right") - 1)


def slots_of(block_table, b, positions, block_size):
    """Physical cache rows of logical positions of request b (its own
    block-table row: block id of position s, times the block size, plus the
    offset of s in its block)."""
    positions = np.asarray(positions)
    return (np.asarray(block_table[b])[positions // block_size] * block_size
            + positions % block_size)


def dense_causal_mla(q, kv, positions, kv_lora_rank, softmax_scale):
    """Dense causal MLA of one request, written as a masked full softmax.

    q [T, H, D], kv [S, D] (logical order), positions [T]; token t attends
    to every s <= positions[t].  Kept separate from ``attend`` so that the
    sparse == dense invariant compares two different formulations.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    T, H, _ = q.shape
    S = kv.shape[0]
    z = softmax_scale * np.einsum("thd,sd->ths", q, kv)      # [T, H, S]
    mask = np.arange(S)[None, :] > np.asarray(positions)[:, None]   # [T, S]
    z = np.where(mask[:, None, :], -np.inf, z)
    m = z.max(axis=2, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=2, keepdims=True)
    out = np.einsum("ths,sr->thr", e / s, kv[:, :kv_lora_rank])
    lse = (m + np.log(s))[:, :, 0]
    return out, lse
