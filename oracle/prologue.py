"""Oracle for the indexer prologue: the q / k / w projections, k_norm and
RoPE that produce the indexer's inputs, then the key's cache write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page "GLM5 TensorCast 适配设计" = GLM5 TensorCast adaptation design):
  * section "mlapo / mlapo_quant and qa_normed": the indexer reuses the MLA
    path's normalised query low-rank activation qa_normed;
  * section "DSA Indexer fused semantic op": the op's inputs are
    hidden_states, qa_normed, the RoPE cos / sin, the indexer cache with
    slot_mapping / block_tables / seq_lens, wq_b_weight, wk_weight,
    weights_proj_weight, k_norm_weight, num_heads, head_dim,
    qk_rope_head_dim and topk_limit; both paths include the query / key
    projection and RoPE, the FP8 path adds rotation and quantisation;
  * section "Performance model design", buckets 1-4: q projection
    qa_normed @ wq_b, k projection hidden_states @ wk, head routing
    projection hidden_states @ weights_proj, RoPE.
  * section "RMSNorm non-default epsilon pattern matching": GLM5's norms are
    RMSNorms with a non-default epsilon (1e-5).

Readings fixed here (the pages name the steps, not their formulas):
  * weights are stored as linear-layer weights, [out_features, in_features]:
    q = qa_normed W_qb^T reshaped [N, H, D]; k = hidden W_k^T [N, D];
    w = hidden W_wp^T [N, H] (no extra scaling: a positive rescale of w
    cannot change the top-k);
  * k_norm is an RMSNorm with the given weight: k / sqrt(mean(k^2) + eps) *
    weight, applied to the projected key before RoPE;
  * RoPE acts on the first qk_rope_head_dim = R dims of each query head and
    of the key, rotate-half style: dim j and dim j + R/2 (j < R/2) form a
    pair turned by the token's angle theta_j: cos / sin arrive as [N, R/2]
    per token;
  * the key is then written to the cache like any new key (a bf16 copy; the
    FP8 path rotates and quantises it, see fp8_indexer).
"""

import numpy as np


def rms_norm(x, weight, eps):
    """x [..., D] -> x / sqrt(mean(x^2) + eps) * weight, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def rope(x, cos, sin, rope_dim):
    """Rotate-half RoPE on the first rope_dim dims of x [..., D]: for
    j < rope_dim / 2, (x_j, x_{j+R/2}) -> (x_j cos_j - x_{j+R/2} sin_j,
    x_{j+R/2} cos_j + x_j sin_j).  cos / sin [..., R/2] broadcast over any
    middle (head) dims."""
    x = np.array(x, dtype=np.float64)
    h = rope_dim // 2
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    while c.ndim < x.ndim:             # [N, R/2] -> [N, 1, R/2] for heads
        c = c[..., None, :]
        s = s[..., None, :]
    a = x[..., :h].copy()
    b = x[..., h:rope_dim].copy()
    x[..., :h] = a * c - b * s
    x[..., h:rope_dim] = b * c + a * s
    return x


def rope_angles(positions, rope_dim, base=10000.0):
    """cos, sin [N, R/2] of the usual inverse-frequency angles pos *
    base^(-2 j / R) (only used to build inputs; RoPE itself takes any
    cos / sin)."""
    j = np.arange(rope_dim // 2, dtype=np.float64)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * base ** (-2.0 * j / rope_dim)
    return np.cos(ang), np.sin(ang)


def prologue(hidden, qa_normed, cos, sin, wq_b, wk, weights_proj, k_norm_weight,
             n_heads, head_dim, rope_dim, eps):
    """The indexer's inputs for N tokens, in float64.
    hidden [N, hidden_dim], qa_normed [N, q_lora_rank], cos / sin [N, R/2],
    wq_b [H * D, q_lora_rank], wk [D, hidden_dim], weights_proj [H, hidden_dim],
    k_norm_weight [D] -> q [N, H, D], k [N, D], w [N, H]."""
    hidden = np.asarray(hidden, dtype=np.float64)
    qa = np.asarray(qa_normed, dtype=np.float64)
    N = hidden.shape[0]
    q = (qa @ np.asarray(wq_b, dtype=np.float64).T).reshape(N, n_heads, head_dim)
    q = rope(q, cos, sin, rope_dim)
    k = rms_norm(hidden @ np.asarray(wk, dtype=np.float64).T, k_norm_weight, eps)
    k = rope(k, cos, sin, rope_dim)
    w = hidden @ np.asarray(weights_proj, dtype=np.float64).T
    return q, k, w
