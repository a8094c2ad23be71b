"""Oracle for the FP8-query indexer variant: activation rotation, per-row
activation quantisation, and the score over e4m3 queries and keys.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page "GLM5 TensorCast 适配设计" = GLM5 TensorCast adaptation design):
  * section "DSA Indexer fused semantic op": the DeepSeek-V3.2 FP8 path of the
    indexer applies rotate_activation and activation quantisation, writes the
    FP8 key cache and its scale cache, computes the FP8 index score and
    selects top-k; the bf16 path drops exactly these steps;
  * section "Performance model design", bucket 5 (FP8-only rotate_activation
    and activation quantisation) and bucket 7 (FP8-only ReLU / q-scale /
    k-scale shaping of the score).

Readings fixed here (the pages name the steps, not their formulas):
  * rotate_activation is the orthonormal Hadamard transform of each head
    vector: x -> x H_d with H_d the Sylvester Hadamard matrix scaled by
    d^-1/2 (symmetric, orthogonal, its own inverse), so it preserves every
    dot product and only spreads a vector's energy over its dims before
    quantisation;
  * activation quantisation is the key recipe applied per row: a query row
    is one head of one token (one scale per token and head), a key row is
    one token: scale = fl32(amax / 448) (1 if amax = 0), code =
    e4m3_RNE_sat(fl32(v / scale));
  * the quantisation decision is taken on the rotation as the kernel computes
    it in fp32: the butterfly stages h = 1, 2, 4, ..., d/2 in that order, each
    (a, b) -> (a + b, a - b) rounded to fp32, then one multiply by
    fl32(d^-1/2) (rotate_f32 below).  rotate_f64 is the definition it
    approximates;
  * score[t, s] = k_scale[s] * sum_h w[t, h] * q_scale[t, h] *
    max(qv[t, h, :] . kv[s, :], 0), with qv, kv the e4m3 values of the codes;
    the scales are positive, so this is the bf16-path formula applied to the
    dequantised rotated vectors.
"""

import numpy as np

from . import codecs, indexer


def hadamard(d):
    """Sylvester Hadamard matrix of order d (a power of two), scaled by
    d^-1/2: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def rotate_f64(x):
    """The definition: rows of x (..., d) times H_d, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x @ hadamard(x.shape[-1])


def rotate_f32(x):
    """The same rotation as the kernel rounds it: float32 butterflies over
    h = 1, 2, ..., d/2, then one multiply by fl32(d^-1/2).  Element i is
    paired with i + h inside each block of 2 h."""
    x = np.array(x, dtype=np.float32)
    shape = x.shape
    d = shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    y = x.reshape(-1, d)
    h = 1
    while h < d:
        blk = y.reshape(y.shape[0], d // (2 * h), 2, h)
        a = blk[:, :, 0, :].copy()
        b = blk[:, :, 1, :].copy()
        blk[:, :, 0, :] = a + b
        blk[:, :, 1, :] = a - b
        y = blk.reshape(-1, d)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(d))).reshape(shape)


def rotate_quantize(x):
    """Rows (..., d) of float32 -> (e4m3 codes (..., d), fp32 scales (...,)):
    rotate_f32, then the per-row quantisation of the key recipe."""
    x = np.asarray(x, dtype=np.float32)
    r = rotate_f32(x).reshape(-1, x.shape[-1])
    codes, scales = indexer.fp8_quantize_rows(r)
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1])


def scores(q_codes, q_scale, w, k_codes, k_scale):
    """One query token over its keys.  q_codes [H, d], q_scale [H], w [H],
    k_codes [L, d], k_scale [L] -> [L] float64.  Products and sums of e4m3
    values are exact in float64 (the scales are applied after)."""
    qv = codecs.e4m3_to_f64(q_codes)
    kv = codecs.e4m3_to_f64(k_codes)
    logits = kv @ qv.T                                       # [L, H], exact
    hw = np.asarray(w, np.float64) * np.asarray(q_scale, np.float32).astype(np.float64)
    return (np.maximum(logits, 0.0) @ hw) * np.asarray(k_scale, np.float32).astype(np.float64)


def indexer_topk(seq_lens, cu_q, block_table, block_size, q_codes, q_scale, w,
                 k_codes, k_scale, topk, tokens=None):
    """Top-k rows of the FP8-query path (same selection and row format as
    indexer.indexer_topk).  q_codes [N, H, d] uint8, q_scale / w [N, H];
    k_codes [num_slots, d] uint8 and k_scale [num_slots] hold the rotated,
    quantised keys."""
    N = q_codes.shape[0]
    out = np.full((N, topk), -1, dtype=np.int32)
    want = set(range(N)) if tokens is None else set(int(t) for t in tokens)
    for b in range(len(seq_lens)):
        t0, t1 = int(cu_q[b]), int(cu_q[b + 1])
        todo = [t for t in range(t0, t1) if t in want]
        if not todo:
            continue
        L = int(seq_lens[b])
        slots = indexer.physical_slots(block_table[b], block_size, L)
        kc, ks = k_codes[slots], k_scale[slots]
        positions = indexer.positions_of_request(L, t1 - t0)
        for t in todo:
            pos = positions[t - t0]
            sc = scores(q_codes[t], q_scale[t], w[t], kc[:pos + 1], ks[:pos + 1])
            out[t] = indexer.select_topk(sc, topk)
    return out
