"""Oracle for the DSA ("lightning") indexer: key-cache write, score, top-k.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page "GLM5 TensorCast 适配设计" = GLM5 TensorCast adaptation design):
  * section "DSA Indexer fused semantic op": the op takes the indexer cache as
    a mutable argument addressed by slot_mapping / block_tables / seq_lens,
    writes the new keys (FP8 path: key cache plus scale cache), scores the
    cache ("cache scoring, head weight mixing, head reduction") and selects
    top-k; the result has shape (batch, seq_len, min(topk_limit,
    active_seq_len)), and a static width topk_limit where lengths are unknown.
  * section "Performance model design", buckets 6-8: q-k index score MMA;
    head-weight multiply, head reduce and ReLU shaping; top-k selection.
  * the score is score[t, s] = sum_h w[t, h] * ReLU(q[t, h, :] . k[s, :]).
    ReLU is applied on every cache dtype (the bf16 path's list omits the
    word, the FP8 path names "relu/q-scale/k-scale shaping"; the reading
    taken is that only the scale factors are FP8-specific).
Page "GLM5 full-stack LoRA" section 1 and section 2.1: torch.topk tie order
is not reproducible across builds; the selection here is deterministic with
ties broken toward the lower position.

Readings fixed here (the pages leave them open):
  * indices are logical positions 0..seq_len-1 of the request; the physical
    slot of position s is block_table[b, s // block_size] * block_size
    + s % block_size;
  * query i of request b (q_len_b queries) sits at position
    seq_len_b - q_len_b + i and sees keys 0..pos (the cache already holds
    this step's keys when scoring runs);
  * the row holds the n = min(topk, pos + 1) selected positions in ascending
    order, then -1 up to the static width topk;
  * FP8 cache write: per token, amax = max_d |k_d| in fp32, scale =
    fl32(amax / 448) (1 when amax == 0), code_d = e4m3_RNE_sat(fl32(k_d /
    scale)); the key's value is code * scale.
"""

import numpy as np

from . import codecs

F32, BF16, FP8 = "f32", "bf16", "fp8"


# --------------------------------------------------------------------------
# key-cache write
# --------------------------------------------------------------------------
def fp8_quantize_rows(k32):
    """Keys [n, d] (float32) -> (e4m3 codes [n, d], fp32 scales [n]).

    Per row: amax = max |k| (exact), scale = fl32(amax / 448) or 1 when
    amax == 0, code = e4m3(fl32(k / scale)).  NumPy float32 division is
    IEEE round-to-nearest-even.
    """
    k32 = np.asarray(k32, dtype=np.float32)
    amax = np.max(np.abs(k32), axis=1) if k32.shape[1] else np.zeros(k32.shape[0], np.float32)
    scale = np.where(amax == 0, np.float32(1.0),
                     (amax / np.float32(codecs.E4M3_MAX)).astype(np.float32)).astype(np.float32)
    v = (k32 / scale[:, None]).astype(np.float32)
    return codecs.f32_to_e4m3(v), scale


def fp8_quantize_token(k32):
    """One token's key (float32 vector) -> (e4m3 codes, fp32 scale)."""
    codes, scale = fp8_quantize_rows(np.asarray(k32, dtype=np.float32)[None, :])
    return codes[0], scale[0]


def cache_write(k_new, slot_mapping, cache, scale=None, cache_dtype=BF16):
    """Write new keys into the paged indexer cache (returns updated copies).

    k_new        float32 array [n, d] holding the exact new key values
                 (an fp32 key, or a bf16 key widened to fp32)
    slot_mapping int array [n]; -1 marks a padding token that is skipped
    cache        f32: float32 [slots, d]; bf16: uint16 bit patterns;
                 fp8: uint8 codes
    scale        float32 [slots] for the fp8 cache, else None
    """
    cache = cache.copy()
    scale = None if scale is None else scale.copy()
    k_new = np.asarray(k_new, dtype=np.float32)
    for i, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        if cache_dtype == F32:
            cache[slot] = k_new[i]
        elif cache_dtype == BF16:
            bits = k_new[i].view(np.uint32)
            if np.any(bits & 0xFFFF):
                raise ValueError("bf16 cache write expects bf16-exact keys")
            cache[slot] = (bits >> 16).astype(np.uint16)
        elif cache_dtype == FP8:
            codes, s = fp8_quantize_token(k_new[i])
            cache[slot] = codes
            scale[slot] = s
        else:
            raise ValueError(cache_dtype)
    return cache, scale


def key_values(cache, scale, cache_dtype, slots):
    """Exact float64 value of the keys stored at the given slots."""
    rows = cache[np.asarray(slots)]
    if cache_dtype == F32:
        return rows.astype(np.float64)
    if cache_dtype == BF16:
        return codecs.bf16_to_f64(rows)
    if cache_dtype == FP8:
        return codecs.e4m3_to_f64(rows) * scale[np.asarray(slots)].astype(
            np.float64)[:, None]
    raise ValueError(cache_dtype)


# --------------------------------------------------------------------------
# score and selection
# --------------------------------------------------------------------------
def positions_of_request(seq_len, q_len):
    """Positions of the q_len query tokens of a request with seq_len keys."""
    return [seq_len - q_len + i for i in range(q_len)]


def physical_slots(block_table_row, block_size, n):
    s = np.arange(n)
    return np.asarray(block_table_row)[s // block_size] * block_size + s % block_size


def indexer_scores(q_t, w_t, keys):
    """score[s] = sum_h w[h] * max(q[h] . k[s], 0), all in float64.

    q_t [H, d], w_t [H], keys [L, d] -> [L]
    """
    logits = keys @ np.asarray(q_t, dtype=np.float64).T        # [L, H]
    return np.maximum(logits, 0.0) @ np.asarray(w_t, dtype=np.float64)


def select_topk(score, topk):
    """Deterministic top-k of one row.

    Picks n = min(topk, len(score)) positions, ordered by (score descending,
    position ascending); returns them in ascending position, padded with -1
    to width topk.  -0.0 and +0.0 compare equal, so their tie falls to the
    position.
    """
    score = np.asarray(score, dtype=np.float64)
    L = score.shape[0]
    n = min(topk, L)
    pos = np.arange(L)
    order = np.lexsort((pos, -score))      # last key is the primary key
    chosen = np.sort(order[:n])
    out = np.full(topk, -1, dtype=np.int32)
    out[:n] = chosen
    return out


def indexer_topk(seq_lens, cu_q, block_table, block_size, q, w, cache, scale,
                 cache_dtype, topk, tokens=None):
    """Top-k indices for every query token (or only the listed ones).

    q [N, H, d] and w [N, H] are float64 (exact values of the inputs).
    Returns int32 [N, topk] (rows not requested stay -1).
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N = q.shape[0]
    out = np.full((N, topk), -1, dtype=np.int32)
    want = set(range(N)) if tokens is None else set(int(t) for t in tokens)
    B = len(seq_lens)
    for b in range(B):
        t0, t1 = int(cu_q[b]), int(cu_q[b + 1])
        qlen = t1 - t0
        L = int(seq_lens[b])
        todo = [t for t in range(t0, t1) if t in want]
        if not todo:
            continue
        keys_all = key_values(cache, scale, cache_dtype,
                              physical_slots(block_table[b], block_size, L))
        positions = positions_of_request(L, qlen)
        for t in todo:
            pos = positions[t - t0]
            sc = indexer_scores(q[t], w[t], keys_all[:pos + 1])
            out[t] = select_topk(sc, topk)
    return out
