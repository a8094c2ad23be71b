"""Pins for the oracle's indexer: cache write, score and top-k (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import codecs, indexer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "indexer_worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example
def test_worked_example_scores_and_topk():
    g = _golden()
    q = np.array(g["q"], dtype=np.float64)
    keys = np.array(g["keys"], dtype=np.float64)
    for case in g["cases"]:
        sc = indexer.indexer_scores(q, np.array(case["w"], dtype=np.float64), keys)
        assert sc.tolist() == case["scores"]
        for k, want in case["topk"].items():
            got = indexer.select_topk(sc, int(k))
            assert got.tolist() == want, (case["w"], k)


def test_worked_example_paged_causal():
    g = _golden()["paged"]
    bs = g["block_size"]
    bt = np.array([g["block_table"]], dtype=np.int32)
    slots = indexer.physical_slots(bt[0], bs, g["seq_len"])
    assert slots.tolist() == g["slots"]
    assert indexer.positions_of_request(g["seq_len"], g["q_len"]) == g["query_positions"]
    keys = np.array(_golden()["keys"], dtype=np.float32)
    cache = np.zeros((bt.max() * bs + bs, 2), dtype=np.float32)
    cache[slots] = keys
    q = np.array(_golden()["q"], dtype=np.float64)
    qq = np.stack([q, q])
    ww = np.array([g["w"], g["w"]], dtype=np.float64)
    for k, rows in ((2, g["topk2_rows"]), (3, g["topk3_rows"])):
        got = indexer.indexer_topk([g["seq_len"]], [0, g["q_len"]], bt, bs, qq, ww,
                                   cache, None, indexer.F32, k)
        assert got.tolist() == rows


# ---------------------------------------------------------------- brute force
def _brute_scores(q, w, keys):
    """Python-integer arithmetic, loop by loop (inputs are integers)."""
    H, d = len(q), len(q[0])
    out = []
    for k in keys:
        s = 0
        for h in range(H):
            dot = sum(int(q[h][i]) * int(k[i]) for i in range(d))
            s += int(w[h]) * max(dot, 0)
        out.append(s)
    return out


def _brute_topk(scores, k):
    pairs = sorted(((s, -p) for p, s in enumerate(scores)), reverse=True)
    chosen = sorted(-mp for _, mp in pairs[:min(k, len(scores))])
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_brute_force_full_sort(seed):
    rng = np.random.default_rng(seed)
    H = int(rng.integers(1, 5))
    d = int(rng.integers(1, 9))
    L = int(rng.integers(1, 70))
    q = rng.integers(-3, 4, size=(H, d))
    w = rng.integers(-2, 3, size=H)
    keys = rng.integers(-3, 4, size=(L, d))
    brute = _brute_scores(q.tolist(), w.tolist(), keys.tolist())
    sc = indexer.indexer_scores(q.astype(np.float64), w.astype(np.float64),
                                keys.astype(np.float64))
    assert sc.tolist() == [float(x) for x in brute]
    for k in (1, 2, 3, 5, 8, 16, L, L + 3):
        assert indexer.select_topk(sc, k).tolist() == _brute_topk(brute, k)


@pytest.mark.parametrize("seed", range(6))
def test_topk_with_float_scores_and_forced_ties(seed):
    rng = np.random.default_rng(100 + seed)
    L = 300
    sc = rng.standard_normal(L)
    # force runs of equal values, including zeros of both signs
    sc[rng.integers(0, L, 40)] = sc[5]
    sc[rng.integers(0, L, 20)] = 0.0
    sc[rng.integers(0, L, 20)] = -0.0
    for k in (1, 7, 64, 150, 299, 300, 301):
        got = indexer.select_topk(sc, k)
        assert got.tolist() == _brute_topk(sc.tolist(), k)


def test_negative_zero_ties_fall_to_position():
    sc = np.array([-0.0, 0.0, -0.0, 0.0])
    assert indexer.select_topk(sc, 2).tolist() == [0, 1]
    sc = np.array([0.0, -0.0, -1.0, -0.0])
    assert indexer.select_topk(sc, 2).tolist() == [0, 1]


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("seed", range(4))
def test_row_invariants_and_threshold_certificate(seed):
    rng = np.random.default_rng(200 + seed)
    L = int(rng.integers(50, 2000))
    sc = np.round(rng.standard_normal(L) * 4) / 4    # many ties
    for k in (1, 16, 100, L // 2, L, L + 10):
        row = indexer.select_topk(sc, k)
        n = min(k, L)
        sel = row[:n]
        assert np.all(row[n:] == -1)
        assert np.all(np.diff(sel) > 0)               # ascending, unique
        assert sel.min() >= 0 and sel.max() < L
        # certificate: every unselected (score, -pos) is below every selected
        mask = np.ones(L, bool)
        mask[sel] = False
        if mask.any() and n:
            worst_sel = min((sc[p], -p) for p in sel)
            best_out = max((sc[p], -p) for p in np.nonzero(mask)[0])
            assert best_out < worst_sel


def test_k_at_least_context_selects_everything():
    rng = np.random.default_rng(7)
    for L in (1, 2, 17, 64):
        sc = rng.standard_normal(L)
        row = indexer.select_topk(sc, L)
        assert row.tolist() == list(range(L))
        row = indexer.select_topk(sc, L + 5)
        assert row.tolist() == list(range(L)) + [-1] * 5


def test_relu_is_applied_per_head_before_mixing():
    # one head with a negative logit must contribute 0, not its negative
    q = np.array([[1.0], [1.0]])
    w = np.array([1.0, 1.0])
    keys = np.array([[-2.0], [1.0]])
    assert indexer.indexer_scores(q, w, keys).tolist() == [0.0, 2.0]


# ---------------------------------------------------------------- FP8 cache write
def test_fp8_quantize_end_points_and_error_bound():
    rng = np.random.default_rng(3)
    for _ in range(50):
        k = rng.standard_normal(128).astype(np.float32)
        codes, scale = indexer.fp8_quantize_token(k)
        assert scale == np.float32(np.max(np.abs(k)) / np.float32(448))
        i = int(np.argmax(np.abs(k)))
        assert codes[i] == (0xFE if k[i] < 0 else 0x7E)
        deq = codecs.e4m3_to_f64(codes) * np.float64(scale)
        # error of one e4m3 rounding of k/scale (relative 2^-4 for normals,
        # absolute 2^-10 * scale in the subnormal range) plus the fp32 division
        v = np.abs(k.astype(np.float64) / np.float64(scale))
        bound = np.maximum(v * 2.0 ** -4, 2.0 ** -10) * np.float64(scale) * (1 + 1e-6)
        assert np.all(np.abs(deq - k) <= bound)


def test_fp8_zero_key_and_padding_slot():
    cache = np.full((4, 8), 0xAA, dtype=np.uint8)
    scale = np.full(4, 7.0, dtype=np.float32)
    k = np.zeros((2, 8), dtype=np.float32)
    k[1, 3] = -2.0
    c2, s2 = indexer.cache_write(k, [2, -1], cache, scale, indexer.FP8)
    assert np.all(c2[2] == 0) and s2[2] == 1.0
    assert np.array_equal(c2[[0, 1, 3]], cache[[0, 1, 3]])   # others untouched
    assert np.array_equal(s2[[0, 1, 3]], scale[[0, 1, 3]])
    c3, s3 = indexer.cache_write(k, [-1, 0], cache, scale, indexer.FP8)
    assert s3[0] == np.float32(2.0 / 448.0)
    assert c3[0, 3] == 0xFE and np.all(np.delete(c3[0], 3) == 0)


def test_bf16_and_f32_cache_write_copy_bits():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((3, 4)).astype(np.float32)
    c, _ = indexer.cache_write(k, [1, 0, -1], np.zeros((3, 4), np.float32), None, indexer.F32)
    assert np.array_equal(c[1], k[0]) and np.array_equal(c[0], k[1]) and np.all(c[2] == 0)
    kb = (k.view(np.uint32) & 0xFFFF0000).view(np.float32)
    c, _ = indexer.cache_write(kb, [2, -1, 0], np.zeros((3, 4), np.uint16), None, indexer.BF16)
    assert np.array_equal(c[2], (kb[0].view(np.uint32) >> 16).astype(np.uint16))
    assert np.array_equal(codecs.bf16_to_f64(c[0]), kb[2].astype(np.float64))


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check a pin fails."""
    g = _golden()
    q = np.array(g["q"], dtype=np.float64)
    keys = np.array(g["keys"], dtype=np.float64)
    case = g["cases"][1]
    w = np.array(case["w"], dtype=np.float64)

    def no_relu(q_t, w_t, keys):
        return (keys @ q_t.T) @ w_t

    def relu_after_mix(q_t, w_t, keys):
        return np.maximum((keys @ q_t.T) @ w_t, 0)

    for bad in (no_relu, relu_after_mix):
        assert bad(q, w, keys).tolist() != case["scores"]

    def ties_to_higher(score, topk):
        L = len(score)
        n = min(topk, L)
        order = np.lexsort((-np.arange(L), -np.asarray(score)))
        out = np.full(topk, -1, np.int32)
        out[:n] = np.sort(order[:n])
        return out

    sc = np.array(case["scores"], dtype=np.float64)
    assert ties_to_higher(sc, 3).tolist() != case["topk"]["3"]


# ---------------------------------------------------------------- integer workload
def test_tiny_prefill_workload_against_brute_force():
    """The integer-valued workload end to end (paging, causal positions):
    exact scores, so every row must equal the brute-force selection."""
    import torch
    from synth import get_config, make_batch, make_layer
    cfg = get_config("tiny_prefill")
    b = make_batch(cfg, "cpu")
    lay = make_layer(cfg, b, "cpu")
    cache = lay.k_src.numpy()
    q = lay.q_idx.numpy().astype(np.float64)
    w = lay.w.numpy().astype(np.float64)
    rows = [0, 1, 15, 16, 17, 100, 255]
    got = indexer.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host,
                               b.block_size, q, w, cache, None, indexer.F32,
                               cfg.topk, tokens=rows)
    slots = indexer.physical_slots(b.block_table_host[0], b.block_size, 256)
    keys = cache[slots].astype(np.int64).tolist()
    for t in rows:
        brute = _brute_scores(q[t].astype(np.int64).tolist(),
                              w[t].astype(np.int64).tolist(), keys[:t + 1])
        assert got[t].tolist() == _brute_topk(brute, cfg.topk), t
