"""Pins for the oracle's FP8-query indexer variant (CPU only): the Hadamard
rotation, its fp32 butterfly form, per-row quantisation of rotated rows, and
the score over e4m3 queries and keys (page "GLM5 TensorCast 适配设计",
section "DSA Indexer fused semantic op", FP8 path; section "Performance
model design", buckets 5 and 7)."""
import json
import os

import numpy as np
import pytest

from oracle import codecs, fp8_indexer as F, indexer as OI

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_query_worked_example.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------ rotation
def test_hadamard_small_orders_by_hand():
    r = 1 / np.sqrt(2)
    assert np.allclose(F.hadamard(2), [[r, r], [r, -r]], rtol=0, atol=1e-16)
    h4 = 0.5 * np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])
    assert np.array_equal(F.hadamard(4), h4)


@pytest.mark.parametrize("d", [2, 4, 8, 32, 64, 128, 256])
def test_hadamard_is_an_orthogonal_involution(d):
    h = F.hadamard(d)
    assert np.allclose(h @ h.T, np.eye(d), atol=1e-13)
    assert np.allclose(h @ h, np.eye(d), atol=1e-13)        # symmetric: its own inverse
    assert np.allclose(np.abs(h), 1 / np.sqrt(d), atol=1e-16)


def test_rotation_preserves_dot_products():
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal((2, 50, 128))
    dots = np.sum(x * y, axis=1)
    rdots = np.sum(F.rotate_f64(x) * F.rotate_f64(y), axis=1)
    assert np.allclose(dots, rdots, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [4, 32, 128])
def test_fp32_butterflies_within_their_rounding_bound(d):
    """Each of the log2(d) stages rounds once, the scaling once more: every
    output is within (log2 d + 1) * 2^-24 * sum |x| / sqrt(d) of the exact
    rotation."""
    rng = np.random.default_rng(d)
    x = (rng.standard_normal((200, d)) * np.exp(rng.standard_normal((200, 1)) * 4)).astype(np.float32)
    exact = F.rotate_f64(x.astype(np.float64))
    got = F.rotate_f32(x).astype(np.float64)
    bound = (np.log2(d) + 1) * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1) / np.sqrt(d)
    assert np.all(np.abs(got - exact) <= bound[:, None] * 1.0001)


def test_rotation_worked_example():
    g = _g()
    assert F.rotate_f32(np.array(g["q"], np.float32)).tolist() == g["q_rotated"]
    assert F.rotate_f64(g["q"]).tolist() == g["q_rotated"]
    assert F.rotate_f32(np.array(g["keys"], np.float32)).tolist() == g["keys_rotated"]


# ------------------------------------------------------------------ quantisation
def test_quantised_rows_worked_example():
    g = _g()
    qc, qs = F.rotate_quantize(np.array([g["q"]], np.float32))
    assert qc[0].tolist() == g["q_codes"] and float(qs[0]) == g["q_scale"]
    kc, ks = F.rotate_quantize(np.array(g["keys"], np.float32))
    assert kc.tolist() == g["k_codes"] and ks.tolist() == g["k_scale"]


def test_quantised_rotated_rows_within_half_a_step():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    codes, scales = F.rotate_quantize(x)
    r = F.rotate_f32(x).astype(np.float64)
    deq = codecs.e4m3_to_f64(codes) * scales.astype(np.float64)[:, None]
    v = np.abs(r / scales.astype(np.float64)[:, None])
    bound = np.maximum(v * 2.0 ** -4, 2.0 ** -10) * scales.astype(np.float64)[:, None] * (1 + 1e-6)
    assert np.all(np.abs(deq - r) <= bound)
    # the largest element of every row lands on +-448
    i = np.argmax(np.abs(r), axis=1)
    assert np.all(np.isin(codes[np.arange(300), i], [0x7E, 0xFE]))


# ------------------------------------------------------------------ score
def test_scores_worked_example():
    g = _g()
    sc = F.scores(np.array([g["q_codes"]], np.uint8), np.array([g["q_scale"]], np.float32),
                  g["w"], np.array(g["k_codes"], np.uint8), np.array(g["k_scale"], np.float32))
    assert sc.tolist() == g["scores"]
    for dot, s, ks in zip(g["code_dots"], g["scores"], g["k_scale"]):
        assert s == dot * g["q_scale"] * ks


def test_fp8_scores_follow_the_bf16_formula_within_quantisation_error():
    """Rotation keeps every q.k, so the FP8 path's scores stay close to the
    unquantised formula; dropping the rotation of either side breaks that."""
    rng = np.random.default_rng(5)
    H, d, L = 8, 128, 400
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = rng.standard_normal((L, d)).astype(np.float32)
    w = rng.standard_normal(H) / np.sqrt(H)
    qc, qs = F.rotate_quantize(q)
    kc, ks = F.rotate_quantize(k)
    got = F.scores(qc, qs, w, kc, ks)
    ref = OI.indexer_scores(q.astype(np.float64), w, k.astype(np.float64))
    err = np.abs(got - ref)
    scale = np.abs(w).sum() * np.sqrt(d) * 1.0
    assert np.max(err) < 0.15 * scale and np.corrcoef(got, ref)[0, 1] > 0.99
    kc2, ks2 = OI.fp8_quantize_rows(k)            # keys not rotated
    bad = F.scores(qc, qs, w, kc2, ks2)
    assert np.corrcoef(bad, ref)[0, 1] < 0.5


def test_fp8q_topk_matches_brute_force():
    rng = np.random.default_rng(9)
    H, d = 4, 32
    bs = 32
    seq_lens, q_lens = [70, 33], [2, 1]
    cu = [0, 2, 3]
    bt = np.array([[2, 0, 4], [1, 3, 0]], dtype=np.int32)
    qc = rng.integers(0, 256, size=(3, H, d)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0                    # no NaN codes
    kc = rng.integers(0, 256, size=(5 * bs, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0
    qs = rng.uniform(0.5, 2, size=(3, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2, size=5 * bs).astype(np.float32)
    w = rng.standard_normal((3, H))
    got = F.indexer_topk(seq_lens, cu, bt, bs, qc, qs, w, kc, ks, 16)
    t = 0
    for b in range(2):
        slots = OI.physical_slots(bt[b], bs, seq_lens[b])
        for i in range(q_lens[b]):
            pos = seq_lens[b] - q_lens[b] + i
            sc = []
            for p in range(pos + 1):
                s = 0.0
                for h in range(H):
                    dot = sum(codecs.e4m3_value(qc[t, h, j]) * codecs.e4m3_value(kc[slots[p], j])
                              for j in range(d))
                    s += w[t, h] * float(qs[t, h]) * max(dot, 0.0)
                sc.append(s * float(ks[slots[p]]))
            order = sorted(range(pos + 1), key=lambda p: (-sc[p], p))[:16]
            want = sorted(order) + [-1] * (16 - len(order))
            assert got[t].tolist() == want, t
            t += 1


# ------------------------------------------------------------------ planted mistakes
def test_planted_mistakes_fail_the_worked_example(monkeypatch):
    g = _g()
    qc = np.array([g["q_codes"]], np.uint8)
    qs = np.array([g["q_scale"]], np.float32)
    kc = np.array(g["k_codes"], np.uint8)
    ks = np.array(g["k_scale"], np.float32)
    # the query scale left out
    bad = (np.maximum(codecs.e4m3_to_f64(kc) @ codecs.e4m3_to_f64(qc).T, 0) @ np.array(g["w"])) * ks
    assert bad.tolist() != g["scores"]
    # keys quantised without the rotation
    kc2, ks2 = OI.fp8_quantize_rows(np.array(g["keys"], np.float32))
    assert F.scores(qc, qs, g["w"], kc2, ks2).tolist() != g["scores"]
    # the rotation left out of the definition
    monkeypatch.setattr(F, "hadamard", lambda d: np.eye(d))
    assert F.rotate_f64(g["q"]).tolist() != g["q_rotated"]
