"""Pins for the oracle's absorbed sparse MLA (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import mla

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mla_worked_example.json")


def test_worked_example():
    with open(GOLDEN) as f:
        g = json.load(f)
    out, lse = mla.attend(np.array([g["q"]]), np.array(g["rows"]), 1, 1.0)
    assert abs(out[0, 0] - g["out"]) < 1e-15
    assert abs(lse[0] - g["lse"]) < 1e-15


def _case(seed, T=40, H=3, R=6, P=2):
    rng = np.random.default_rng(seed)
    D = R + P
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    return q, kv, R, 1.0 / math.sqrt(D)


@pytest.mark.parametrize("seed", range(4))
def test_sparse_equals_dense_when_k_covers_context(seed):
    q, kv, R, sc = _case(seed)
    T = q.shape[0]
    pos = np.arange(T)
    d_out, d_lse = mla.dense_causal_mla(q, kv, pos, R, sc)
    bt = np.array([[0]])
    idx = np.full((T, T + 3), -1, np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)
    s_out, s_lse = mla.sparse_mla([T], [0, T], bt, T + 3, q, lambda s: kv[s],
                                  idx, R, sc)
    assert np.allclose(s_out, d_out, atol=1e-13, rtol=1e-12)
    assert np.allclose(s_lse, d_lse, atol=1e-13, rtol=1e-12)


def test_first_position_row_is_the_value():
    q, kv, R, sc = _case(11)
    out, lse = mla.attend(q[0], kv[:1], R, sc)
    for h in range(q.shape[1]):
        assert np.array_equal(out[h], kv[0, :R])
        assert abs(lse[h] - sc * q[0, h] @ kv[0]) < 1e-14


def test_uniform_logits_give_mean_and_log_n():
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((9, 5))
    out, lse = mla.attend(np.zeros((2, 5)), rows, 3, 0.7)
    assert np.allclose(out, rows[:, :3].mean(axis=0), atol=1e-15)
    assert np.allclose(lse, math.log(9), atol=1e-15)


def test_permutation_invariance_hull_and_lse():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 10))
    rows = rng.standard_normal((30, 10))
    out, lse = mla.attend(q, rows, 8, 0.3)
    perm = rng.permutation(30)
    out2, lse2 = mla.attend(q, rows[perm], 8, 0.3)
    assert np.allclose(out, out2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)
    assert np.all(out <= rows[:, :8].max(axis=0) + 1e-14)
    assert np.all(out >= rows[:, :8].min(axis=0) - 1e-14)
    z = 0.3 * q @ rows.T
    assert np.allclose(lse, np.log(np.exp(z).sum(axis=1)), atol=1e-13)


def test_padding_indices_are_ignored_and_empty_row():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 2, 4))
    kv = rng.standard_normal((8, 4))
    bt = np.array([[0]])
    idx = np.array([[3, 5, -1, -1], [-1, -1, -1, -1]], np.int32)
    out, lse = mla.sparse_mla([8], [0, 2], bt, 8, q, lambda s: kv[s], idx, 3, 0.5)
    o_ref, l_ref = mla.attend(q[0], kv[[3, 5]], 3, 0.5)
    assert np.array_equal(out[0], o_ref) and np.array_equal(lse[0], l_ref)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_pins_catch_planted_mistakes():
    with open(GOLDEN) as f:
        g = json.load(f)
    q = np.array([g["q"]])
    rows = np.array(g["rows"])
    # value taken from the rope tail instead of the latent head
    z = q @ rows.T
    p = np.exp(z) / np.exp(z).sum()
    assert abs((p @ rows[:, 1:])[0, 0] - g["out"]) > 1e-3
    # softmax without the max shift is still right; a missing scale is not
    q2 = np.array([[2.0, 0.0]])
    out_s, _ = mla.attend(q2, rows, 1, 0.5)
    out_n, _ = mla.attend(q2, rows, 1, 1.0)
    assert abs(out_s[0, 0] - g["out"]) < 1e-15
    assert abs(out_n[0, 0] - g["out"]) > 1e-3
