"""Pins for the oracle's indexer prologue (CPU only): projections, RMSNorm
k_norm and rotate-half RoPE (page "GLM5 TensorCast 适配设计", section "DSA
Indexer fused semantic op", the op's inputs; section "Performance model
design", buckets 1-4)."""
import json
import os

import numpy as np
import pytest

from oracle import prologue as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prologue_worked_example.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def _run(g):
    return P.prologue(g["hidden"], g["qa_normed"], g["cos"], g["sin"], g["wq_b"], g["wk"],
                      g["weights_proj"], g["k_norm_weight"], g["n_heads"], g["head_dim"],
                      g["rope_dim"], g["eps"])


def _matches(g):
    q, k, w = _run(g)
    return (np.allclose(q, g["q"], rtol=0, atol=1e-14) and np.allclose(k, g["k"], rtol=0, atol=1e-14)
            and np.allclose(w, g["w"], rtol=0, atol=1e-14))


def test_worked_example():
    g = _g()
    assert _matches(g)
    # the intermediate steps by hand
    qa, wq = np.array(g["qa_normed"]), np.array(g["wq_b"], float)
    assert np.array_equal(qa @ wq.T, g["q_projected"])
    kp = np.array(g["hidden"]) @ np.array(g["wk"], float).T
    assert np.array_equal(kp, g["k_projected"])
    assert np.allclose(P.rms_norm(kp, g["k_norm_weight"], 0.0), g["k_normed"], atol=1e-15)


def test_rms_norm_properties():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((20, 128))
    y = P.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    assert np.allclose(P.rms_norm(7.5 * x, np.ones(128), 0.0), y, atol=1e-14)   # scale free
    assert np.allclose(P.rms_norm([3.0, 4.0], [1.0, 1.0], 0.0),
                       [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], atol=1e-15)
    # eps keeps a zero row finite
    assert np.all(P.rms_norm(np.zeros(8), np.ones(8), 1e-5) == 0)


def test_rope_properties():
    rng = np.random.default_rng(1)
    R, D = 64, 128
    x = rng.standard_normal((30, D))
    cos, sin = P.rope_angles(np.arange(30), R)
    y = P.rope(x, cos, sin, R)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    assert np.array_equal(y[:, R:], x[:, R:])                    # dims past R untouched
    assert np.allclose(P.rope(x, np.ones((30, R // 2)), np.zeros((30, R // 2)), R), x)
    back = P.rope(y, cos, -sin, R)                               # the inverse angle
    assert np.allclose(back, x, atol=1e-12)
    # relative positions: rope(q, m) . rope(k, n) depends on m - n only
    q, k = rng.standard_normal((2, D))
    def dot(m, n):
        cm, sm = P.rope_angles([m], R)
        cn, sn = P.rope_angles([n], R)
        return float(P.rope(q[None], cm, sm, R)[0] @ P.rope(k[None], cn, sn, R)[0])
    assert abs(dot(5, 2) - dot(105, 102)) < 1e-10
    assert abs(dot(5, 2) - dot(2, 5)) > 1e-3


def test_rope_broadcasts_over_heads():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 4, 16))
    cos, sin = P.rope_angles([1, 7, 30], 8)
    y = P.rope(x, cos, sin, 8)
    for h in range(4):
        assert np.allclose(y[:, h], P.rope(x[:, h], cos, sin, 8))


def test_planted_mistakes_fail_the_worked_example(monkeypatch):
    g = _g()
    real = P.rope

    def interleaved(x, cos, sin, rope_dim):       # pairs (2j, 2j + 1)
        x = np.array(x, dtype=np.float64)
        perm = list(range(0, rope_dim, 2)) + list(range(1, rope_dim, 2))
        inv = np.argsort(perm + list(range(rope_dim, x.shape[-1])))
        xp = x[..., perm + list(range(rope_dim, x.shape[-1]))]
        return real(xp, cos, sin, rope_dim)[..., inv]

    def last_dims(x, cos, sin, rope_dim):          # RoPE on the last R dims
        x = np.array(x, dtype=np.float64)
        D = x.shape[-1]
        perm = list(range(D - rope_dim, D)) + list(range(D - rope_dim))
        return real(x[..., perm], cos, sin, rope_dim)[..., np.argsort(perm)]

    def layer_norm(x, weight, eps):                # LayerNorm instead of RMSNorm
        x = np.asarray(x, dtype=np.float64)
        x = x - x.mean(axis=-1, keepdims=True)
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps + 1e-12) * weight

    for name, bad in (("rope", interleaved), ("rope", last_dims), ("rms_norm", layer_norm)):
        monkeypatch.setattr(P, name, bad)
        assert not _matches(g), (name, bad.__name__)
        monkeypatch.undo()
    assert _matches(g)
