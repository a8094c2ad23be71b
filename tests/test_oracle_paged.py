"""Pins for the oracle's paged, multi-request and FP8-cache paths (CPU only).

A hand-worked batch of two requests with permuted block tables and an FP8
key cache whose slots carry distinct scales (tests/golden/
paged_fp8_two_requests.json; page "GLM5 TensorCast 适配设计", section "DSA
Indexer fused semantic op": slot_mapping / block_tables / seq_lens address
the caches, the FP8 path keeps key codes plus a per-token scale).  Unused
slots hold values that would dominate any result that read them.

Each pin is also run against plausible mistakes planted in the oracle
(monkeypatched, on the CPU): dividing by the scale, taking the scale of
the wrong row, the first request's block table for every request, an
off-by-one request lookup.  Every planted mistake must fail a pin."""
import json
import os

import numpy as np
import pytest

from oracle import codecs, indexer as OI, mla as OM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_fp8_two_requests.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def _cache(g):
    return (np.array(g["fp8_codes"], dtype=np.uint8),
            np.array(g["scales"], dtype=np.float32))


# ------------------------------------------------------------------ the pins
def _key_values_ok(g):
    codes, scales = _cache(g)
    # the slots in the order the requests' positions visit them
    slots = g["slots_req1"] + g["slots_req0"]
    got = OI.key_values(codes, scales, OI.FP8, slots)
    return np.array_equal(got, np.array(g["key_values_by_slot"])[slots])


def _topk_ok(g):
    codes, scales = _cache(g)
    bt = np.array(g["block_table"], dtype=np.int32)
    q = np.array(g["q"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    for k, rows in g["topk_rows"].items():
        got = OI.indexer_topk(g["seq_lens"], g["cu_q"], bt, g["block_size"], q, w,
                              codes, scales, OI.FP8, int(k))
        if got.tolist() != rows:
            return False
    return True


def _scores_ok(g):
    codes, scales = _cache(g)
    q = np.array(g["q"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    slots = [g["slots_req0"], g["slots_req1"], g["slots_req1"]]
    for t, want in enumerate(g["scores"].values()):
        keys = OI.key_values(codes, scales, OI.FP8, slots[t][:len(want)])
        if OI.indexer_scores(q[t], w[t], keys).tolist() != want:
            return False
    return True


def _mla_ok(g):
    m = g["mla"]
    kv = np.array(m["kv_rows_by_slot"], dtype=np.float64)
    q = np.zeros((3, 1, 3))
    q[:, 0, 2] = np.log(2.0)
    out, lse = OM.sparse_mla(g["seq_lens"], g["cu_q"], np.array(g["block_table"]),
                             g["block_size"], q, lambda s: kv[np.asarray(s)],
                             np.array(m["topk_idx"], dtype=np.int32), m["kv_lora_rank"],
                             m["softmax_scale"])
    return (np.allclose(out[:, 0, :], m["out"], rtol=0, atol=1e-12)
            and np.allclose(lse[:, 0], m["lse"], rtol=0, atol=1e-12))


def test_golden_is_self_consistent():
    """The hand-listed key values are the code table's values times each
    slot's own scale, and the slot lists follow the block tables."""
    g = _g()
    codes, scales = _cache(g)
    for s in range(g["num_slots"]):
        want = [codecs.e4m3_value(c) * float(scales[s]) for c in codes[s]]
        assert want == g["key_values_by_slot"][s]
    bs = g["block_size"]
    for b, key in ((0, "slots_req0"), (1, "slots_req1")):
        want = [g["block_table"][b][p // bs] * bs + p % bs for p in range(g["seq_lens"][b])]
        assert want == g[key]


def test_fp8_key_values_multiply_by_each_slots_scale():
    assert _key_values_ok(_g())


def test_indexer_scores_over_paged_fp8_keys():
    assert _scores_ok(_g())


def test_indexer_topk_two_requests_permuted_block_tables():
    assert _topk_ok(_g())


def test_sparse_mla_two_requests_permuted_block_tables():
    assert _mla_ok(_g())


# ------------------------------------------------------------------ planted mistakes
def _divide_by_scale(cache, scale, cache_dtype, slots):
    slots = np.asarray(slots)
    return codecs.e4m3_to_f64(cache[slots]) / scale[slots].astype(np.float64)[:, None]


def _scale_of_position(cache, scale, cache_dtype, slots):
    # the scale indexed by the position in the list instead of the slot
    slots = np.asarray(slots)
    return codecs.e4m3_to_f64(cache[slots]) * scale[np.arange(len(slots))].astype(
        np.float64)[:, None]


def _codes_only(cache, scale, cache_dtype, slots):
    return codecs.e4m3_to_f64(cache[np.asarray(slots)])


@pytest.mark.parametrize("bad", [_divide_by_scale, _scale_of_position, _codes_only])
def test_planted_fp8_scale_mistakes_fail_the_pins(monkeypatch, bad):
    g = _g()
    monkeypatch.setattr(OI, "key_values", bad)
    assert not _key_values_ok(g)
    assert not _topk_ok(g)


def test_planted_first_block_table_for_every_request_fails(monkeypatch):
    g = _g()
    bt0 = np.array(g["block_table"][0])
    real = OI.physical_slots
    monkeypatch.setattr(OI, "physical_slots", lambda row, bs, n: real(bt0, bs, n))
    assert not _topk_ok(g)
    monkeypatch.undo()
    realm = OM.slots_of
    monkeypatch.setattr(OM, "slots_of", lambda bt, b, pos, bs: realm(bt, 0, pos, bs))
    assert not _mla_ok(g)


def test_planted_off_by_one_request_lookup_fails(monkeypatch):
    g = _g()
    monkeypatch.setattr(OM, "request_of_token",
                        lambda cu_q, t: int(np.searchsorted(np.asarray(cu_q), t, side="left") - 1)
                        if t > 0 else 0)
    assert not _mla_ok(g)
    monkeypatch.undo()
    monkeypatch.setattr(OM, "request_of_token",
                        lambda cu_q, t: min(len(cu_q) - 2,
                                            int(np.searchsorted(np.asarray(cu_q), t, side="right"))))
    assert not _mla_ok(g)


def test_planted_prefill_positions_for_decode_queries_fail(monkeypatch):
    """Queries placed at 0 .. q_len - 1 (as in a prefill from an empty
    cache) instead of at the end of their request's context."""
    g = _g()
    monkeypatch.setattr(OI, "positions_of_request", lambda seq_len, q_len: list(range(q_len)))
    assert not _topk_ok(g)
