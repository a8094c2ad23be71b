"""Pins for the oracle's IndexShare resolution and stack (CPU only)."""
import pytest

from oracle import indexshare as ix

F, S = ix.FULL, ix.SHARED


def test_source_map_of_the_eight_layer_pattern():
    # hand-derived: each shared layer takes the nearest preceding full layer
    assert ix.resolve_sources([F, S, S, S, F, S, S, S], 8) == [0, 0, 0, 0, 4, 4, 4, 4]


@pytest.mark.parametrize("types,n,want", [
    ([F], 1, [0]),
    ([F, F, F], 3, [0, 1, 2]),
    ([F, S, F, S, S], 5, [0, 0, 2, 2, 2]),
    ([F, S, S, F, S, S, S, S], 4, [0, 0, 0, 3]),      # longer list is allowed
])
def test_source_maps(types, n, want):
    assert ix.resolve_sources(types, n) == want


@pytest.mark.parametrize("types,n", [
    ([S, F], 2),              # shared with no preceding full
    ([F, S], 3),              # too short
    ([F, "dense"], 2),        # unknown type
    ([F, S, "Full"], 2),      # unknown type outside the used prefix
    ([], 1),
])
def test_rejections(types, n):
    with pytest.raises(ValueError):
        ix.resolve_sources(types, n)


def test_forward_chain_full_shared_shared():
    calls = []

    def run_indexer(layer):
        calls.append(layer)
        return ("topk", layer)

    res, actives, n = ix.forward([F, S, S, F, S], list(range(5)), run_indexer,
                                 lambda layer, tk: (layer, tk))
    assert n == 2 and calls == [0, 3]
    assert actives == [("topk", 0)] * 3 + [("topk", 3)] * 2
    assert res[2] == (2, ("topk", 0))
