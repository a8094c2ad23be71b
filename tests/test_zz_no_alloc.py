"""The allocation-free indexer entry point (dsa_indexer_topk_noalloc, scratch
in a static per-device array) against dsa_indexer_topk with a workspace,
through the C ABI: two calls in a row, the second on a smaller batch (the
array still holds the first call's scores), bit-identical index rows."""
import pytest
import torch

from _util import ensure_library
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _case(dsa, seq_lens, q_lens, topk, cid, fp8=False):
    cfg = get_config("decode_32k_mtp").scaled(
        name="noalloc", cid=cid, num_reqs=len(seq_lens), topk=topk,
        idx_cache_dtype="fp8" if fp8 else "bf16")
    b = make_batch(cfg, DEV, seq_lens=seq_lens, q_lens=q_lens)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    if fp8:
        cache = torch.zeros((b.num_slots, 128), dtype=torch.uint8, device=DEV)
        scale = torch.zeros((b.num_slots,), dtype=torch.float32, device=DEV)
        all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=DEV)
        dsa.dsa_indexer_cache_write(lay.k_src, all_slots, cache, scale)
    else:
        cache, scale = lay.k_src, None
    return b, bb, lay, cache, scale


def _both(dsa, bb, lay, cache, scale, topk, N):
    ref = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, cache, scale, topk)
    got = torch.full((N, topk), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_indexer_topk_noalloc(bb, lay.q_idx, lay.w, cache, scale, topk, got)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_the_workspace_call_twice(dsa):
    # first call: rows past the register path's reach (chunk ranges in the
    # scratch), several query tokens per request
    b, bb, lay, cache, scale = _case(dsa, [40000, 3000, 33000, 700, 5003, 2049],
                                     [1, 2, 1, 2, 2, 1], 2048, 81)
    got, ref = _both(dsa, bb, lay, cache, scale, 2048, b.num_q_tokens)
    assert torch.equal(got, ref)
    # second call right after, smaller and of another cache dtype: the scratch
    # still holds the first call's rows
    b2, bb2, lay2, cache2, scale2 = _case(dsa, [1000, 2500], [1, 2], 256, 82, fp8=True)
    got2, ref2 = _both(dsa, bb2, lay2, cache2, scale2, 256, b2.num_q_tokens)
    assert torch.equal(got2, ref2)


def test_noalloc_rejects_a_batch_beyond_its_scratch(dsa):
    cfg = get_config("decode_32k_mtp").scaled(name="noalloc", cid=83, num_reqs=2)
    b = make_batch(cfg, DEV, seq_lens=[70000, 70000], q_lens=[64, 64])
    lay = make_layer(cfg, b, DEV, with_indexer=True)
    bb = dsa.Batch.from_synth(b)
    assert dsa.dsa_indexer_topk_workspace_size(bb, 2048) > 32 << 20
    out = torch.full((b.num_q_tokens, 2048), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_indexer_topk_noalloc(bb, lay.q_idx, lay.w, lay.k_src, None, 2048, out)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.all(out == -7)          # nothing was enqueued
