"""GPU parity of the prefill-shaped score pass through the C ABI.

Batches with at least 16 query tokens in some request, bf16 queries and
keys, 32 heads of 128 dims take the pass that reuses each key across 16
query tokens (one workgroup per 16-token block and key chunk).  The top-k
rows are compared with the oracle's: bit-exact where the scores are exact
(integer inputs) or the row is shorter than k, recall otherwise."""
import numpy as np
import pytest
import torch

from _util import check_row_invariants, ensure_library, np_bits, np_f64, recall
from oracle import indexer as OI
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _cfg(**kw):
    return get_config("decode_32k_mtp").scaled(name="prefill_small", cid=63, **kw)


def _run(dsa, cfg, b, lay, topk):
    print("prefill case: seq_lens %s q_lens %s topk %d" % (b.seq_lens, b.q_lens, topk),
          flush=True)
    idx = dsa.dsa_indexer_topk(dsa.Batch.from_synth(b), lay.q_idx, lay.w, lay.k_src, None, topk)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                          np_f64(lay.q_idx), np_f64(lay.w), np_bits(lay.k_src), None,
                          OI.BF16, topk)
    return got, ref


def _positions(b):
    return [b.seq_lens[bi] - b.q_lens[bi] + i for bi in range(b.num_reqs)
            for i in range(b.q_lens[bi])]


@pytest.mark.parametrize("topk", [64, 2048])
def test_prefill_blocks_ragged_batch(dsa, topk):
    """Chunked-prefill queries at the end of their contexts, token counts
    that leave partial 16-token blocks (40, 77), a request with a single
    query token, a full prefill from position 0, and contexts that end
    inside a key chunk and inside a 64-key group."""
    cfg = _cfg(num_reqs=5, topk=topk)
    b = make_batch(cfg, DEV, seq_lens=[300, 5000, 2100, 64, 3001],
                   q_lens=[40, 77, 16, 64, 1])
    lay = make_layer(cfg, b, DEV)
    got, ref = _run(dsa, cfg, b, lay, topk)
    for t, pos in enumerate(_positions(b)):
        check_row_invariants(got[t], pos, topk)
        if pos + 1 <= topk:
            assert np.array_equal(got[t], ref[t]), t
    r, worst = recall(got, ref)
    assert r >= 0.999, (r, worst)


@pytest.mark.parametrize("topk", [16, 300])
def test_prefill_integer_scores_bit_exact(dsa, topk):
    """Integer queries, keys and weights: every score is an exact integer on
    both sides, so the rows (ties broken by position) must match bit for
    bit, including ties across the 16 tokens of a block."""
    cfg = _cfg(num_reqs=2, topk=topk, idx_values="int3", w_values="one_two")
    b = make_batch(cfg, DEV, seq_lens=[1000, 333], q_lens=[1000, 50])
    lay = make_layer(cfg, b, DEV)
    got, ref = _run(dsa, cfg, b, lay, topk)
    assert np.array_equal(got, ref)


def test_prefill_rows_past_the_register_reach(dsa):
    """Rows of 40,000 keys: the pass also records per-chunk score ranges,
    which the top-k's long-row path reads instead of a range pass."""
    cfg = _cfg(num_reqs=1, topk=2048)
    b = make_batch(cfg, DEV, seq_lens=[40000], q_lens=[24])
    lay = make_layer(cfg, b, DEV)
    got, ref = _run(dsa, cfg, b, lay, 2048)
    for t, pos in enumerate(_positions(b)):
        check_row_invariants(got[t], pos, 2048)
    r, worst = recall(got, ref)
    assert r >= 0.999, (r, worst)


def test_prefill_and_decode_paths_agree(dsa):
    """The same tokens scored by the prefill-shaped pass (the batch has a
    16-token request) and by the decode-shaped pass (each token alone in a
    batch of single-token requests over the same cache) select the same
    rows up to score ties near the threshold."""
    cfg = _cfg(num_reqs=1, topk=512)
    b = make_batch(cfg, DEV, seq_lens=[4000], q_lens=[16])
    lay = make_layer(cfg, b, DEV)
    idx = dsa.dsa_indexer_topk(dsa.Batch.from_synth(b), lay.q_idx, lay.w, lay.k_src, None, 512)
    # the decode-shaped view: 16 requests of one query token each, with the
    # same block table and the contexts ending at each token's position
    pos = _positions(b)
    bt = torch.from_numpy(np.repeat(b.block_table_host, 16, axis=0)).to(DEV)
    single = dsa.Batch(seq_lens=torch.tensor([p + 1 for p in pos], dtype=torch.int32, device=DEV),
                       cu_q=torch.arange(17, dtype=torch.int32, device=DEV),
                       block_table=bt, num_q_tokens=16, max_q_len=1,
                       max_seq_len=max(pos) + 1, block_size=b.block_size,
                       num_slots=b.num_slots)
    idx1 = dsa.dsa_indexer_topk(single, lay.q_idx, lay.w, lay.k_src, None, 512)
    torch.cuda.synchronize()
    r, worst = recall(idx.cpu().numpy(), idx1.cpu().numpy())
    assert r >= 0.999, (r, worst)
