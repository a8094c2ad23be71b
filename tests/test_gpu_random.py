"""Seeded random batches through both calls against the oracle.

Each case draws a ragged batch (1 to 8 requests, contexts of 1 to 6000
positions, 0 to 20 query tokens per request, at least one token), a block
size, an indexer head count, a top-k width and, for odd seeds, a workspace
between the least the indexer accepts and the whole batch's (the call then
works window by window), then runs dsa_indexer_topk and sparse_mla_attn on
it.  The indexer inputs are small integers (q and k
uniform in -3..3, stored as bf16, w in {1, 2}), so every score is exact on
the matrix-core path too and every index row must equal the oracle's bit
for bit (ties fall to the lower position on both sides); the attention runs
on the indexer's own rows and is compared elementwise with the oracle."""
import numpy as np
import pytest
import torch

from _util import attn_close, check_row_invariants, ensure_library, np_bits, np_f64
from oracle import indexer as OI, mla as OM
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _case(seed):
    g = np.random.default_rng(1000 + seed)
    R = int(g.integers(1, 9))
    lens = [int(x) for x in g.integers(1, 6001, size=R)]
    qls = [int(g.integers(0, min(L, 20) + 1)) for L in lens]
    if sum(qls) == 0:
        qls[0] = 1
    topk = int(g.choice([1, 5, 64, 300, 2048]))
    bs = int(g.choice([32, 64, 128]))
    heads = int(g.choice([32, 64]))
    extra = float(g.uniform(0.0, 1.0))
    return lens, qls, topk, bs, heads, extra


@pytest.mark.parametrize("seed", range(24))
def test_random_batch_both_calls(dsa, seed):
    lens, qls, topk, bs, heads, extra = _case(seed)
    cfg = get_config("decode_32k_mtp").scaled(
        name="random", cid=70 + seed, num_reqs=len(lens), topk=topk, block_size=bs,
        n_idx_heads=heads, idx_values="int3", w_values="one_two")
    b = make_batch(cfg, DEV, seq_lens=lens, q_lens=qls)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    ws_bytes = dsa.dsa_indexer_topk_workspace_size(bb, topk)
    if seed % 2:
        least = dsa.dsa_indexer_topk_workspace_min(bb, topk)
        ws_bytes = least + int(extra * (ws_bytes - least))
    print("random case %d: seq_lens %s q_lens %s topk %d block %d heads %d workspace %d"
          % (seed, lens, qls, topk, bs, heads, ws_bytes), flush=True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    idx = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, lay.k_src, None, topk, workspace=ws)
    out, lse = dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                                   cfg.softmax_scale)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, bs, np_f64(lay.q_idx),
                          np_f64(lay.w), np_bits(lay.k_src), None, OI.BF16, topk)
    t = 0
    for bi in range(b.num_reqs):
        for i in range(b.q_lens[bi]):
            check_row_invariants(got[t], b.seq_lens[bi] - b.q_lens[bi] + i, topk)
            t += 1
    assert np.array_equal(got, ref)
    kv = lay.kv_cache

    def kv_values(slots):
        s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=kv.device)
        return np_f64(kv[s])

    ro, rl = OM.sparse_mla(b.seq_lens, b.cu_q_host, b.block_table_host, bs,
                           np_f64(lay.q_mla), kv_values, got, cfg.kv_lora_rank,
                           cfg.softmax_scale)
    assert attn_close(np_f64(out), ro) <= 0
    assert attn_close(lse.cpu().numpy(), rl, 1e-3, 1e-4) <= 0


@pytest.mark.parametrize("seed", range(8))
def test_random_batch_fp8_cache(dsa, seed):
    """The same random batches over an e4m3 indexer cache written by
    dsa_indexer_cache_write (normal keys): the cache's codes and scales equal
    the oracle's bit for bit, every row keeps the selection invariants, and
    the selected sets reach recall 0.999 against the oracle on the dequantised
    keys (scores are no longer exact, so near-ties may resolve differently)."""
    from _util import recall
    lens, qls, topk, bs, heads, _ = _case(100 + seed)
    cfg = get_config("decode_32k_mtp").scaled(
        name="random_fp8", cid=90 + seed, num_reqs=len(lens), topk=topk, block_size=bs,
        n_idx_heads=heads, idx_cache_dtype="fp8")
    b = make_batch(cfg, DEV, seq_lens=lens, q_lens=qls)
    print("random fp8 case %d: seq_lens %s q_lens %s topk %d block %d heads %d"
          % (seed, lens, qls, topk, bs, heads), flush=True)
    lay = make_layer(cfg, b, DEV)
    cache = torch.zeros((b.num_slots, 128), dtype=torch.uint8, device=DEV)
    scale = torch.zeros((b.num_slots,), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_cache_write(lay.k_src, torch.arange(b.num_slots, dtype=torch.int64,
                                                        device=DEV), cache, scale)
    bb = dsa.Batch.from_synth(b)
    idx = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, cache, scale, topk)
    torch.cuda.synchronize()
    codes, scales = OI.fp8_quantize_rows(np_f64(lay.k_src).astype(np.float32))
    assert np.array_equal(np_bits(cache), codes)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), scales.view(np.uint32))
    got = idx.cpu().numpy()
    ref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, bs, np_f64(lay.q_idx),
                          np_f64(lay.w), codes, scales, OI.FP8, topk)
    t = 0
    for bi in range(b.num_reqs):
        for i in range(b.q_lens[bi]):
            check_row_invariants(got[t], b.seq_lens[bi] - b.q_lens[bi] + i, topk)
            t += 1
    r, worst = recall(got, ref)
    assert r >= 0.999, (r, worst)
