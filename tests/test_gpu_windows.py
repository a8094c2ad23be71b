"""GPU tests of the indexer with a workspace smaller than the whole batch's.

dsa_indexer_topk scores and selects the query tokens in windows of as many
tokens as the workspace holds (whole blocks of 16 when it can).  Windows
start at global token offsets, so they cut the score kernels' token blocks
(two tokens per request at decode, sixteen per request in prefill-shaped
batches) wherever a request's tokens do not start on a multiple of 16.  The
rows must come out bit for bit as with the full workspace, which the other
tests hold to the oracle, on every score path: decode-shaped blocks with
rows past the register reach (per-chunk score ranges), prefill-shaped
blocks, the even split of single-token e4m3 requests, and the vector path."""
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
    return get_config("decode_32k_mtp").scaled(name="windows", cid=65, **kw)


def _both(dsa, b, q, w, cache, scale, topk, extra=0):
    """Rows with the full workspace and with the least accepted one (plus
    `extra` bytes), and the window count the latter implies."""
    bb = dsa.Batch.from_synth(b)
    full = dsa.dsa_indexer_topk_workspace_size(bb, topk)
    least = dsa.dsa_indexer_topk_workspace_min(bb, topk)
    assert 0 < least <= full
    ws_full = torch.empty(full, dtype=torch.uint8, device=DEV)
    ws_small = torch.empty(least + extra, dtype=torch.uint8, device=DEV)
    print("windows case: %d tokens, workspace %d of %d bytes" % (b.num_q_tokens, least + extra,
                                                                 full), flush=True)
    ref = dsa.dsa_indexer_topk(bb, q, w, cache, scale, topk, workspace=ws_full)
    got = dsa.dsa_indexer_topk(bb, q, w, cache, scale, topk, workspace=ws_small)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_windows_decode_blocks_with_long_rows(dsa):
    """Requests of 1 to 3 query tokens (blocks of two cut by the windows),
    rows past 32768 keys (the score pass records chunk ranges, the top-k
    streams its rows) and short ones."""
    q_lens = [3, 1, 2, 2, 3, 1, 2, 3, 2, 1, 3, 2, 2, 1, 3, 2, 3, 1]
    lens = [40000 - 1500 * i for i in range(len(q_lens))]
    cfg = _cfg(num_reqs=len(q_lens), topk=512)
    b = make_batch(cfg, DEV, seq_lens=lens, q_lens=q_lens)
    assert b.num_q_tokens > 32
    lay = make_layer(cfg, b, DEV)
    ref, got = _both(dsa, b, lay.q_idx, lay.w, lay.k_src, None, 512)
    assert np.array_equal(got, ref)


def test_windows_prefill_blocks(dsa):
    """Prefill-shaped blocks of 16 tokens per request, ragged token counts,
    so the 16-token windows cut most blocks; a second run with a workspace
    between two window sizes."""
    cfg = _cfg(num_reqs=5, topk=256)
    b = make_batch(cfg, DEV, seq_lens=[300, 5000, 2100, 64, 3001], q_lens=[40, 77, 16, 64, 1])
    lay = make_layer(cfg, b, DEV)
    ref, got = _both(dsa, b, lay.q_idx, lay.w, lay.k_src, None, 256)
    assert np.array_equal(got, ref)
    bb = dsa.Batch.from_synth(b)
    per16 = dsa.dsa_indexer_topk_workspace_min(bb, 256)
    ref2, got2 = _both(dsa, b, lay.q_idx, lay.w, lay.k_src, None, 256, extra=per16 + 1000)
    assert np.array_equal(got2, ref)


def test_windows_fp8_even_split(dsa):
    """Single-token requests over long e4m3 caches (the even split of the
    batch's key tiles, which counts only the window's requests), with a
    request without a query token; the windowed rows also against the
    oracle."""
    g = np.random.default_rng(11)
    lens = [int(x) for x in g.integers(100, 40000, size=48)]
    lens[2], lens[30] = 32769, 39999
    q_lens = [1] * 48
    q_lens[7] = 0
    cfg = _cfg(num_reqs=48, q_len=1, idx_cache_dtype="fp8", topk=2048)
    b = make_batch(cfg, DEV, seq_lens=lens, q_lens=q_lens)
    lay = make_layer(cfg, b, DEV)
    cache = torch.zeros((b.num_slots, 128), dtype=torch.uint8, device=DEV)
    scale = torch.zeros((b.num_slots,), dtype=torch.float32, device=DEV)
    all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=DEV)
    dsa.dsa_indexer_cache_write(lay.k_src, all_slots, cache, scale)
    ref, got = _both(dsa, b, lay.q_idx, lay.w, cache, scale, 2048)
    assert np.array_equal(got, ref)
    codes, scales = OI.fp8_quantize_rows(np_f64(lay.k_src).astype(np.float32))
    oref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                           np_f64(lay.q_idx), np_f64(lay.w), codes, scales, OI.FP8, 2048)
    t = 0
    for bi in range(b.num_reqs):
        for _ in range(b.q_lens[bi]):
            check_row_invariants(got[t], b.seq_lens[bi] - 1, 2048)
            t += 1
    r, worst = recall(got, oref)
    assert r >= 0.999, (r, worst)


def test_windows_vector_path(dsa):
    """The fp32 vector score path (tiny prefill, 256 causal tokens): exact
    integer scores, so the windowed rows equal the oracle's bit for bit."""
    cfg = get_config("tiny_prefill")
    b = make_batch(cfg, DEV)
    lay = make_layer(cfg, b, DEV)
    ref, got = _both(dsa, b, lay.q_idx, lay.w, lay.k_src, None, cfg.topk)
    assert np.array_equal(got, ref)
    oref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                           np_f64(lay.q_idx), np_f64(lay.w), np_bits(lay.k_src), None,
                           OI.F32, cfg.topk)
    assert np.array_equal(got, oref)
