"""GPU tests of the split merge of sparse MLA.

When a token's keys are split over several workgroups, each split stores
bf16 partial rows and log-sum-exps, then counts its arrival at the token's
word in the workspace (tagged with the call).  The heads are merged in
parts, two halves with two splits and four parts of 16 heads with more,
each by its owner once every split has arrived, or by the last split when
the owner gave its part up (always when the grid is larger than the device
holds at once, or when the owner stopped waiting).  Every part is merged
once, in split order, so the result must match the oracle and repeat bit
for bit for every split count, grid size and wait bound, and graph replays,
which reuse the tag they were captured with, must find the word their
previous run left (every split counted) as no arrival."""
import numpy as np
import pytest
import torch

from _util import attn_close, ensure_library, np_f64
from oracle import mla as OM
from synth import get_config, make_batch, make_layer, make_random_indices

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _cfg(**kw):
    return get_config("decode_32k_mtp").scaled(name="merge", cid=66, **kw)


def _oracle(b, lay, idx_np, R, scale, tokens=None):
    kv = lay.kv_cache

    def kv_values(slots):
        s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=kv.device)
        return np_f64(kv[s])

    return OM.sparse_mla(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                         np_f64(lay.q_mla), kv_values, idx_np, R, scale, tokens=tokens)


def _setup(dsa, n_tokens, topk, seed):
    """n_tokens single-token requests over contexts of 1,500 to 5,000 keys."""
    g = np.random.default_rng(seed)
    lens = [int(x) for x in g.integers(1500, 5000, size=n_tokens)]
    cfg = _cfg(num_reqs=n_tokens, q_len=1, topk=topk)
    b = make_batch(cfg, DEV, seq_lens=lens, q_lens=[1] * n_tokens)
    lay = make_layer(cfg, b, DEV, with_indexer=False)
    idx = make_random_indices(b, topk, seed + 1, DEV)
    bb = dsa.Batch.from_synth(b)
    nbytes = dsa.sparse_mla_attn_workspace_size(bb, 64, cfg.kv_lora_rank,
                                                lay.q_mla.shape[2] - cfg.kv_lora_rank, topk, 1)
    return cfg, b, lay, idx, bb, nbytes


def _splits(nbytes, n_tokens):
    """Key splits per token, from the workspace size: bf16 partial rows
    (64 heads x 512 dims per split and token) beside much smaller log-sum-
    exps and arrival words."""
    return nbytes // (n_tokens * 64 * 512 * 2)


def _run(dsa, cfg, bb, lay, idx, ws, out=None, lse=None):
    return dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                               cfg.softmax_scale, out=out, lse=lse, workspace=ws)


# (query tokens, top-k): key splits per token 2, 3, 4, 5, 8, 16 (split count
# ceil(256 / tokens), at most top-k / 128); grids of 256 workgroups, and of
# 258 and 260 (three and five splits) just past one workgroup per CU
SPLITS = {2: (128, 256), 3: (86, 384), 4: (64, 512), 5: (52, 640), 8: (32, 1024),
          16: (16, 2048)}


@pytest.mark.parametrize("n_split", sorted(SPLITS))
def test_merge_for_each_split_count(dsa, n_split):
    n_tokens, topk = SPLITS[n_split]
    cfg, b, lay, idx, bb, nbytes = _setup(dsa, n_tokens, topk, 900 + n_split)
    assert _splits(nbytes, n_tokens) == n_split
    print("merge case: %d tokens, top-k %d, %d splits" % (n_tokens, topk, n_split), flush=True)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    o0, l0 = _run(dsa, cfg, bb, lay, idx, ws)
    o0, l0 = o0.clone(), l0.clone()
    for rep in range(3):
        o, l = _run(dsa, cfg, bb, lay, idx, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0), rep
    tokens = sorted(set(np.linspace(0, n_tokens - 1, 12).astype(int).tolist()))
    ro, rl = _oracle(b, lay, idx.cpu().numpy(), cfg.kv_lora_rank, cfg.softmax_scale, tokens)
    assert attn_close(np_f64(o0)[tokens], ro[tokens]) <= 0
    assert attn_close(l0.cpu().numpy()[tokens], rl[tokens], 1e-3, 1e-4) <= 0


@pytest.mark.parametrize("n_tokens,topk", [(160, 512), (300, 4096)])
def test_merge_with_more_workgroups_than_the_device_holds(dsa, n_tokens, topk):
    """Grids past one workgroup per CU (320 splits of 256 indices; 600
    splits of 2,048 on the one-workgroup-per-token kernel), so some splits
    start only after others have finished and nobody waits."""
    cfg, b, lay, idx, bb, nbytes = _setup(dsa, n_tokens, topk, 950 + n_tokens)
    assert _splits(nbytes, n_tokens) == 2
    print("merge case: %d tokens, top-k %d" % (n_tokens, topk), flush=True)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    o0, l0 = _run(dsa, cfg, bb, lay, idx, ws)
    o0, l0 = o0.clone(), l0.clone()
    o1, l1 = _run(dsa, cfg, bb, lay, idx, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    tokens = sorted(set(np.linspace(0, n_tokens - 1, 10).astype(int).tolist()))
    ro, rl = _oracle(b, lay, idx.cpu().numpy(), cfg.kv_lora_rank, cfg.softmax_scale, tokens)
    assert attn_close(np_f64(o0)[tokens], ro[tokens]) <= 0
    assert attn_close(l0.cpu().numpy()[tokens], rl[tokens], 1e-3, 1e-4) <= 0


@pytest.mark.parametrize("n_tokens,topk", [(16, 2048), (64, 2048), (128, 4096)])
def test_graph_replays_match_eager(dsa, n_tokens, topk):
    """A captured call replays with the tag it was captured with, so each
    replay must find the token words as its previous run left them (every
    split counted) and count from zero.  Eager calls on the same
    workspace (other tags) run between the replays; every replay equals the
    eager result bit for bit."""
    cfg, b, lay, idx, bb, nbytes = _setup(dsa, n_tokens, topk, 970 + n_tokens)
    print("graph merge case: %d tokens, top-k %d, %d splits" %
          (n_tokens, topk, _splits(nbytes, n_tokens)), flush=True)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.empty((n_tokens, 64, cfg.kv_lora_rank), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n_tokens, 64), dtype=torch.float32, device=DEV)
    o0, l0 = _run(dsa, cfg, bb, lay, idx, ws)
    o0, l0 = o0.clone(), l0.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(dsa, cfg, bb, lay, idx, ws, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(0)
        lse.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o0) and torch.equal(lse, l0), rep
        o, l = _run(dsa, cfg, bb, lay, idx, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0), rep
    del graph


@pytest.mark.parametrize("n_tokens,topk", [(128, 256), (64, 512), (16, 2048), (128, 4096)])
def test_merge_does_not_depend_on_the_wait(dsa, n_tokens, topk, monkeypatch):
    """DSA_MERGE_WAIT_TICKS bounds how long a split waits for its token's
    other splits before it stores its own rows and leaves its part to the
    last split.  With no wait (the last split merges every part), a wait
    of one or five ticks (owners give their parts up about when the last
    split arrives, so both outcomes of that race occur) and the default,
    the bits are the same, and they match the oracle.  Shapes: two splits
    on each kernel, four and sixteen splits."""
    cfg, b, lay, idx, bb, nbytes = _setup(dsa, n_tokens, topk, 990 + n_tokens + topk)
    print("merge wait case: %d tokens, top-k %d, %d splits" %
          (n_tokens, topk, _splits(nbytes, n_tokens)), flush=True)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    got = []
    for wait in (None, "0", "1", "5", "1", None):
        if wait is None:
            monkeypatch.delenv("DSA_MERGE_WAIT_TICKS", raising=False)
        else:
            monkeypatch.setenv("DSA_MERGE_WAIT_TICKS", wait)
        o, l = _run(dsa, cfg, bb, lay, idx, ws)
        torch.cuda.synchronize()
        got.append((wait, o.clone(), l.clone()))
    o0, l0 = got[0][1], got[0][2]
    for wait, o, l in got[1:]:
        assert torch.equal(o, o0) and torch.equal(l, l0), wait
    tokens = sorted(set(np.linspace(0, n_tokens - 1, 8).astype(int).tolist()))
    ro, rl = _oracle(b, lay, idx.cpu().numpy(), cfg.kv_lora_rank, cfg.softmax_scale, tokens)
    assert attn_close(np_f64(o0)[tokens], ro[tokens]) <= 0
    assert attn_close(l0.cpu().numpy()[tokens], rl[tokens], 1e-3, 1e-4) <= 0
