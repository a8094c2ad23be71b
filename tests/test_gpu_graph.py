"""A decode step (cache write, indexer and top-k, sparse MLA) captured in a
HIP graph and replayed: the library allocates nothing and enqueues no
memset inside its calls, so the capture holds only its kernels.  Each
replay, with eager calls of the same step on the same buffers between the
replays, must give the eager step's bits."""
import pytest
import torch

from _util import ensure_library
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


@pytest.mark.parametrize("shape", ["two_splits", "many_splits"])
def test_decode_step_graph_replays_match_eager(dsa, shape):
    if shape == "two_splits":       # 128 tokens: two key splits each
        cfg = get_config("decode_32k_mtp").scaled(name="graph", cid=67, num_reqs=64, topk=2048)
        b = make_batch(cfg, DEV, seq_lens=[3000 + 37 * i for i in range(64)], q_lens=[2] * 64)
    else:                           # 6 tokens: sixteen key splits each
        cfg = get_config("decode_32k_mtp").scaled(name="graph", cid=68, num_reqs=3, topk=2048)
        b = make_batch(cfg, DEV, seq_lens=[5000, 2500, 4100], q_lens=[2, 2, 2])
    print("graph step case: %s, %d tokens" % (shape, b.num_q_tokens), flush=True)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    N = b.num_q_tokens
    k_cache = lay.k_src.clone()
    k_new = lay.k_src[b.slot_mapping_t].contiguous()
    idx = torch.empty((N, cfg.topk), dtype=torch.int32, device=DEV)
    out = torch.empty((N, cfg.n_heads, cfg.kv_lora_rank), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((N, cfg.n_heads), dtype=torch.float32, device=DEV)
    nbytes = max(dsa.dsa_indexer_topk_workspace_size(bb, cfg.topk),
                 dsa.sparse_mla_attn_workspace_size(bb, cfg.n_heads, cfg.kv_lora_rank,
                                                    cfg.rope_dim, cfg.topk, dsa.DSA_BF16))
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=DEV)

    def step():
        dsa.dsa_indexer_cache_write(k_new, b.slot_mapping_t, k_cache)
        dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, k_cache, None, cfg.topk, topk_idx=idx,
                             workspace=ws)
        dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                            cfg.softmax_scale, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        idx.fill_(-7)
        out.fill_(0)
        lse.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(out, ref[1]) and torch.equal(lse, ref[2]), rep
        step()                                      # eager, same buffers and workspace
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(out, ref[1]) and torch.equal(lse, ref[2]), rep
    del graph
