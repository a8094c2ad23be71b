"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle computes sampled query tokens one by one; every
row is checked for the invariants that hold at any size."""
import numpy as np
import pytest
import torch

from _util import attn_close, check_row_invariants, ensure_library, np_bits, np_f64, recall
from oracle import indexer as OI, indexshare as OX, mla as OM
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _positions(b):
    pos = []
    for bi in range(b.num_reqs):
        for i in range(b.q_lens[bi]):
            pos.append(b.seq_lens[bi] - b.q_lens[bi] + i)
    return pos


def _all_rows_valid(idx, b, topk):
    got = idx.cpu().numpy()
    for t, p in enumerate(_positions(b)):
        check_row_invariants(got[t], p, topk)
    return got


def _mla_oracle(b, lay, idx_np, cfg, tokens):
    kv = lay.kv_cache

    def kv_values(slots):
        s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=kv.device)
        return np_f64(kv[s])

    return OM.sparse_mla(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                         np_f64(lay.q_mla), kv_values, idx_np, cfg.kv_lora_rank,
                         cfg.softmax_scale, tokens=tokens)


def _check_sampled(b, lay, cfg, got_idx, out, lse, cache_np, scale_np, cdt, tokens):
    ref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                          np_f64(lay.q_idx), np_f64(lay.w), cache_np, scale_np, cdt,
                          cfg.topk, tokens=tokens)
    r, worst = recall(got_idx[tokens], ref[tokens])
    print("sampled recall %.6f (worst row %.6f)" % (r, worst), flush=True)
    assert r >= 0.999, (r, worst)
    ro, rl = _mla_oracle(b, lay, ref, cfg, tokens)
    go, gl = np_f64(out), lse.cpu().numpy()
    for t in tokens:
        assert attn_close(go[t], ro[t]) <= 0, t
        assert attn_close(gl[t], rl[t], 2e-2, 1e-3) <= 0, t


def test_decode_32k_mtp_full(dsa):
    cfg = get_config("decode_32k_mtp")
    b = make_batch(cfg, DEV)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    cache = lay.k_src.clone()
    cache[b.slot_mapping_t] = 0                     # this step's keys not yet written
    k_new = lay.k_src[b.slot_mapping_t].contiguous()
    dsa.dsa_indexer_cache_write(k_new, b.slot_mapping_t, cache)
    idx = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, cache, None, cfg.topk)
    out, lse = dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                                   cfg.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(cache, lay.k_src)
    got = _all_rows_valid(idx, b, cfg.topk)
    idx2 = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, cache, None, cfg.topk)
    assert torch.equal(idx, idx2)                   # run-to-run determinism
    # attention repeats bit for bit at the timed shape (a race moves outputs
    # by about one bf16 unit, inside the oracle tolerance)
    for _ in range(3):
        out2, lse2 = dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                                         cfg.softmax_scale)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _check_sampled(b, lay, cfg, got, out, lse, np_bits(cache), None, OI.BF16,
                   [0, 1, 2, 63, 64, 126, 127])


def test_prefill_16k_full(dsa):
    cfg = get_config("prefill_16k")
    b = make_batch(cfg, DEV)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    idx = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, lay.k_src, None, cfg.topk)
    out, lse = dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                                   cfg.softmax_scale)
    torch.cuda.synchronize()
    got = _all_rows_valid(idx, b, cfg.topk)
    # rows with t < topk take every position 0..t
    for t in (0, 1, 777, 2047):
        assert np.array_equal(got[t][:t + 1], np.arange(t + 1))
    _check_sampled(b, lay, cfg, got, out, lse, np_bits(lay.k_src), None, OI.BF16,
                   [0, 5, 2047, 2048, 2049, 9000, 16383])


def test_fp8_decode_varlen_full(dsa):
    cfg = get_config("fp8_decode_varlen")
    b = make_batch(cfg, DEV)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    cache = torch.empty((b.num_slots, cfg.d_idx), dtype=torch.uint8, device=DEV)
    scale = torch.empty((b.num_slots,), dtype=torch.float32, device=DEV)
    all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=DEV)
    dsa.dsa_indexer_cache_write(lay.k_src, all_slots, cache, scale)
    idx = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, cache, scale, cfg.topk)
    out, lse = dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                                   cfg.softmax_scale)
    torch.cuda.synchronize()
    got = _all_rows_valid(idx, b, cfg.topk)
    lens = np.array(b.seq_lens)
    reqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 0, 77})
    # oracle cache: quantise exactly the rows these requests use
    codes = np.zeros((b.num_slots, cfg.d_idx), dtype=np.uint8)
    scales = np.ones(b.num_slots, dtype=np.float32)
    for r in reqs:
        slots = OI.physical_slots(b.block_table_host[r], b.block_size, b.seq_lens[r])
        k32 = np_f64(lay.k_src[torch.as_tensor(slots, device=DEV)]).astype(np.float32)
        c, s = OI.fp8_quantize_rows(k32)
        codes[slots], scales[slots] = c, s
        gs = torch.as_tensor(slots, device=DEV)
        assert np.array_equal(np_bits(cache[gs]), c), r
        assert np.array_equal(scale[gs].cpu().numpy().view(np.uint32), s.view(np.uint32)), r
    _check_sampled(b, lay, cfg, got, out, lse, codes, scales, OI.FP8, reqs)


def test_indexshare_8layer_full(dsa):
    cfg = get_config("indexshare_8layer")
    types = cfg.indexer_types
    b = make_batch(cfg, DEV)
    bb = dsa.Batch.from_synth(b)
    src = OX.resolve_sources(types, 8)
    N = b.num_q_tokens
    lays, L = [], []
    for i in range(8):
        full = src[i] == i
        lay = make_layer(cfg, b, DEV, layer=i, with_indexer=True)
        lays.append(lay)
        L.append(dsa.Layer(
            q_mla=lay.q_mla, kv_cache=lay.kv_cache,
            out=torch.empty((N, 64, 512), dtype=torch.bfloat16, device=DEV),
            lse=torch.empty((N, 64), dtype=torch.float32, device=DEV),
            # shared layers get their own (never read) indexer tensors
            q_idx=lay.q_idx, w=lay.w, k_cache=lay.k_src,
            topk_idx=torch.empty((N, cfg.topk), dtype=torch.int32, device=DEV) if full else None))
    dims = dsa.StackDims(32, 128, dsa.DSA_BF16, dsa.DSA_BF16, cfg.topk, 64, 512, 64,
                         dsa.DSA_BF16, cfg.softmax_scale)
    codes = [dsa.DSA_LAYER_FULL if t == "full" else dsa.DSA_LAYER_SHARED for t in types]
    active = dsa.indexshare_forward(bb, codes, L, dims)
    torch.cuda.synchronize()
    for i in range(8):
        assert active[i] == L[src[i]].topk_idx.data_ptr()
    # perturb the shared layers' own indexer inputs: nothing may change
    before = [l.out.clone() for l in L]
    for i in range(8):
        if src[i] != i:
            lays[i].q_idx.mul_(-3.0)
            lays[i].w.add_(5.0)
            lays[i].k_src.zero_()
    dsa.indexshare_forward(bb, codes, L, dims)
    torch.cuda.synchronize()
    for i in range(8):
        assert torch.equal(before[i], L[i].out), i
    tokens = [0, 31, 63]
    for i in (0, 1, 4, 7):
        s = src[i]
        got = _all_rows_valid(L[s].topk_idx, b, cfg.topk)
        ref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, 64,
                              np_f64(lays[s].q_idx), np_f64(lays[s].w), np_bits(lays[s].k_src),
                              None, OI.BF16, cfg.topk, tokens=tokens)
        r, _ = recall(got[tokens], ref[tokens])
        assert r >= 0.999
        ro, _ = _mla_oracle(b, lays[i], ref, cfg, tokens)
        go = np_f64(L[i].out)
        for t in tokens:
            assert attn_close(go[t], ro[t]) <= 0, (i, t)
