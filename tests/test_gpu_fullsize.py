"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle recomputes every query token of the decode
workloads (the FP8 cache's codes and scales for every key), and 72 query
tokens spread over the 16384-token prefill; every row is also checked for the
invariants that hold at any size."""
import numpy as np
import pytest
import torch

from _util import (attn_close, bf16_bits_to_f32, check_row_invariants, ensure_library,
                   np_bits, np_f64, pool_map, recall)
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


def _oracle_topk(b, q64, w64, cache_np, scale_np, cdt, topk, tokens):
    """The oracle's rows for the given tokens, one request per pool task."""
    req_of = np.searchsorted(b.cu_q_host, np.asarray(tokens), side="right") - 1
    groups = {}
    for t, r in zip(tokens, req_of):
        groups.setdefault(int(r), []).append(int(t))

    def one(ts):
        return ts, OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host,
                                   b.block_size, q64, w64, cache_np, scale_np, cdt,
                                   topk, tokens=ts)

    ref = np.full((b.num_q_tokens, topk), -1, dtype=np.int32)
    for ts, rows in pool_map(one, groups.values()):
        ref[ts] = rows[ts]
    return ref


def _mla_oracle(b, lay, idx_np, cfg, tokens):
    kv = lay.kv_cache

    def kv_values(slots):
        s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=kv.device)
        return np_f64(kv[s])

    return OM.sparse_mla(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                         np_f64(lay.q_mla), kv_values, idx_np, cfg.kv_lora_rank,
                         cfg.softmax_scale, tokens=tokens)


def _check(b, lay, cfg, got_idx, out, lse, cache_np, scale_np, cdt, tokens):
    ref = _oracle_topk(b, np_f64(lay.q_idx), np_f64(lay.w), cache_np, scale_np, cdt,
                       cfg.topk, tokens)
    r, worst = recall(got_idx[tokens], ref[tokens])
    print("recall over %d rows %.6f (worst row %.6f)" % (len(tokens), r, worst), flush=True)
    assert r >= 0.999, (r, worst)
    ro, rl = _mla_oracle(b, lay, ref, cfg, tokens)
    go, gl = np_f64(out), lse.cpu().numpy()
    for t in tokens:
        assert attn_close(go[t], ro[t]) <= 0, t
        assert attn_close(gl[t], rl[t], 2e-2, 1e-3) <= 0, t
    return ref


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
    _check(b, lay, cfg, got, out, lse, np_bits(cache), None, OI.BF16,
           list(range(b.num_q_tokens)))


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
    for t in range(cfg.topk):
        assert np.array_equal(got[t][:t + 1], np.arange(t + 1)), t
    # 64 rows spread evenly over the sequence, plus the edges of the
    # top-k width
    tokens = sorted(set(np.linspace(0, 16383, 64).astype(int).tolist())
                    | {0, 5, 2046, 2047, 2048, 2049, 4095, 16383})
    _check(b, lay, cfg, got, out, lse, np_bits(lay.k_src), None, OI.BF16, tokens)


def _oracle_fp8_cache(k_src, chunk=32768):
    """The oracle's e4m3 codes and scales of every key (bf16 keys, quantised
    on the host in chunks, one per pool task)."""
    bits = np_bits(k_src)
    n = bits.shape[0]
    codes = np.empty(bits.shape, dtype=np.uint8)
    scales = np.empty(n, dtype=np.float32)

    def one(s):
        e = min(n, s + chunk)
        codes[s:e], scales[s:e] = OI.fp8_quantize_rows(bf16_bits_to_f32(bits[s:e]))

    pool_map(one, range(0, n, chunk))
    return codes, scales


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
    # every key's codes and scale, bit for bit
    codes, scales = _oracle_fp8_cache(lay.k_src)
    print("fp8 cache: %d keys compared" % codes.shape[0], flush=True)
    assert np.array_equal(np_bits(cache), codes)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), scales.view(np.uint32))
    _check(b, lay, cfg, got, out, lse, codes, scales, OI.FP8, list(range(b.num_q_tokens)))


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
    tokens = list(range(N))
    refs = {}
    for s in sorted(set(src)):
        got = _all_rows_valid(L[s].topk_idx, b, cfg.topk)
        refs[s] = _oracle_topk(b, np_f64(lays[s].q_idx), np_f64(lays[s].w),
                               np_bits(lays[s].k_src), None, OI.BF16, cfg.topk, tokens)
        r, worst = recall(got, refs[s])
        print("layer %d recall %.6f (worst row %.6f)" % (s, r, worst), flush=True)
        assert r >= 0.999, (s, r, worst)
    for i in range(8):
        ro, rl = _mla_oracle(b, lays[i], refs[src[i]], cfg, tokens)
        go, gl = np_f64(L[i].out), L[i].lse.cpu().numpy()
        for t in tokens:
            assert attn_close(go[t], ro[t]) <= 0, (i, t)
            assert attn_close(gl[t], rl[t], 2e-2, 1e-3) <= 0, (i, t)
