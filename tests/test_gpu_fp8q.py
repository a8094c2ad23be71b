"""GPU parity of the FP8-query indexer variant through the C ABI: the
activation rotation + quantisation (bit-exact codes and scales against the
oracle, which takes the quantisation decision on the same fp32 butterflies),
and the score + top-k over e4m3 queries and keys (recall against the oracle's
FP8-query path on the oracle's own codes, which equal the GPU's)."""
import numpy as np
import pytest
import torch

from _util import check_row_invariants, ensure_library, np_bits, np_f64, recall
from oracle import fp8_indexer as F, indexer as OI
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _rows(n, d, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(n, d, generator=g) * torch.exp(torch.randn(n, 1, generator=g) * 3)
    x[0] = 0.0                                   # zero row: scale 1, codes 0
    x[1] = 1e-3
    x[1, 5] = -300.0                             # one dominant element
    x[2] = torch.arange(d, dtype=torch.float32) - d / 2
    return x


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rotate_quantize_bit_exact(dsa, d, dt):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = _rows(70, d, d).to(tdt).to(DEV)
    codes, scales = dsa.dsa_rotate_quantize(x)
    torch.cuda.synchronize()
    rc, rs = F.rotate_quantize(np_f64(x).astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_rotate_quantize_into_cache_slots(dsa):
    """Keys written through a slot mapping: listed rows get the codes and
    scales, padding (-1) and out-of-range slots are skipped, other rows keep
    their contents; rows given as [tokens, heads, d] (queries) match too."""
    d, n, slots = 128, 40, 96
    x = _rows(n, d, 7).to(torch.bfloat16).to(DEV)
    g = torch.Generator(device="cpu").manual_seed(3)
    slot_map = torch.randperm(slots, generator=g)[:n].to(torch.int64)
    slot_map[[4, 17]] = -1
    slot_map[9] = slots + 5
    slot_map = slot_map.to(DEV)
    cache = torch.full((slots, d), 0x3C, dtype=torch.uint8, device=DEV)
    kscale = torch.full((slots,), 2.5, dtype=torch.float32, device=DEV)
    dsa.dsa_rotate_quantize(x, cache, kscale, row_slots=slot_map)
    torch.cuda.synchronize()
    rc, rs = F.rotate_quantize(np_f64(x).astype(np.float32))
    want_c = np.full((slots, d), 0x3C, np.uint8)
    want_s = np.full(slots, 2.5, np.float32)
    for i, sl in enumerate(slot_map.cpu().numpy()):
        if 0 <= sl < slots:
            want_c[sl], want_s[sl] = rc[i], rs[i]
    assert np.array_equal(cache.cpu().numpy(), want_c)
    assert np.array_equal(kscale.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    q = x.view(10, 4, d)
    qc, qs = dsa.dsa_rotate_quantize(q)
    torch.cuda.synchronize()
    assert qc.shape == (10, 4, d) and qs.shape == (10, 4)
    assert np.array_equal(qc.cpu().numpy().reshape(n, d), rc)


def _prepare(dsa, cfg, b, lay):
    """The library's FP8 path inputs (cache and queries) next to the
    oracle's own codes of the same bf16 values."""
    N = b.num_q_tokens
    cache = torch.zeros((b.num_slots, cfg.d_idx), dtype=torch.uint8, device=DEV)
    kscale = torch.zeros((b.num_slots,), dtype=torch.float32, device=DEV)
    all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=DEV)
    dsa.dsa_rotate_quantize(lay.k_src, cache, kscale, row_slots=all_slots)
    qc, qs = dsa.dsa_rotate_quantize(lay.q_idx)
    torch.cuda.synchronize()
    rkc, rks = F.rotate_quantize(np_f64(lay.k_src).astype(np.float32))
    rqc, rqs = F.rotate_quantize(np_f64(lay.q_idx).astype(np.float32))
    assert np.array_equal(cache.cpu().numpy(), rkc)
    assert np.array_equal(qc.cpu().numpy(), rqc)
    assert np.array_equal(kscale.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), rqs.view(np.uint32))
    return cache, kscale, qc, qs, (rkc, rks, rqc, rqs)


def _small(**kw):
    return get_config("fp8q_decode_32k_mtp").scaled(name="fp8q_small", cid=62, **kw)


@pytest.mark.parametrize("q_lens,topk,heads", [([1, 2, 3, 1, 2, 4], 64, 32),
                                               ([1, 1, 1, 1, 1, 1], 2048, 32),
                                               ([1, 2, 1, 2, 2, 2], 300, 64)])
def test_fp8q_ragged_matrix_core_path(dsa, q_lens, topk, heads):
    cfg = _small(num_reqs=6, topk=topk, n_idx_heads=heads)
    b = make_batch(cfg, DEV, seq_lens=[1, 37, 200, 1000, 3000, 5003], q_lens=q_lens)
    lay = make_layer(cfg, b, DEV)
    cache, kscale, qc, qs, (rkc, rks, rqc, rqs) = _prepare(dsa, cfg, b, lay)
    idx = dsa.dsa_indexer_topk_fp8q(dsa.Batch.from_synth(b), qc, qs, lay.w, cache, kscale, topk)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = F.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size, rqc, rqs,
                         np_f64(lay.w), rkc, rks, topk)
    t = 0
    for bi in range(b.num_reqs):
        for i in range(b.q_lens[bi]):
            pos = b.seq_lens[bi] - b.q_lens[bi] + i
            check_row_invariants(got[t], pos, topk)
            if pos + 1 <= topk:
                assert np.array_equal(got[t], ref[t])
            t += 1
    r, worst = recall(got, ref)
    assert r >= 0.999, (r, worst)


def test_fp8q_vector_path_and_long_rows(dsa):
    """Shapes off the matrix-core path (5 heads x 64 dims), and rows past the
    top-k's register reach on the matrix-core path."""
    cfg = _small(num_reqs=3, n_idx_heads=5, d_idx=64, topk=40)
    b = make_batch(cfg, DEV, seq_lens=[50, 129, 700], q_lens=[2, 1, 3])
    lay = make_layer(cfg, b, DEV)
    cache, kscale, qc, qs, (rkc, rks, rqc, rqs) = _prepare(dsa, cfg, b, lay)
    idx = dsa.dsa_indexer_topk_fp8q(dsa.Batch.from_synth(b), qc, qs, lay.w, cache, kscale, 40)
    torch.cuda.synchronize()
    ref = F.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size, rqc, rqs,
                         np_f64(lay.w), rkc, rks, 40)
    r, _ = recall(idx.cpu().numpy(), ref)
    assert r >= 0.999
    cfg = _small(num_reqs=2, q_len=1, topk=2048)
    b = make_batch(cfg, DEV, seq_lens=[40000, 70001], q_lens=[1, 1])
    lay = make_layer(cfg, b, DEV)
    cache, kscale, qc, qs, (rkc, rks, rqc, rqs) = _prepare(dsa, cfg, b, lay)
    idx = dsa.dsa_indexer_topk_fp8q(dsa.Batch.from_synth(b), qc, qs, lay.w, cache, kscale, 2048)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = F.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size, rqc, rqs,
                         np_f64(lay.w), rkc, rks, 2048)
    for t in range(2):
        check_row_invariants(got[t], b.seq_lens[t] - 1, 2048)
    r, _ = recall(got, ref)
    assert r >= 0.999


def test_fp8q_decode_32k_mtp_full(dsa):
    """The FP8-query path at the decode workload's full size, every row."""
    from _util import pool_map
    cfg = get_config("fp8q_decode_32k_mtp")
    b = make_batch(cfg, DEV)
    lay = make_layer(cfg, b, DEV)
    N = b.num_q_tokens
    cache = torch.empty((b.num_slots, cfg.d_idx), dtype=torch.uint8, device=DEV)
    kscale = torch.empty((b.num_slots,), dtype=torch.float32, device=DEV)
    all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=DEV)
    dsa.dsa_rotate_quantize(lay.k_src, cache, kscale, row_slots=all_slots)
    qc, qs = dsa.dsa_rotate_quantize(lay.q_idx)
    idx = dsa.dsa_indexer_topk_fp8q(dsa.Batch.from_synth(b), qc, qs, lay.w, cache, kscale,
                                    cfg.topk)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    pos = [b.seq_lens[bi] - b.q_lens[bi] + i for bi in range(b.num_reqs)
           for i in range(b.q_lens[bi])]
    for t in range(N):
        check_row_invariants(got[t], pos[t], cfg.topk)
    # the oracle's own codes of every key (in chunks) and of the queries
    kbits = np_bits(lay.k_src)
    n = kbits.shape[0]
    rkc = np.empty(kbits.shape, np.uint8)
    rks = np.empty(n, np.float32)

    def one(s):
        e = min(n, s + 32768)
        k32 = (kbits[s:e].astype(np.uint32) << np.uint32(16)).view(np.float32)
        rkc[s:e], rks[s:e] = F.rotate_quantize(k32)

    pool_map(one, range(0, n, 32768))
    assert np.array_equal(cache.cpu().numpy(), rkc)
    rqc, rqs = F.rotate_quantize(np_f64(lay.q_idx).astype(np.float32))
    assert np.array_equal(qc.cpu().numpy(), rqc)
    w64 = np_f64(lay.w)

    def req(bi):
        toks = list(range(int(b.cu_q_host[bi]), int(b.cu_q_host[bi + 1])))
        return toks, F.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host,
                                    b.block_size, rqc, rqs, w64, rkc, rks, cfg.topk,
                                    tokens=toks)

    ref = np.full_like(got, -1)
    for toks, rows in pool_map(req, range(b.num_reqs)):
        ref[toks] = rows[toks]
    r, worst = recall(got, ref)
    print("fp8q recall over %d rows %.6f (worst row %.6f)" % (N, r, worst), flush=True)
    assert r >= 0.999, (r, worst)
