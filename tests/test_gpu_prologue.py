"""GPU parity of the indexer prologue through the C ABI (page "GLM5
TensorCast 适配设计", section "DSA Indexer fused semantic op"; section
"Performance model design", buckets 1-4): q, k and w against the float64
oracle, elementwise, to the rounding of bf16 outputs over fp32 products;
the fused cache write bit for bit against the key the call returned."""
import numpy as np
import pytest
import torch

from _util import ensure_library, np_bits, np_f64, recall
from oracle import fp8_indexer as F, indexer as OI, prologue as P
from synth import get_config, make_batch, make_layer, make_prologue

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    return ensure_library()


def _close(gpu, ref, rtol=2.0 ** -8, arel=2e-3):
    """|gpu - ref| <= rtol |ref| + arel * rms(ref over the last dim): two bf16
    half-steps of the value, plus a small share of its row's scale for
    entries that cancel."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return float(np.max(np.abs(gpu - ref) - (rtol * np.abs(ref) + arel * rms)))


def _oracle(pi, cfg):
    return P.prologue(np_f64(pi.hidden), np_f64(pi.qa_normed), np_f64(pi.cos), np_f64(pi.sin),
                      np_f64(pi.wq_b), np_f64(pi.wk), np_f64(pi.weights_proj),
                      np_f64(pi.k_norm_weight), cfg.n_idx_heads, cfg.d_idx, cfg.idx_rope_dim,
                      cfg.norm_eps)


def _call(dsa, pi, cfg, **kw):
    return dsa.dsa_indexer_prologue(pi.hidden, pi.qa_normed, pi.cos, pi.sin, pi.wq_b, pi.wk,
                                    pi.weights_proj, pi.k_norm_weight, cfg.n_idx_heads,
                                    cfg.idx_rope_dim, cfg.norm_eps, **kw)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("heads,rope", [(4, 64), (7, 32), (32, 128)])
def test_prologue_small(dsa, cache, heads, rope):
    cfg = get_config("decode_32k_mtp").scaled(name="prologue_small", cid=63, num_reqs=5,
                                              n_idx_heads=heads, hidden_dim=512,
                                              q_lora_rank=256, idx_rope_dim=rope)
    b = make_batch(cfg, DEV, seq_lens=[100, 3000, 70, 2500, 90], q_lens=[9, 13, 1, 12, 2])
    pi = make_prologue(cfg, b, DEV)
    N = b.num_q_tokens                              # 37: a ragged last token tile
    slots = b.slot_mapping_t.clone()
    slots[[3, 20]] = -1
    if cache == "bf16":
        kc = torch.full((b.num_slots, 128), 7.0, dtype=torch.bfloat16, device=DEV)
        ks = None
    else:
        kc = torch.full((b.num_slots, 128), 0x3C, dtype=torch.uint8, device=DEV)
        ks = torch.full((b.num_slots,), 3.0, dtype=torch.float32, device=DEV)
    before = np_bits(kc).copy()
    q, k, w = _call(dsa, pi, cfg, slot_mapping=slots, k_cache=kc, k_scale=ks)
    torch.cuda.synchronize()
    rq, rk, rw = _oracle(pi, cfg)
    assert _close(np_f64(q), rq) <= 0
    assert _close(np_f64(k), rk) <= 0
    assert _close(w.cpu().numpy(), rw, rtol=1e-5, arel=1e-5) <= 0
    # the cache rows written are exactly the returned key (bf16), or its
    # rotation and quantisation (FP8); others keep their contents
    sl = slots.cpu().numpy()
    got = np_bits(kc)
    if cache == "bf16":
        want = before.copy()
        want[sl[sl >= 0]] = np_bits(k)[sl >= 0]
        assert np.array_equal(got, want)
    else:
        codes, scales = F.rotate_quantize(np_f64(k).astype(np.float32))
        want = before.copy()
        want[sl[sl >= 0]] = codes[sl >= 0]
        assert np.array_equal(got, want)
        sc = ks.cpu().numpy()
        assert np.array_equal(sc[sl[sl >= 0]].view(np.uint32), scales[sl >= 0].view(np.uint32))
    # repeatable bit for bit
    q2, k2, w2 = _call(dsa, pi, cfg)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(w, w2)


def test_prologue_decode_size_then_indexer(dsa):
    """The decode workload's new tokens (128 tokens, hidden 6144, q_lora_rank
    2048, 32 heads x 128, RoPE on 64 dims): every output against the oracle,
    then the indexer over the cache the prologue wrote, against the oracle
    on the same inputs."""
    cfg = get_config("decode_32k_mtp")
    b = make_batch(cfg, DEV)
    lay = make_layer(cfg, b, DEV)
    pi = make_prologue(cfg, b, DEV)
    kc = lay.k_src.clone()
    q, k, w = _call(dsa, pi, cfg, slot_mapping=b.slot_mapping_t, k_cache=kc)
    torch.cuda.synchronize()
    rq, rk, rw = _oracle(pi, cfg)
    assert _close(np_f64(q), rq) <= 0
    assert _close(np_f64(k), rk) <= 0
    assert _close(w.cpu().numpy(), rw, rtol=1e-5, arel=1e-5) <= 0
    assert torch.equal(kc[b.slot_mapping_t], k)
    bb = dsa.Batch.from_synth(b)
    idx = dsa.dsa_indexer_topk(bb, q, w, kc, None, cfg.topk)
    torch.cuda.synchronize()
    toks = list(range(0, b.num_q_tokens, 9))
    ref = OI.indexer_topk(b.seq_lens, b.cu_q_host, b.block_table_host, b.block_size,
                          np_f64(q), w.cpu().numpy().astype(np.float64), np_bits(kc), None,
                          OI.BF16, cfg.topk, tokens=toks)
    r, worst = recall(idx.cpu().numpy()[toks], ref[toks])
    assert r >= 0.999, (r, worst)
