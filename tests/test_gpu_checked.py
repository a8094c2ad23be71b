"""GPU tests of the checked build (libdsa_debug.so, -DDSA_DEBUG).

The checked build enqueues, around every call, a validation of the
device-resident metadata against the batch's host-side bounds, canary fills
of the outputs and workspace, and afterwards a check that every output was
written and every indexer row is a valid selection.  On valid input it must
find nothing and give the release library's results bit for bit (the checks
never change the arithmetic, and the canaries show that no output element is
left unwritten and no result depends on what the workspace held).  On bad
metadata it must raise the matching fault bit; every case below is one the
release kernels already clamp or skip, so no memory outside the buffers is
touched."""
import dataclasses

import pytest
import torch

from _util import ensure_library
from synth import get_config, make_batch, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    d = ensure_library()
    d.load_library("debug")
    return d


def _cfg(**kw):
    return get_config("decode_32k_mtp").scaled(name="checked", cid=64, **kw)


def _calls(dsa, bb, lay, cfg, idx=None):
    if idx is None:
        idx = dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, lay.k_src, None, cfg.topk)
    out, lse = dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, idx, cfg.kv_lora_rank,
                                   cfg.softmax_scale)
    torch.cuda.synchronize()
    return idx, out, lse


@pytest.mark.parametrize("shape", ["decode", "prefill"])
def test_checked_build_matches_release_and_finds_nothing(dsa, shape):
    """Decode-shaped (2 query tokens per request, split attention) and
    prefill-shaped (blocks of 16 query tokens, one workgroup per token)
    batches, plus a cache write: no fault, and the same bits as the
    release build."""
    if shape == "decode":
        cfg = _cfg(num_reqs=4, topk=512)
        b = make_batch(cfg, DEV, seq_lens=[3000, 700, 5000, 1300], q_lens=[2, 2, 1, 2])
    else:
        cfg = _cfg(num_reqs=2, topk=256)
        b = make_batch(cfg, DEV, seq_lens=[600, 2000], q_lens=[40, 300])
    print("checked build case: %s seq_lens %s q_lens %s" % (shape, b.seq_lens, b.q_lens),
          flush=True)
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    with dsa.use_library("release"):
        ref = _calls(dsa, bb, lay, cfg)
    with dsa.use_library("debug"):
        dsa.debug_faults(clear=True)
        got = _calls(dsa, bb, lay, cfg)
        # a cache write of this step's keys to their own slots
        slots = b.slot_mapping_t
        dsa.dsa_indexer_cache_write(lay.k_src[slots].contiguous(), slots, lay.k_src)
        assert dsa.debug_faults() == 0
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


def _faults_of(dsa, fn):
    with dsa.use_library("debug"):
        dsa.debug_faults(clear=True)
        fn()
        torch.cuda.synchronize()
        return dsa.debug_faults()


def test_checked_build_reports_bad_metadata(dsa):
    cfg = _cfg(num_reqs=3, topk=256)
    b = make_batch(cfg, DEV, seq_lens=[1500, 900, 2400], q_lens=[2, 2, 2])
    lay = make_layer(cfg, b, DEV)
    bb = dsa.Batch.from_synth(b)
    with dsa.use_library("release"):
        idx, _, _ = _calls(dsa, bb, lay, cfg)

    # an attention index past its token's position (token 0 sits at 1498)
    print("checked build case: index past the position", flush=True)
    bad_idx = idx.clone()
    bad_idx[0, 5] = 1499 + 7
    f = _faults_of(dsa, lambda: _calls(dsa, bb, lay, cfg, idx=bad_idx))
    assert f & dsa.DSA_FAULT_TOPK_INPUT, f

    # a block of request 1 that is in use points past the cache
    print("checked build case: block id past the cache", flush=True)
    bt = bb.block_table.clone()
    bt[1, 1] = b.num_slots // b.block_size + 5
    bad = dataclasses.replace(bb, block_table=bt)
    f = _faults_of(dsa, lambda: _calls(dsa, bad, lay, cfg))
    assert f & dsa.DSA_FAULT_BLOCK_TABLE, f

    # a context longer than the batch's max_seq_len
    print("checked build case: seq_len past max_seq_len", flush=True)
    sl = bb.seq_lens.clone()
    sl[2] = b.max_seq_len + 100
    bad = dataclasses.replace(bb, seq_lens=sl)
    f = _faults_of(dsa, lambda: _calls(dsa, bad, lay, cfg))
    assert f & dsa.DSA_FAULT_SEQ_LENS, f

    # a cache-write slot past the cache (the kernel skips it)
    print("checked build case: slot past the cache", flush=True)
    slots = b.slot_mapping_t.clone()
    keys = lay.k_src[slots].contiguous()
    slots[1] = b.num_slots + 3
    f = _faults_of(dsa, lambda: dsa.dsa_indexer_cache_write(keys, slots, lay.k_src))
    assert f == dsa.DSA_FAULT_SLOT_MAPPING, f

    # and a valid call afterwards finds nothing again
    f = _faults_of(dsa, lambda: _calls(dsa, bb, lay, cfg))
    assert f == 0, f
