"""The C-ABI library loads on a host without a GPU, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest
import torch

from _util import ROOT, ensure_library

HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(?:int|size_t|const char\s*\*)\s+(\w+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    dsa = ensure_library()
    lib = dsa.load_library()
    declared = _declared()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(dsa.exported_symbols()) == declared


def test_checked_build_exports_every_declared_symbol():
    """libdsa_debug.so (the -DDSA_DEBUG build) carries the same ABI."""
    dsa = ensure_library()
    lib = dsa.load_library("debug")
    for name in _declared():
        assert hasattr(lib, name), name


def test_fault_word_only_in_the_checked_build():
    """The release library has no fault word: dsa_debug_faults sets 0 and
    reports DSA_ERR_UNSUPPORTED; both builds reject a NULL destination on
    the host (no device call is made in any of these)."""
    dsa = ensure_library()
    with dsa.use_library("release") as rel:
        out = ctypes.c_uint32(77)
        assert rel.dsa_debug_faults(ctypes.byref(out), 1) == -2
        assert out.value == 0
        assert "checked build" in dsa.dsa_last_error()
        assert rel.dsa_debug_faults(None, 0) == -1
        with pytest.raises(dsa.DSAError):
            dsa.debug_faults()
    assert dsa.load_library("debug").dsa_debug_faults(None, 0) == -1


def test_checked_build_validates_arguments_on_the_host_first():
    """The checked build rejects bad arguments before it enqueues its own
    checks (fake device addresses are never touched)."""
    dsa = ensure_library()
    lib = dsa.load_library("debug")
    assert _topk(lib, _batch(dsa), q=None) == -1
    assert _topk(lib, _batch(dsa), ws_bytes=16) == -5
    assert _topk(lib, _batch(dsa, num_reqs=-1)) == -1


def test_resolve_sources_matches_the_oracle():
    from oracle import indexshare as ix
    dsa = ensure_library()
    F, S = dsa.DSA_LAYER_FULL, dsa.DSA_LAYER_SHARED
    names = {F: ix.FULL, S: ix.SHARED}
    cases = [([F, S, S, S, F, S, S, S], 8), ([F], 1), ([F, F, S], 3),
             ([F, S, F, S, S], 5), ([F, S, S, F, S, S, S, S], 4)]
    for types, n in cases:
        assert dsa.dsa_resolve_indexer_sources(types, n) == \
            ix.resolve_sources([names[t] for t in types], n)
    for types, n in ([S, F], 2), ([F, S], 3), ([F, 7], 2), ([F, S, -1], 2):
        with pytest.raises(ValueError):
            dsa.dsa_resolve_indexer_sources(types, n)
        with pytest.raises(ValueError):
            ix.resolve_sources([names.get(t, "bogus") for t in types], n)


# Fake device addresses: every call below must fail host validation before
# anything touches them.
_FAKE = 1 << 40


def _batch(lib_mod, **kw):
    b = dict(num_reqs=2, num_q_tokens=4, max_q_len=2, max_seq_len=128,
             max_blocks=2, block_size=64, num_slots=256, seq_lens=_FAKE,
             cu_q=_FAKE, block_table=_FAKE)
    b.update(kw)
    return lib_mod._binding._CBatch(**b)


def _topk(lib, cb, **kw):
    a = dict(q=_FAKE, q_dtype=1, w=_FAKE, n_heads=32, d_idx=128,
             k_cache=_FAKE, k_scale=None, cache_dtype=1, topk=16,
             topk_idx=_FAKE, ws=_FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.dsa_indexer_topk(ctypes.byref(cb), a["q"], a["q_dtype"], a["w"],
                                a["n_heads"], a["d_idx"], a["k_cache"],
                                a["k_scale"], a["cache_dtype"], a["topk"],
                                a["topk_idx"], a["ws"], a["ws_bytes"],
                                a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(topk_idx=None), -1),
    (dict(q_dtype=9), -1),
    (dict(q_dtype=2, cache_dtype=2), -2),
    (dict(cache_dtype=2), -1),            # FP8 cache without k_scale
    (dict(q_dtype=0, cache_dtype=1), -2),
    (dict(n_heads=65), -2),
    (dict(d_idx=300), -2),
    (dict(topk=0), -2),
    (dict(topk=5000), -2),
    (dict(ws=None), -5),
    (dict(ws_bytes=10), -5),
    (dict(ws=_FAKE + 8), -1),             # misaligned workspace
])
def test_indexer_topk_rejects_on_host(kw, code):
    dsa = ensure_library()
    lib = dsa.load_library()
    assert _topk(lib, _batch(dsa), **kw) == code
    assert dsa.dsa_last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(num_reqs=0), -1),
    (dict(block_size=48), -2),
    (dict(max_blocks=1), -1),             # 1 * 64 < max_seq_len 128
    (dict(max_q_len=200), -1),
    (dict(seq_lens=None), -1),
    (dict(num_slots=0), -1),
])
def test_batch_geometry_is_validated(kw, code):
    dsa = ensure_library()
    lib = dsa.load_library()
    assert _topk(lib, _batch(dsa, **kw)) == code


def test_workspace_size_formula():
    dsa = ensure_library()
    lib = dsa.load_library()
    cb = _batch(dsa)
    def up(x):
        return (x + 255) // 256 * 256
    # fp32 score rows padded to a multiple of 64 positions, then per token
    # 4 (min, max) float pairs for each possible chunk of 128 keys
    assert lib.dsa_indexer_topk_workspace_size(ctypes.byref(cb), 16) == (
        up(4 * 128 * 4) + up(4 * 4 * 1 * 8))
    cb100 = _batch(dsa, max_seq_len=100)
    assert lib.dsa_indexer_topk_workspace_size(ctypes.byref(cb100), 16) == (
        up(4 * 128 * 4) + up(4 * 4 * 1 * 8))
    cb_long = _batch(dsa, max_seq_len=32768)
    assert lib.dsa_indexer_topk_workspace_size(ctypes.byref(cb_long), 16) == (
        up(4 * 32768 * 4) + up(4 * 4 * 256 * 8))
    # no split for the vector path, so no MLA workspace
    assert lib.sparse_mla_attn_workspace_size(ctypes.byref(cb), 4, 64, 16, 16, 0) == 0
    # the matrix-core path with few workgroups splits the keys of a token:
    # 4 tokens -> 16 splits (at least 4 tiles of 32 keys each, enough
    # workgroups for 256 CUs); bf16 partials [N, split, H, R], their
    # log-sum-exps [N, split, H] and a 128-byte line per token for its
    # arrival word, each region 256-byte aligned
    th = 4 * 16 * 64
    assert lib.sparse_mla_attn_workspace_size(ctypes.byref(cb), 64, 512, 64, 2048, 1) == (
        up(th * 512 * 2) + up(th * 4) + up(4 * 128))
    # 128 decode tokens: 2 splits
    cb128 = _batch(dsa, num_reqs=64, num_q_tokens=128, max_q_len=2)
    th = 128 * 2 * 64
    assert lib.sparse_mla_attn_workspace_size(ctypes.byref(cb128), 64, 512, 64, 2048, 1) == (
        up(th * 512 * 2) + up(th * 4) + up(128 * 128))


def test_indexer_workspace_windows():
    """The least accepted indexer workspace is a window of 16 query tokens
    (score rows and range entries), or the whole batch when it has fewer;
    one byte less is refused on the host before anything is enqueued."""
    dsa = ensure_library()
    lib = dsa.load_library()
    def up(x):
        return (x + 255) // 256 * 256
    cb = _batch(dsa, num_reqs=64, num_q_tokens=128, max_q_len=2, max_seq_len=32768,
                max_blocks=512, num_slots=64 * 32768)
    full = lib.dsa_indexer_topk_workspace_size(ctypes.byref(cb), 2048)
    least = lib.dsa_indexer_topk_workspace_min(ctypes.byref(cb), 2048)
    assert full == up(128 * 32768 * 4) + up(128 * 4 * 256 * 8)
    assert least == up(16 * 32768 * 4) + up(16 * 4 * 256 * 8)
    assert _topk(lib, cb, topk=2048, ws_bytes=least - 1) == -5
    assert "at least" in dsa.dsa_last_error()
    small = _batch(dsa)                                  # 4 query tokens
    assert (lib.dsa_indexer_topk_workspace_min(ctypes.byref(small), 16) ==
            lib.dsa_indexer_topk_workspace_size(ctypes.byref(small), 16))


def test_mla_and_cache_write_reject_on_host():
    dsa = ensure_library()
    lib = dsa.load_library()
    cb = _batch(dsa)
    P = _FAKE
    # bad dtype
    assert lib.sparse_mla_attn(ctypes.byref(cb), P, P, 2, 4, 64, 16, P, 16,
                               ctypes.c_float(0.1), P, None, None, 0, None) == -2
    # missing workspace for the split path
    assert lib.sparse_mla_attn(ctypes.byref(cb), P, P, 1, 64, 512, 64, P, 2048,
                               ctypes.c_float(0.1), P, None, None, 0, None) == -5
    assert lib.sparse_mla_attn(ctypes.byref(cb), None, P, 1, 4, 64, 16, P, 16,
                               ctypes.c_float(0.1), P, None, None, 0, None) == -1
    # the softmax scale must be finite and positive
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert lib.sparse_mla_attn(ctypes.byref(cb), P, P, 1, 4, 64, 16, P, 16,
                                   ctypes.c_float(bad), P, None, None, 0, None) == -1
    # cache write: bf16 keys into an f32 cache, fp8 without scale, bad d
    assert lib.dsa_indexer_cache_write(P, 1, 4, 128, P, 256, P, None, 0, None) == -2
    assert lib.dsa_indexer_cache_write(P, 1, 4, 128, P, 256, P, None, 2, None) == -1
    assert lib.dsa_indexer_cache_write(P, 1, 4, 0, P, 256, P, None, 1, None) == -1
    assert lib.dsa_indexer_cache_write(P, 2, 4, 128, P, 256, P, P, 2, None) == -2
    # n_new == 0 is a no-op that succeeds without touching the GPU
    assert lib.dsa_indexer_cache_write(None, 1, 0, 128, None, 256, None, None, 1, None) == 0


def test_indexshare_rejects_on_host():
    dsa = ensure_library()
    b = dsa.Batch(seq_lens=torch.zeros(2, dtype=torch.int32),
                  cu_q=torch.zeros(3, dtype=torch.int32),
                  block_table=torch.zeros((2, 2), dtype=torch.int32),
                  num_q_tokens=2, max_q_len=1, max_seq_len=128, block_size=64,
                  num_slots=256)
    dims = dsa.StackDims(32, 128, dsa.DSA_BF16, dsa.DSA_BF16, 16, 64, 512, 64,
                         dsa.DSA_BF16, 0.04)
    t = torch.zeros(8, dtype=torch.bfloat16)
    L = dsa.Layer(q_mla=t, kv_cache=t, out=t, q_idx=t, w=t.float(), k_cache=t,
                  topk_idx=None)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    # shared first layer -> ValueError; full layer without top-k buffer too
    with pytest.raises(ValueError, match="no preceding full"):
        dsa.indexshare_forward(b, [dsa.DSA_LAYER_SHARED, dsa.DSA_LAYER_FULL], [L, L], dims, workspace=ws)
    with pytest.raises(ValueError, match="no topk_idx"):
        dsa.indexshare_forward(b, [dsa.DSA_LAYER_FULL, dsa.DSA_LAYER_SHARED], [L, L], dims, workspace=ws)
    with pytest.raises(ValueError, match="entries"):
        dsa.indexshare_forward(b, [dsa.DSA_LAYER_FULL], [L, L], dims, workspace=ws)


def test_noalloc_rejects_oversized_batches_on_the_host():
    """The allocation-free indexer call refuses a batch whose scratch would
    exceed its static array, before touching the device."""
    dsa = ensure_library()
    lib = dsa.load_library()
    cb = _batch(dsa, num_q_tokens=128, max_q_len=1, max_seq_len=131072, max_blocks=2048,
                num_slots=1 << 24)
    rc = lib.dsa_indexer_topk_noalloc(ctypes.byref(cb), _FAKE, 1, _FAKE, 32, 128, _FAKE,
                                      None, 1, 2048, _FAKE, None)
    assert rc == -5
    assert "allocation-free" in dsa.dsa_last_error()


def test_fp8_query_entry_points_reject_on_the_host():
    dsa = ensure_library()
    lib = dsa.load_library()
    # rotation sizes: powers of two in 32..256 only
    for d, code in ((100, -2), (16, -2), (512, -2)):
        assert lib.dsa_rotate_quantize(_FAKE, 1, 4, d, None, 4, _FAKE, _FAKE, None) == code
    assert lib.dsa_rotate_quantize(_FAKE, 2, 4, 128, None, 4, _FAKE, _FAKE, None) == -2
    assert lib.dsa_rotate_quantize(_FAKE, 1, 8, 128, None, 4, _FAKE, _FAKE, None) == -1
    cb = _batch(dsa)
    assert lib.dsa_indexer_topk_fp8q(ctypes.byref(cb), _FAKE, None, _FAKE, 32, 128, _FAKE,
                                     _FAKE, 16, _FAKE, _FAKE, 1 << 30, None) == -1
    assert lib.dsa_indexer_topk_fp8q(ctypes.byref(cb), _FAKE, _FAKE, _FAKE, 32, 128, _FAKE,
                                     None, 16, _FAKE, _FAKE, 1 << 30, None) == -1
