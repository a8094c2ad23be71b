"""ctypes marshalling for include/dsa.h (no computation here)."""

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# "release": libdsa.so; "debug": the checked build libdsa_debug.so (metadata
# validation and output canaries around every call, see dsa_debug_faults).
# DSA_LIBRARY=debug in the environment selects the checked build.
_LIB_NAMES = {"release": "libdsa.so", "debug": "libdsa_debug.so"}
_variant = os.environ.get("DSA_LIBRARY", "release")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED = 0, -1, -2
DSA_ERR_INDEXER_TYPES, DSA_ERR_MISSING_TOPK = -3, -4
DSA_ERR_WORKSPACE, DSA_ERR_HIP = -5, -6
DSA_LAYER_FULL, DSA_LAYER_SHARED = 0, 1

EXPORTS = [
    "dsa_indexer_cache_write", "dsa_indexer_topk_workspace_size",
    "dsa_indexer_topk_workspace_min",
    "dsa_indexer_topk", "dsa_indexer_topk_noalloc", "dsa_rotate_quantize",
    "dsa_indexer_topk_fp8q", "dsa_indexer_prologue_workspace_size", "dsa_indexer_prologue",
    "sparse_mla_attn_workspace_size",
    "sparse_mla_attn",
    "dsa_resolve_indexer_sources", "indexshare_forward_workspace_size",
    "indexshare_forward", "dsa_fp8_decode_check", "dsa_debug_faults", "dsa_last_error",
]
DSA_FAULT_SEQ_LENS, DSA_FAULT_CU_Q, DSA_FAULT_BLOCK_TABLE = 1, 2, 4
DSA_FAULT_SLOT_MAPPING, DSA_FAULT_TOPK_INPUT, DSA_FAULT_TOPK_OUTPUT = 8, 16, 32
DSA_FAULT_UNWRITTEN = 64


class DSAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libdsa error %d: %s" % (code, msg))
        self.code = code


class _CBatch(ctypes.Structure):
    _fields_ = [
        ("num_reqs", ctypes.c_int32), ("num_q_tokens", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_slots", ctypes.c_int64), ("seq_lens", ctypes.c_void_p),
        ("cu_q", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
    ]


class _CLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q_idx", "w", "k_cache", "k_scale", "topk_idx", "q_mla", "kv_cache",
        "out", "lse")]


class _CPrologueDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden_dim", "q_lora_rank", "n_heads", "head_dim", "rope_dim")] + [
        ("eps", ctypes.c_float)]


class _CDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_idx_heads", "d_idx", "q_idx_dtype", "idx_cache_dtype", "topk",
        "n_heads", "kv_lora_rank", "rope_dim", "mla_dtype")] + [
        ("softmax_scale", ctypes.c_float)]


_loaded = {}


def library_path(variant=None):
    if variant not in _LIB_NAMES:
        variant = _variant
    return os.path.join(HERE, _LIB_NAMES[variant])


def load_library(variant=None):
    """Load the active library (or `variant`) once; raises if it is missing
    (no fallback path)."""
    v = variant if variant in _LIB_NAMES else _variant
    if v in _loaded:
        return _loaded[v]
    path = library_path() if variant is None else library_path(v)
    if not os.path.exists(path):
        raise RuntimeError(
            "%s not found; build it with "
            "`python -m sparse_attention_topk_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    F = ctypes.c_float
    sig = {
        "dsa_indexer_cache_write": (ctypes.c_int, [P, I32, I32, I32, P, I64, P, P, I32, P]),
        "dsa_indexer_topk_workspace_size": (SZ, [P, I32]),
        "dsa_indexer_topk_workspace_min": (SZ, [P, I32]),
        "dsa_indexer_topk": (ctypes.c_int, [P, P, I32, P, I32, I32, P, P, I32, I32, P, P, SZ, P]),
        "dsa_indexer_topk_noalloc": (ctypes.c_int, [P, P, I32, P, I32, I32, P, P, I32, I32, P, P]),
        "dsa_rotate_quantize": (ctypes.c_int, [P, I32, I64, I32, P, I64, P, P, P]),
        "dsa_indexer_topk_fp8q": (ctypes.c_int, [P, P, P, P, I32, I32, P, P, I32, P, P, SZ, P]),
        "dsa_indexer_prologue_workspace_size": (SZ, [I32, P]),
        "dsa_indexer_prologue": (ctypes.c_int, [I32, P, P, P, P, P, P, P, P, P, P, I64, P, P,
                                                I32, P, P, P, P, SZ, P]),
        "sparse_mla_attn_workspace_size": (SZ, [P, I32, I32, I32, I32, I32]),
        "sparse_mla_attn": (ctypes.c_int, [P, P, P, I32, I32, I32, I32, P, I32, F, P, P, P, SZ, P]),
        "dsa_resolve_indexer_sources": (ctypes.c_int, [I32, P, I32, P]),
        "indexshare_forward_workspace_size": (SZ, [P, P]),
        "indexshare_forward": (ctypes.c_int, [P, I32, P, I32, P, P, P, P, SZ, P]),
        "dsa_fp8_decode_check": (ctypes.c_int, [P, P, I32, P]),
        "dsa_debug_faults": (ctypes.c_int, [P, I32]),
        "dsa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _loaded[v] = lib
    return lib


@contextlib.contextmanager
def use_library(variant):
    """Make `variant` ("release" or "debug") the library every call goes
    through inside the block."""
    global _variant
    if variant not in _LIB_NAMES:
        raise ValueError("unknown library variant %r" % (variant,))
    prev = _variant
    _variant = variant
    try:
        yield load_library()
    finally:
        _variant = prev


def debug_faults(clear=True):
    """The checked build's fault word (DSA_FAULT_* bits) for the current
    device; waits for the device.  Raises DSAError on the release build."""
    out = ctypes.c_uint32(0)
    _check(load_library().dsa_debug_faults(ctypes.byref(out), 1 if clear else 0))
    return out.value


def exported_symbols():
    lib = load_library()
    return [n for n in EXPORTS if hasattr(lib, n)]


def dsa_last_error():
    return load_library().dsa_last_error().decode()


def _check(code):
    if code == DSA_OK:
        return
    msg = dsa_last_error()
    if code in (DSA_ERR_INDEXER_TYPES, DSA_ERR_MISSING_TOPK):
        raise ValueError(msg)
    raise DSAError(code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch_stream(stream):
    """A torch stream object for `stream` (a torch.cuda.Stream or a raw
    hipStream_t handle)."""
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream):
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    if stream is not None:
        return ctypes.c_void_p(stream)
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(0)


def _dtype(t):
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3
    raise TypeError("unsupported dtype %s" % t.dtype)


def _contig(name, t):
    if t is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


@dataclass
class Batch:
    """Ragged batch + paged-cache geometry (device tensors + host bounds)."""
    seq_lens: torch.Tensor          # int32 [B]
    cu_q: torch.Tensor              # int32 [B+1]
    block_table: torch.Tensor       # int32 [B, max_blocks]
    num_q_tokens: int
    max_q_len: int
    max_seq_len: int
    block_size: int
    num_slots: int

    def c(self):
        for n in ("seq_lens", "cu_q", "block_table"):
            t = getattr(self, n)
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("%s must be contiguous int32" % n)
        cb = _CBatch(
            num_reqs=self.seq_lens.numel(), num_q_tokens=self.num_q_tokens,
            max_q_len=self.max_q_len, max_seq_len=self.max_seq_len,
            max_blocks=self.block_table.shape[1], block_size=self.block_size,
            num_slots=self.num_slots, seq_lens=self.seq_lens.data_ptr(),
            cu_q=self.cu_q.data_ptr(), block_table=self.block_table.data_ptr())
        return cb

    @staticmethod
    def from_synth(b):
        """From a synth.Batch (same fields)."""
        return Batch(seq_lens=b.seq_lens_t, cu_q=b.cu_q_t,
                     block_table=b.block_table_t, num_q_tokens=b.num_q_tokens,
                     max_q_len=b.max_q_len, max_seq_len=b.max_seq_len,
                     block_size=b.block_size, num_slots=b.num_slots)


def dsa_indexer_cache_write(k_new, slot_mapping, k_cache, k_scale=None,
                            stream=None):
    lib = load_library()
    _contig("k_new", k_new), _contig("k_cache", k_cache)
    n_new, d = (k_new.shape[0], k_new.shape[1]) if k_new.dim() == 2 else (0, k_cache.shape[-1])
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    _check(lib.dsa_indexer_cache_write(
        _ptr(k_new), _dtype(k_new), n_new, d, _ptr(slot_mapping),
        k_cache.shape[0], _ptr(k_cache), _ptr(k_scale), _dtype(k_cache),
        _stream(stream)))


def dsa_indexer_topk_workspace_size(batch, topk):
    cb = batch.c()
    return load_library().dsa_indexer_topk_workspace_size(ctypes.byref(cb), topk)


def dsa_indexer_topk_workspace_min(batch, topk):
    """The least workspace dsa_indexer_topk accepts (it then works through the
    query tokens in windows)."""
    cb = batch.c()
    return load_library().dsa_indexer_topk_workspace_min(ctypes.byref(cb), topk)


def _workspace(nbytes, device, workspace, stream=None):
    """The caller's workspace, or a fresh one.  A fresh one is allocated on
    the stream the kernels run on, so the caching allocator does not hand its
    memory to other work before those kernels are done with it."""
    if workspace is not None:
        return workspace
    if nbytes == 0:
        return None
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(_torch_stream(stream)):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def dsa_indexer_topk(batch, q, w, k_cache, k_scale, topk, topk_idx=None,
                     workspace=None, cache_dtype=None, stream=None):
    lib = load_library()
    for n, t in (("q", q), ("w", w), ("k_cache", k_cache), ("k_scale", k_scale)):
        _contig(n, t)
    N, H, D = q.shape
    if topk_idx is None:
        topk_idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    cb = batch.c()
    ws = _workspace(lib.dsa_indexer_topk_workspace_size(ctypes.byref(cb), topk),
                    q.device, workspace, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsa_indexer_topk(
        ctypes.byref(cb), _ptr(q), _dtype(q), _ptr(w), H, D, _ptr(k_cache),
        _ptr(k_scale), _dtype(k_cache) if cache_dtype is None else cache_dtype,
        topk, _ptr(topk_idx), _ptr(ws), ws_bytes, _stream(stream)))
    return topk_idx


def dsa_indexer_topk_noalloc(batch, q, w, k_cache, k_scale, topk, topk_idx,
                             cache_dtype=None, stream=None):
    """The allocation-free indexer call: the caller passes the output buffer;
    the library's static per-device scratch replaces the workspace."""
    lib = load_library()
    for n, t in (("q", q), ("w", w), ("k_cache", k_cache), ("k_scale", k_scale),
                 ("topk_idx", topk_idx)):
        _contig(n, t)
    N, H, D = q.shape
    cb = batch.c()
    _check(lib.dsa_indexer_topk_noalloc(
        ctypes.byref(cb), _ptr(q), _dtype(q), _ptr(w), H, D, _ptr(k_cache),
        _ptr(k_scale), _dtype(k_cache) if cache_dtype is None else cache_dtype,
        topk, _ptr(topk_idx), _stream(stream)))
    return topk_idx


def dsa_rotate_quantize(x, codes=None, scales=None, row_slots=None, stream=None):
    """Hadamard-rotate and e4m3-quantise the rows of x [..., d].  Without
    row_slots the outputs have x's row shape (allocated when not given);
    with row_slots (int64, one per row) codes / scales are the destination
    cache [num_out, d] / [num_out] and row i goes to row row_slots[i]."""
    lib = load_library()
    _contig("x", x)
    d = x.shape[-1]
    n = x.numel() // d if d else 0
    if row_slots is None:
        if codes is None:
            codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if scales is None:
            scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        num_out = n
    else:
        if codes is None or scales is None:
            raise ValueError("row_slots needs the destination codes and scales")
        if row_slots.dtype != torch.int64 or row_slots.numel() != n:
            raise ValueError("row_slots must be int64 with one entry per row")
        num_out = codes.shape[0]
    _contig("codes", codes), _contig("scales", scales)
    _check(lib.dsa_rotate_quantize(_ptr(x), _dtype(x), n, d, _ptr(row_slots), num_out,
                                   _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def dsa_indexer_topk_fp8q(batch, q_codes, q_scale, w, k_cache, k_scale, topk,
                          topk_idx=None, workspace=None, stream=None):
    lib = load_library()
    for n, t in (("q_codes", q_codes), ("q_scale", q_scale), ("w", w),
                 ("k_cache", k_cache), ("k_scale", k_scale)):
        _contig(n, t)
    N, H, D = q_codes.shape
    if topk_idx is None:
        topk_idx = torch.empty((N, topk), dtype=torch.int32, device=q_codes.device)
    cb = batch.c()
    ws = _workspace(lib.dsa_indexer_topk_workspace_size(ctypes.byref(cb), topk),
                    q_codes.device, workspace, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dsa_indexer_topk_fp8q(
        ctypes.byref(cb), _ptr(q_codes), _ptr(q_scale), _ptr(w), H, D, _ptr(k_cache),
        _ptr(k_scale), topk, _ptr(topk_idx), _ptr(ws), ws_bytes, _stream(stream)))
    return topk_idx


def dsa_indexer_prologue(hidden, qa_normed, cos, sin, wq_b, wk, weights_proj, k_norm_weight,
                         n_heads, rope_dim, eps, slot_mapping=None, k_cache=None, k_scale=None,
                         q_out=None, k_out=None, w_out=None, workspace=None, want_k=True,
                         stream=None):
    """q [N, H, D] bf16, k [N, D] bf16 (or None), w [N, H] fp32 of N new tokens;
    with slot_mapping, k is also written into k_cache (bf16 copy, or rotated
    and quantised into an e4m3 cache with k_scale)."""
    lib = load_library()
    for n, t in (("hidden", hidden), ("qa_normed", qa_normed), ("cos", cos), ("sin", sin),
                 ("wq_b", wq_b), ("wk", wk), ("weights_proj", weights_proj),
                 ("k_norm_weight", k_norm_weight), ("k_cache", k_cache)):
        _contig(n, t)
    N, hidden_dim = hidden.shape
    D = wk.shape[0]
    dims = _CPrologueDims(hidden_dim=hidden_dim, q_lora_rank=qa_normed.shape[1],
                          n_heads=n_heads, head_dim=D, rope_dim=rope_dim, eps=eps)
    dev = hidden.device
    if q_out is None:
        q_out = torch.empty((N, n_heads, D), dtype=torch.bfloat16, device=dev)
    if k_out is None and want_k:
        k_out = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    if w_out is None:
        w_out = torch.empty((N, n_heads), dtype=torch.float32, device=dev)
    ws = _workspace(lib.dsa_indexer_prologue_workspace_size(N, ctypes.byref(dims)), dev,
                    workspace, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    cache_dtype = _dtype(k_cache) if k_cache is not None else DSA_BF16
    num_slots = k_cache.shape[0] if k_cache is not None else 0
    _check(lib.dsa_indexer_prologue(
        N, ctypes.byref(dims), _ptr(hidden), _ptr(qa_normed), _ptr(cos), _ptr(sin), _ptr(wq_b),
        _ptr(wk), _ptr(weights_proj), _ptr(k_norm_weight), _ptr(slot_mapping), num_slots,
        _ptr(k_cache), _ptr(k_scale), cache_dtype, _ptr(q_out), _ptr(k_out), _ptr(w_out),
        _ptr(ws), ws_bytes, _stream(stream)))
    return q_out, k_out, w_out


def sparse_mla_attn_workspace_size(batch, n_heads, kv_lora_rank, rope_dim,
                                   topk, dtype):
    cb = batch.c()
    return load_library().sparse_mla_attn_workspace_size(
        ctypes.byref(cb), n_heads, kv_lora_rank, rope_dim, topk, dtype)


def sparse_mla_attn(batch, q, kv_cache, topk_idx, kv_lora_rank, softmax_scale,
                    out=None, lse=None, workspace=None, want_lse=True,
                    stream=None):
    lib = load_library()
    for n, t in (("q", q), ("kv_cache", kv_cache), ("topk_idx", topk_idx)):
        _contig(n, t)
    N, H, Dl = q.shape
    rope = Dl - kv_lora_rank
    topk = topk_idx.shape[1]
    if out is None:
        out = torch.empty((N, H, kv_lora_rank), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((N, H), dtype=torch.float32, device=q.device)
    cb = batch.c()
    dt = _dtype(q)
    ws = _workspace(lib.sparse_mla_attn_workspace_size(
        ctypes.byref(cb), H, kv_lora_rank, rope, topk, dt), q.device, workspace, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.sparse_mla_attn(
        ctypes.byref(cb), _ptr(q), _ptr(kv_cache), dt, H, kv_lora_rank, rope,
        _ptr(topk_idx), topk, ctypes.c_float(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))
    return out, lse


def dsa_resolve_indexer_sources(types: Sequence[int], n_layers: int):
    lib = load_library()
    arr = (ctypes.c_int32 * max(1, len(types)))(*types)
    src = (ctypes.c_int32 * max(1, n_layers))()
    _check(lib.dsa_resolve_indexer_sources(n_layers, arr, len(types), src))
    return list(src)[:n_layers]


@dataclass
class Layer:
    q_mla: torch.Tensor
    kv_cache: torch.Tensor
    out: torch.Tensor
    lse: Optional[torch.Tensor] = None
    q_idx: Optional[torch.Tensor] = None
    w: Optional[torch.Tensor] = None
    k_cache: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    topk_idx: Optional[torch.Tensor] = None


@dataclass
class StackDims:
    n_idx_heads: int
    d_idx: int
    q_idx_dtype: int
    idx_cache_dtype: int
    topk: int
    n_heads: int
    kv_lora_rank: int
    rope_dim: int
    mla_dtype: int
    softmax_scale: float

    def c(self):
        return _CDims(**self.__dict__)


def indexshare_forward_workspace_size(batch, dims):
    cb, cd = batch.c(), dims.c()
    return load_library().indexshare_forward_workspace_size(ctypes.byref(cb),
                                                            ctypes.byref(cd))


def indexshare_forward(batch, types: Sequence[int], layers: List[Layer],
                       dims: StackDims, workspace=None, device=None,
                       stream=None):
    """Returns the device address of the top-k buffer each layer used."""
    lib = load_library()
    cb, cd = batch.c(), dims.c()
    arr = (ctypes.c_int32 * max(1, len(types)))(*types)
    cl = (_CLayer * len(layers))()
    for i, L in enumerate(layers):
        for n in _CLayer._fields_:
            t = getattr(L, n[0])
            setattr(cl[i], n[0], None if t is None else t.data_ptr())
    device = device or layers[0].q_mla.device
    ws = _workspace(lib.indexshare_forward_workspace_size(ctypes.byref(cb),
                                                          ctypes.byref(cd)),
                    device, workspace, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    act = (ctypes.c_void_p * len(layers))()
    _check(lib.indexshare_forward(ctypes.byref(cb), len(layers), arr, len(types),
                                  cl, ctypes.byref(cd), act, _ptr(ws), ws_bytes,
                                  _stream(stream)))
    return [a or 0 for a in act]


def dsa_fp8_decode_check(codes, out=None, stream=None):
    lib = load_library()
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib.dsa_fp8_decode_check(_ptr(codes), _ptr(out), codes.numel(),
                                    _stream(stream)))
    return out
