"""Shared test plumbing: tensor -> numpy views, library loading, metrics.

No arithmetic of the method lives here."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_library():
    """Load the in-tree library; build it first only if it is missing."""
    import sparse_attention_topk_amd as dsa
    if not os.path.exists(dsa.library_path()):
        from sparse_attention_topk_amd.build import build
        build()
    dsa.load_library()
    return dsa


def np_bits(t):
    """Raw storage of a tensor as numpy (bf16 -> uint16, fp8 -> uint8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def np_f64(t):
    """Exact float64 values of a float / bf16 tensor."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def recall(gpu_rows, ref_rows):
    """sum_rows |S_gpu & S_ref| / sum_rows |S_ref| and the per-row minimum."""
    hit = tot = 0
    worst = 1.0
    for g, r in zip(gpu_rows, ref_rows):
        rs = set(int(x) for x in r if x >= 0)
        gs = set(int(x) for x in g if x >= 0)
        h = len(rs & gs)
        hit += h
        tot += len(rs)
        if rs:
            worst = min(worst, h / len(rs))
    return (hit / tot if tot else 1.0), worst


def check_row_invariants(row, pos, topk):
    """count = min(topk, pos+1), ascending, unique, 0 <= idx <= pos, -1 tail."""
    row = np.asarray(row)
    n = min(topk, pos + 1)
    sel = row[:n]
    assert np.all(row[n:] == -1), "padding"
    assert np.all(sel >= 0) and np.all(sel <= pos), "range"
    assert np.all(np.diff(sel) > 0), "ascending/unique"


def attn_close(gpu, ref, atol=2e-2, rtol=1e-2):
    """Elementwise |gpu - ref| <= atol + rtol |ref|; returns the worst excess."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    excess = np.abs(gpu - ref) - (atol + rtol * np.abs(ref))
    return float(np.max(excess)) if excess.size else -1.0


def pool_map(fn, items, workers=None):
    """fn over items in a thread pool sized to the host's cores (NumPy and
    BLAS release the GIL in the heavy parts).  Results in item order."""
    items = list(items)
    n = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)
