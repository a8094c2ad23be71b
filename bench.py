"""Benchmark of the DSA decode hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. dsa_indexer_cache_write  - the step's new indexer keys into the cache
  2. dsa_indexer_topk         - indexer score over every causal cached key,
                                then the deterministic top-k per query token
  3. sparse_mla_attn          - absorbed MLA over the selected latent rows
Default workload ("decode_32k_mtp"): 64 requests x 32768 cached tokens, two
query tokens per request (one plus one MTP draft), indexer 32 heads x 128
dims bf16, top-k 2048, MLA 64 heads x (512 latent + 64 rope) bf16.  All
inputs are resident in HBM before timing starts.

Timing protocol: before every timed rep a 1 GiB read evicts L2 and the
last-level cache (a read leaves no dirty lines behind); one HIP event pair
brackets the rep only (no event between the calls of a step).  The events
are created with hipEventDisableSystemFence, so recording one does not write
back the caches.  `ms_per_step` is the median over the K reps; p10 and p90
are reported beside it, and each call is timed the same way on its own.

Prints one JSON line.  `value` is query tokens per second of the whole step
(IndexShare stack: amortised microseconds per layer).  `roofline` is for the
dominant call: algorithmic bytes (or flops) / its median flushed duration.
`cpu_baseline` times the plain CPU oracle on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--warm]
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, vendor figure
SIMD_COUNT = 1024              # 256 CUs x 4 SIMDs
METRIC = "decode query-tokens/s (indexer+top-k+sparse MLA) and % HBM roofline, 32K ctx"
WORKLOADS = ["decode_32k_mtp", "fp8_decode_varlen", "indexshare_8layer", "prefill_16k",
             "fp8q_decode_32k_mtp"]


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_32k_mtp", choices=WORKLOADS)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--graph", action="store_true",
                   help="also time the step captured in a HIP graph (replayed, same protocol)")
    p.add_argument("--warm", action="store_true",
                   help="also time K steps and calls back to back without eviction")
    p.add_argument("--pmc-run", action="store_true",
                   help="for rocprofv3 --pmc: one conversion of known size (calibration), "
                        "then K steps back to back; prints nothing else")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 counter_collection.csv files (FETCH_SIZE "
                        "run, WRITE_SIZE run) into a traffic summary (JSON on stdout); "
                        "no GPU needed")
    p.add_argument("--stats-summary", nargs=3, metavar=("STATS_CSV", "TITLE", "COMMAND"),
                   help="turn a rocprofv3 --stats kernel_stats.csv into the text table "
                        "kept under profiles/; no GPU needed")
    p.add_argument("--mfma-counter", default="SQ_INSTS_VALU_MFMA_MOPS_BF16",
                   help="the flop counter --mfma-summary reads (_BF16 or _F8)")
    p.add_argument("--mfma-summary", metavar="CSV",
                   help="turn a rocprofv3 counter_collection.csv of SQ_INSTS_VALU_MFMA_"
                        "MOPS_BF16 and MfmaUtil into a per-kernel summary (JSON on "
                        "stdout); no GPU needed")
    return p.parse_args()


# ------------------------------------------------------------------ work
def _rows(b, topk):
    """Selected rows per query token: min(topk, pos + 1)."""
    n = 0
    for bi in range(b.num_reqs):
        for i in range(b.q_lens[bi]):
            n += min(topk, b.seq_lens[bi] - b.q_lens[bi] + i + 1)
    return n


def _pairs(b):
    """Causal (query token, key) pairs."""
    n = 0
    for bi in range(b.num_reqs):
        L, ql = b.seq_lens[bi], b.q_lens[bi]
        n += sum(L - ql + i + 1 for i in range(ql))
    return n


def indexer_bytes(b, cfg):
    """Algorithmic bytes of one indexer + top-k call: every causal key read
    once per request (+ its fp32 scale for an FP8 cache), queries and head
    weights read once, indices written once, block tables read once."""
    key_b = cfg.d_idx * (1 if cfg.idx_cache_dtype == "fp8" else 2)
    if cfg.idx_cache_dtype == "fp8":
        key_b += 4
    keys = sum(b.seq_lens) * key_b
    q = b.num_q_tokens * cfg.n_idx_heads * cfg.d_idx * 2   # bf16 queries read once
    w = b.num_q_tokens * cfg.n_idx_heads * 4
    out = b.num_q_tokens * cfg.topk * 4
    bt = b.num_reqs * b.max_blocks * 4
    return keys + q + w + out + bt


def indexer_flops(b, cfg):
    return 2 * _pairs(b) * cfg.n_idx_heads * cfg.d_idx


def mla_bytes(b, cfg):
    """One latent row per (query token, selected index), queries, indices,
    bf16 output and fp32 lse."""
    N, H = b.num_q_tokens, cfg.n_heads
    return (_rows(b, cfg.topk) * cfg.d_latent * 2 + N * H * cfg.d_latent * 2
            + N * cfg.topk * 4 + N * H * cfg.kv_lora_rank * 2 + N * H * 4)


def mla_flops(b, cfg):
    return 2 * _rows(b, cfg.topk) * cfg.n_heads * (cfg.d_latent + cfg.kv_lora_rank)


def prologue_bytes(b, cfg):
    """Weights read once (bf16), activations read once, q / k / w written
    once, cos / sin read once, the new keys' cache rows written once."""
    N, H, D = b.num_q_tokens, cfg.n_idx_heads, cfg.d_idx
    weights = (H * D * cfg.q_lora_rank + D * cfg.hidden_dim + H * cfg.hidden_dim) * 2
    acts = N * (cfg.hidden_dim + cfg.q_lora_rank) * 2 + N * cfg.idx_rope_dim * 4
    outs = N * H * D * 2 + N * D * 2 + N * H * 4 + N * (D * 2 + 8)
    return weights + acts + outs


def cache_write_bytes(b, cfg):
    per = cfg.d_idx * (1 if cfg.idx_cache_dtype == "fp8" else 2)
    return b.num_q_tokens * (cfg.d_idx * 2 + per + 8)


# ------------------------------------------------------------------ traffic
CSRC = os.path.join(ROOT, "sparse_attention_topk_amd", "csrc")
# the dominant call's kernels, and the sources they are built from
INDEXER_KERNELS = ("k_score_dma", "k_score_prefill", "k_topk", "k_topk_reg")
INDEXER_SRCS = ("common.h", "indexer_score.hip", "topk.hip")
CALIB_ELEMS = 1 << 28          # calibration: fp32 -> bf16 conversion of 1 GiB
CALIB_READ, CALIB_WRITE = CALIB_ELEMS * 4, CALIB_ELEMS * 2


def source_sha(names=INDEXER_SRCS):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", "traffic_indexer_%s.json" % workload)


def _read_counters(path, counter):
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"]), int(r["Grid_Size"])))
    return rows


def _short(name):
    return name.split("::")[-1].split("(")[0]


def pmc_summary(fetch_csv, write_csv):
    """HBM bytes per launch of every library kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads for
    a conversion kernel of known size (1 GiB read, 512 MiB written) run in the
    same process."""

    def read(path, counter):
        per, calib = {}, []
        for name, v, grid in _read_counters(path, counter):
            v *= 1024.0
            if "copy" in name and "dsa::" not in name and grid >= CALIB_ELEMS // 8:
                calib.append((v, name[:120]))
            if "dsa::" in name:
                per.setdefault(_short(name), []).append(v)
        return per, calib

    fetch, fcal = read(fetch_csv, "FETCH_SIZE")
    write, wcal = read(write_csv, "WRITE_SIZE")
    if len(fcal) != 1 or len(wcal) != 1:
        raise SystemExit("expected one calibration dispatch per run, found %d / %d"
                         % (len(fcal), len(wcal)))
    f_scale = CALIB_READ / fcal[0][0]
    w_scale = CALIB_WRITE / wcal[0][0]
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        fb = sum(fetch.get(k, [0])) / max(1, len(fetch.get(k, []))) * f_scale
        wb = sum(write.get(k, [0])) / max(1, len(write.get(k, []))) * w_scale
        kernels[k] = {"fetch_bytes": fb, "write_bytes": wb,
                      "launches": len(fetch.get(k, []))}
    call = sum(v["fetch_bytes"] + v["write_bytes"] for k, v in kernels.items()
               if k.split("<")[0] in INDEXER_KERNELS)
    return {"commands": [
                "rocprofv3 --pmc FETCH_SIZE -d prof/pmc -o fetch --output-format csv"
                " -- python3 -u bench.py --pmc-run --steps 3 --warmup 1 --no-cpu",
                "rocprofv3 --pmc WRITE_SIZE -d prof/pmc -o write --output-format csv"
                " -- python3 -u bench.py --pmc-run --steps 3 --warmup 1 --no-cpu",
                "python3 bench.py --pmc-summary prof/pmc/fetch_counter_collection.csv"
                " prof/pmc/write_counter_collection.csv"],
            "note": "per-launch means; FETCH_SIZE and WRITE_SIZE scaled by the ratio of "
                    "known to counted bytes of the calibration kernel",
            "source_sha256": source_sha(), "sources": list(INDEXER_SRCS),
            "calibration": {"kernel": fcal[0][1], "read_bytes": CALIB_READ,
                            "write_bytes": CALIB_WRITE,
                            "fetch_counted_bytes": fcal[0][0],
                            "write_counted_bytes": wcal[0][0],
                            "fetch_scale": f_scale, "write_scale": w_scale},
            "indexer_call_traffic_bytes": call, "kernels": kernels}


def mfma_summary(csv_path, counter="SQ_INSTS_VALU_MFMA_MOPS_BF16"):
    """Per library kernel: matrix-core flops per dispatch of one data type
    (the counter, SQ_INSTS_VALU_MFMA_MOPS_BF16 or _F8, counts units of 512
    flops) and the fraction of cycles the matrix cores were busy while it
    ran (MfmaUtil = summed SQ_VALU_MFMA_BUSY_CYCLES over every SIMD /
    (GRBM_GUI_ACTIVE x SIMDs))."""
    mops, util = {}, {}
    for name, v, _ in _read_counters(csv_path, counter):
        if "dsa::" in name:
            mops.setdefault(_short(name), []).append(v * 512.0)
    for name, v, _ in _read_counters(csv_path, "MfmaUtil"):
        if "dsa::" in name:
            util.setdefault(_short(name), []).append(v)
    out = {}
    for k in sorted(set(mops) | set(util)):
        m, u = mops.get(k, []), util.get(k, [])
        out[k] = {"mfma_flops_per_dispatch": sum(m) / len(m) if m else None,
                  "mfma_busy_pct": sum(u) / len(u) if u else None,
                  "dispatches": max(len(m), len(u))}
    return out


def stats_summary(stats_csv, title, command):
    """Text table of a rocprofv3 kernel_stats.csv (per-kernel calls and
    durations), headed by what it covers and the command that made it."""
    import csv
    import re

    def short(n):
        n = re.sub(r"\(anonymous namespace\)::", "", n)
        m = re.match(r"(void )?([\w:<>, ]+?)\(", n)
        return (m.group(2) if m else n)[:60]

    out = ["# %s" % title, "", "command (from the repository root on an MI355X, "
           "TMPDIR=/tmp):", "", "    " + command, "",
           "%-60s %6s %12s %12s %12s %6s" % ("kernel", "calls", "avg_us", "min_us",
                                             "max_us", "pct")]
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            out.append("%-60s %6s %12.2f %12.2f %12.2f %6.2f" % (
                short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def load_traffic(workload):
    """Measured HBM bytes per dsa_indexer_topk call, or None when no summary
    exists or a kernel source changed since the counters were taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_sha():
        return None
    return rec["indexer_call_traffic_bytes"]


# ------------------------------------------------------------------ timing
class HipTimer:
    """HIP events on the launch stream, created with hipEventDisableSystemFence
    (0x20000000): recording one then needs no system-scope cache write-back,
    which would otherwise idle the GPU for microseconds around each call.
    Elapsed times are read after a device-wide synchronisation.  The HIP
    runtime is the one torch already loaded."""
    FLAGS = 0x20000000

    def __init__(self, stream_handle):
        with open("/proc/self/maps") as f:
            path = next(l.split()[-1] for l in f if "libamdhip64" in l)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [P, P]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        lib.hipEventDestroy.argtypes = [P]
        self.lib, self.stream = lib, P(stream_handle)

    def _event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(ev), self.FLAGS)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        return ev

    def _record(self, ev):
        rc = self.lib.hipEventRecord(ev, self.stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def _elapsed(self, e0, e1):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def reps(self, fn, k, before=None):
        """k reps of fn(), each bracketed by its own event pair; before()
        runs ahead of each rep, outside the pair.  Returns ms per rep."""
        import torch
        evs = [(self._event(), self._event()) for _ in range(k)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            if before is not None:
                before()
            self._record(e0)
            fn()
            self._record(e1)
        torch.cuda.synchronize()
        out = [self._elapsed(e0, e1) for e0, e1 in evs]
        for e0, e1 in evs:
            self.lib.hipEventDestroy(e0)
            self.lib.hipEventDestroy(e1)
        return out

    def back_to_back(self, fn, k):
        """Mean ms of fn() run k times back to back under one event pair."""
        return self.reps(lambda: [fn() for _ in range(k)], 1)[0] / k


def stats(v):
    s = sorted(v)

    def pct(p):
        x = (len(s) - 1) * p / 100.0
        lo, hi = int(math.floor(x)), int(math.ceil(x))
        return s[lo] + (s[hi] - s[lo]) * (x - lo)

    return {"median_ms": pct(50), "p10_ms": pct(10), "p90_ms": pct(90),
            "mean_ms": sum(s) / len(s), "reps": len(s)}


def make_flush(torch, dev):
    junk = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB
    return lambda: junk.sum()


def hbm_roofline(name, nbytes, ms, traffic=None, kernels=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "kernel": name, "achieved": gbs, "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
         "bytes_per_launch": nbytes, "median_ms": ms}
    if kernels:
        r["traffic_kernels"] = list(kernels)
    return r


def mfma_roofline(name, flops, ms):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": name, "achieved": tf, "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS, "traffic": None,
            "flops_per_launch": flops, "median_ms": ms}


def threads_used():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


# ------------------------------------------------------------------ cpu leg
def cpu_baseline(cfg, b, lay, seconds, units):
    """Time the oracle (as it stands) on units of the same workload, cycling
    over them until about `seconds` of compute have run.  A unit is
    (request, None): every query token of the request, or (request, i): its
    query i alone (keys 0..its position).  Host copies and, for an FP8 cache,
    the quantisation of the cache as it stands before the step are set-up,
    not timed.  Returns (query-tokens/s, tokens, passes, units used, seconds,
    mean context of the units used)."""
    import numpy as np
    import torch
    from oracle import fp8_indexer as F8, indexer as OI, mla as OM
    bs = b.block_size
    fp8 = cfg.idx_cache_dtype == "fp8"

    def host_inputs(unit):
        bi, i = unit
        L, ql = b.seq_lens[bi], b.q_lens[bi]
        t0 = int(b.cu_q_host[bi])
        if i is not None:                       # one query: keys 0 .. its position
            L, t0, ql = L - ql + i + 1, t0 + i, 1
        slots = torch.as_tensor(OI.physical_slots(b.block_table_host[bi], bs, L),
                                device=lay.k_src.device)
        kbits = lay.k_src[slots].cpu().view(torch.int16).numpy().view(np.uint16)
        if fp8:
            k32 = (kbits.astype(np.uint32) << np.uint32(16)).view(np.float32)
            quant = F8.rotate_quantize if cfg.idx_q_fp8 else OI.fp8_quantize_rows
            keys, scale, kd = (*quant(k32), OI.FP8)
        else:
            keys, scale, kd = kbits, None, OI.BF16
        kv = lay.kv_cache[slots].cpu().float().numpy()
        q = lay.q_idx[t0:t0 + ql].float().cpu().numpy().astype(np.float64)
        w = lay.w[t0:t0 + ql].cpu().numpy().astype(np.float64)
        qm = lay.q_mla[t0:t0 + ql].float().cpu().numpy().astype(np.float64)
        ident = np.arange((L + bs - 1) // bs, dtype=np.int64)[None, :]
        return L, ql, keys, scale, kd, kv, q, w, qm, ident

    pool, spent, tokens, runs = [], 0.0, 0, 0
    while spent < seconds:
        if len(pool) < min(16, len(units)):
            pool.append(host_inputs(units[len(pool)]))
        L, ql, keys, scale, kd, kv, q, w, qm, ident = pool[runs % len(pool)]
        start = time.perf_counter()
        if cfg.idx_q_fp8:
            qc, qs = F8.rotate_quantize(q.astype(np.float32))
            idx = F8.indexer_topk([L], [0, ql], ident, bs, qc, qs, w, keys, scale, cfg.topk)
        else:
            idx = OI.indexer_topk([L], [0, ql], ident, bs, q, w, keys, scale, kd, cfg.topk)
        OM.sparse_mla([L], [0, ql], ident, bs, qm, lambda s: kv[s], idx,
                      cfg.kv_lora_rank, cfg.softmax_scale)
        spent += time.perf_counter() - start
        tokens += ql
        runs += 1
    mean_ctx = sum(p[0] for p in pool) / len(pool)
    return tokens / spent, tokens, runs, len(pool), spent, mean_ctx


def cpu_leg(cfg, b, lay, seconds):
    """The cpu_baseline object for the single-layer workloads."""
    import numpy as np
    if cfg.name == "prefill_16k":
        # 16 query rows spread evenly over the sequence (mean context about half)
        units = [(0, int(i)) for i in np.linspace(0, b.num_q_tokens - 1, 16)]
        what = "16 query rows spread evenly over the 16384-token sequence"
        batch_ctx = sum(b.seq_lens[0] - b.q_lens[0] + i + 1 for i in range(b.q_lens[0])) \
            / b.num_q_tokens
    else:
        units = [(bi, None) for bi in range(b.num_reqs)]
        what = "the first requests of %d" % b.num_reqs
        batch_ctx = sum(b.seq_lens) / b.num_reqs
    v, tok, runs, npool, spent, ctx = cpu_baseline(cfg, b, lay, seconds, units)
    sample = ("%d passes over %d units (%s; mean context %.0f against %.0f for the "
              "whole workload), %d query tokens of %s: float64 NumPy oracle%s, indexer + "
              "top-k + sparse MLA, compute only, %.1f s"
              % (runs, npool, what, ctx, batch_ctx, tok, cfg.name,
                 " (FP8 cache quantised by the oracle beforehand)"
                 if cfg.idx_cache_dtype == "fp8" else "", spent))
    return {"value": v, "unit": "query-tokens/s", "cores": threads_used(),
            "kind": "oracle", "sample": sample}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.pmc_summary:
        print(json.dumps(pmc_summary(*args.pmc_summary), indent=1))
        return
    if args.stats_summary:
        print(stats_summary(*args.stats_summary))
        return
    if args.mfma_summary:
        print(json.dumps(mfma_summary(args.mfma_summary, args.mfma_counter), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(requests shard independently across GPUs; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_topk_amd as dsa
    from synth import get_config, make_batch, make_layer
    dsa.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    cfg = get_config(args.workload)
    log("generating %s inputs" % cfg.name)
    b = make_batch(cfg, dev)
    bb = dsa.Batch.from_synth(b)
    N = b.num_q_tokens
    stream = torch.cuda.current_stream()

    if args.pmc_run:
        src = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
        dst = torch.empty(CALIB_ELEMS, dtype=torch.bfloat16, device=dev)
        dst.copy_(src)                     # the calibration kernel
        torch.cuda.synchronize()
        del src, dst
    if cfg.name == "indexshare_8layer":
        return bench_indexshare(args, cfg, b, bb, dsa, torch, stream)

    lay = make_layer(cfg, b, dev)
    # the cache before this step: every slot populated through the cache write
    if cfg.idx_q_fp8:
        k_cache = torch.empty((b.num_slots, cfg.d_idx), dtype=torch.uint8, device=dev)
        k_scale = torch.empty((b.num_slots,), dtype=torch.float32, device=dev)
        all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=dev)
        dsa.dsa_rotate_quantize(lay.k_src, k_cache, k_scale, row_slots=all_slots)
        q_codes = torch.empty(lay.q_idx.shape, dtype=torch.uint8, device=dev)
        q_scale = torch.empty(lay.q_idx.shape[:2], dtype=torch.float32, device=dev)
    elif cfg.idx_cache_dtype == "fp8":
        k_cache = torch.empty((b.num_slots, cfg.d_idx), dtype=torch.uint8, device=dev)
        k_scale = torch.empty((b.num_slots,), dtype=torch.float32, device=dev)
        all_slots = torch.arange(b.num_slots, dtype=torch.int64, device=dev)
        dsa.dsa_indexer_cache_write(lay.k_src, all_slots, k_cache, k_scale)
    else:
        k_cache = lay.k_src
        k_scale = None
    k_new = lay.k_src[b.slot_mapping_t].contiguous()       # this step's keys
    topk_idx = torch.empty((N, cfg.topk), dtype=torch.int32, device=dev)
    out = torch.empty((N, cfg.n_heads, cfg.kv_lora_rank), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((N, cfg.n_heads), dtype=torch.float32, device=dev)
    ws_bytes = max(dsa.dsa_indexer_topk_workspace_size(bb, cfg.topk),
                   dsa.sparse_mla_attn_workspace_size(bb, cfg.n_heads, cfg.kv_lora_rank,
                                                      cfg.rope_dim, cfg.topk, dsa.DSA_BF16))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def cache_write():
        if cfg.idx_q_fp8:        # rotated, quantised keys into the FP8 cache
            dsa.dsa_rotate_quantize(k_new, k_cache, k_scale, row_slots=b.slot_mapping_t)
        else:
            dsa.dsa_indexer_cache_write(k_new, b.slot_mapping_t, k_cache, k_scale)

    def indexer():
        if cfg.idx_q_fp8:        # rotated, quantised queries, then the e4m3 score
            dsa.dsa_rotate_quantize(lay.q_idx, q_codes, q_scale)
            dsa.dsa_indexer_topk_fp8q(bb, q_codes, q_scale, lay.w, k_cache, k_scale,
                                      cfg.topk, topk_idx=topk_idx, workspace=ws)
        else:
            dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, k_cache, k_scale, cfg.topk,
                                 topk_idx=topk_idx, workspace=ws)

    def attention():
        dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, topk_idx, cfg.kv_lora_rank,
                            cfg.softmax_scale, out=out, lse=lse, workspace=ws)

    def step():
        cache_write()
        indexer()
        attention()

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.pmc_run:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return

    timer = HipTimer(stream.cuda_stream)
    flush = make_flush(torch, dev)
    with_prologue = cfg.name in ("decode_32k_mtp", "fp8q_decode_32k_mtp")
    log("timing %d steps, caches evicted before each" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st = stats(timer.reps(step, args.steps, flush))
    wall = time.perf_counter() - t0
    log("timing each call %d times, caches evicted before each" % args.steps)
    calls = {"cache_write": stats(timer.reps(cache_write, args.steps, flush)),
             "indexer_topk": stats(timer.reps(indexer, args.steps, flush)),
             "sparse_mla_attn": stats(timer.reps(attention, args.steps, flush))}
    if with_prologue:
        # the indexer prologue of this step's new tokens (projections, k_norm,
        # RoPE, the keys' cache write); reported beside the step, not in it
        from synth import make_prologue
        pi = make_prologue(cfg, b, dev)
        pq = torch.empty((N, cfg.n_idx_heads, cfg.d_idx), dtype=torch.bfloat16, device=dev)
        pw = torch.empty((N, cfg.n_idx_heads), dtype=torch.float32, device=dev)
        pws = torch.empty(max(256, dsa.load_library().dsa_indexer_prologue_workspace_size(
            N, ctypes.byref(dsa._binding._CPrologueDims(
                cfg.hidden_dim, cfg.q_lora_rank, cfg.n_idx_heads, cfg.d_idx,
                cfg.idx_rope_dim, cfg.norm_eps)))), dtype=torch.uint8, device=dev)

        def prologue():
            dsa.dsa_indexer_prologue(pi.hidden, pi.qa_normed, pi.cos, pi.sin, pi.wq_b, pi.wk,
                                     pi.weights_proj, pi.k_norm_weight, cfg.n_idx_heads,
                                     cfg.idx_rope_dim, cfg.norm_eps,
                                     slot_mapping=b.slot_mapping_t, k_cache=k_cache,
                                     k_scale=k_scale, q_out=pq, w_out=pw, workspace=pws,
                                     want_k=False)
        prologue()
        torch.cuda.synchronize()
        pst = stats(timer.reps(prologue, args.steps, flush))
        pb = prologue_bytes(b, cfg)
        pst.update(bytes=pb, note="not part of the step: q / k / w projections, k_norm, "
                                  "RoPE and the new keys' cache write (hidden %d, q_lora_rank "
                                  "%d); bytes: weights, activations and outputs once"
                                  % (cfg.hidden_dim, cfg.q_lora_rank))
        pst["frac_hbm"] = pb / (pst["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        calls["indexer_prologue"] = pst
    ms_step = st["median_ms"]
    ib, mb, cb = indexer_bytes(b, cfg), mla_bytes(b, cfg), cache_write_bytes(b, cfg)
    ifl, mfl = indexer_flops(b, cfg), mla_flops(b, cfg)
    calls["cache_write"]["bytes"] = cb
    calls["indexer_topk"].update(bytes=ib, flops=ifl)
    calls["sparse_mla_attn"].update(bytes=mb, flops=mfl)
    prefill = cfg.name == "prefill_16k"
    for k, fl in (("indexer_topk", ifl), ("sparse_mla_attn", mfl)):
        c = calls[k]
        if prefill and k == "sparse_mla_attn":
            # the gathered latent rows (every token's top-k) come from a
            # cache-resident context: not HBM traffic, so no HBM fraction
            c["note"] = "bytes: latent rows gathered (cache-resident context, not HBM traffic)"
        else:
            c["GB/s"] = c["bytes"] / (c["median_ms"] * 1e-3) / 1e9
            c["frac_hbm"] = c["GB/s"] / HBM_PEAK_GBS
        c["TFLOP/s"] = fl / (c["median_ms"] * 1e-3) / 1e12
        c["frac_mfma_bf16"] = c["TFLOP/s"] / BF16_PEAK_TFLOPS
    ix_ms, ml_ms = calls["indexer_topk"]["median_ms"], calls["sparse_mla_attn"]["median_ms"]
    if prefill:
        # latent rows and keys stay cache-resident: matrix-core bound
        roof = (mfma_roofline("sparse_mla_attn (k_mla_prefill: one workgroup per token)", mfl, ml_ms) if ml_ms >= ix_ms
                else mfma_roofline("dsa_indexer_topk", ifl, ix_ms))
    elif cfg.idx_q_fp8:
        roof = hbm_roofline("dsa_rotate_quantize (queries) + dsa_indexer_topk_fp8q", ib, ix_ms)
    else:
        roof = hbm_roofline("dsa_indexer_topk (score + top-k)", ib, ix_ms,
                            load_traffic(cfg.name), INDEXER_KERNELS)
    res = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if cfg.idx_cache_dtype != "fp8" else
                  "fp8 indexer (e4m3 q and k), bf16 MLA" if cfg.idx_q_fp8 else
                  "bf16+fp8-cache"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "requests": b.num_reqs,
                   "max_context": b.max_seq_len, "total_context": int(sum(b.seq_lens)),
                   "query_tokens": N, "indexer_heads": cfg.n_idx_heads,
                   "d_idx": cfg.d_idx, "topk": cfg.topk, "mla_heads": cfg.n_heads,
                   "kv_lora_rank": cfg.kv_lora_rank, "rope_dim": cfg.rope_dim,
                   "idx_cache": cfg.idx_cache_dtype, "parallelism": "single-gpu"},
        "roofline": roof,
        "timing": {"protocol": "median over K reps; before each rep a 1 GiB read "
                               "evicts L2 and the last-level cache; one HIP event pair "
                               "(no system fence) per rep, none between the calls of "
                               "a step", "step": st, "timed_loop_wall_s": wall},
        "calls": calls,
        "step_frac_hbm": (None if prefill else
                          (ib + mb + cb) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS),
        "cpu_baseline": None,
    }
    if args.graph:
        # the same step captured once into a HIP graph (the library allocates
        # nothing and enqueues no memset, so the capture holds only its
        # kernels), replayed under the same protocol
        log("graph pass: %d replays, caches evicted before each" % args.steps)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gst = stats(timer.reps(graph.replay, args.steps, flush))
        gst["value"] = N / (gst["median_ms"] * 1e-3)
        res["graph_step"] = gst
        del graph
    if args.warm:
        log("warm pass: %d steps and calls back to back" % args.steps)
        res["warm_back_to_back_ms"] = {
            "step": timer.back_to_back(step, args.steps),
            "indexer_topk": timer.back_to_back(indexer, args.steps),
            "sparse_mla_attn": timer.back_to_back(attention, args.steps)}
    if not args.no_cpu:
        log("cpu oracle baseline (~%.0f s)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_leg(cfg, b, lay, args.cpu_seconds)
    print(json.dumps(res))


def bench_indexshare(args, cfg, b, bb, dsa, torch, stream):
    """IndexShare stack: 8 layers, amortised time per layer."""
    import numpy as np
    from synth import make_layer
    dev = "cuda"
    types = cfg.indexer_types
    codes = [dsa.DSA_LAYER_FULL if t == "full" else dsa.DSA_LAYER_SHARED for t in types]
    # each layer's top-k source, from the library (the layers that own an
    # indexer are those that are their own source)
    src = dsa.dsa_resolve_indexer_sources(codes, len(types))
    N = b.num_q_tokens
    layers, lays = [], []
    for i in range(len(types)):
        full = src[i] == i
        lay = make_layer(cfg, b, dev, layer=i, with_indexer=full)
        lays.append(lay)
        layers.append(dsa.Layer(
            q_mla=lay.q_mla, kv_cache=lay.kv_cache,
            out=torch.empty((N, cfg.n_heads, cfg.kv_lora_rank), dtype=torch.bfloat16, device=dev),
            lse=torch.empty((N, cfg.n_heads), dtype=torch.float32, device=dev),
            q_idx=lay.q_idx if full else None, w=lay.w if full else None,
            k_cache=lay.k_src if full else None,
            topk_idx=torch.empty((N, cfg.topk), dtype=torch.int32, device=dev) if full else None))
    dims = dsa.StackDims(cfg.n_idx_heads, cfg.d_idx, dsa.DSA_BF16, dsa.DSA_BF16, cfg.topk,
                         cfg.n_heads, cfg.kv_lora_rank, cfg.rope_dim, dsa.DSA_BF16,
                         cfg.softmax_scale)
    ws = torch.empty(max(256, dsa.indexshare_forward_workspace_size(bb, dims)),
                     dtype=torch.uint8, device=dev)

    def stack():
        dsa.indexshare_forward(bb, codes, layers, dims, workspace=ws)

    def one_mla():      # layer 1 (shared) attends with layer 0's indices
        L1 = layers[1]
        dsa.sparse_mla_attn(bb, L1.q_mla, L1.kv_cache, layers[0].topk_idx, cfg.kv_lora_rank,
                            cfg.softmax_scale, out=L1.out, lse=L1.lse, workspace=ws)

    def one_indexer():
        L0 = layers[0]
        dsa.dsa_indexer_topk(bb, L0.q_idx, L0.w, L0.k_cache, None, cfg.topk,
                             topk_idx=L0.topk_idx, workspace=ws)

    for _ in range(args.warmup):
        stack()
    torch.cuda.synchronize()
    if args.pmc_run:
        for _ in range(args.steps):
            stack()
        torch.cuda.synchronize()
        return
    timer = HipTimer(stream.cuda_stream)
    flush = make_flush(torch, dev)
    log("timing %d stacks, caches evicted before each" % args.steps)
    st = stats(timer.reps(stack, args.steps, flush))
    ml = stats(timer.reps(one_mla, args.steps, flush))
    ix = stats(timer.reps(one_indexer, args.steps, flush))
    n_layers = len(types)
    n_full = sum(1 for i in range(n_layers) if src[i] == i)
    ib, mb = indexer_bytes(b, cfg), mla_bytes(b, cfg)
    by = n_full * ib + n_layers * mb
    ms = st["median_ms"]
    res = {
        "metric": "IndexShare stack amortised us/layer (8 layers, 2 indexer runs)",
        "value": ms * 1e3 / n_layers, "unit": "us/layer", "higher_is_better": False,
        "ms_per_step": ms, "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": types, "requests": b.num_reqs,
                   "max_context": b.max_seq_len, "query_tokens": N, "topk": cfg.topk},
        "roofline": hbm_roofline("sparse_mla_attn (k_mla_ws: four key splits per token), one layer", mb,
                                 ml["median_ms"]),
        "timing": {"protocol": "median over K reps, caches evicted before each rep, one "
                               "HIP event pair (no system fence) per rep", "stack": st},
        "calls": {"sparse_mla_attn": dict(ml, bytes=mb), "indexer_topk": dict(ix, bytes=ib)},
        "stack_bytes": by,
        "stack_frac_hbm": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        log("cpu oracle baseline (~%.0f s)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_indexshare(cfg, b, lays, src, args.cpu_seconds)
    print(json.dumps(res))


def cpu_indexshare(cfg, b, lays, src, seconds):
    """The oracle over the whole stack (two indexer runs, eight attentions)
    for whole requests, cycling over a sample until about `seconds` have run;
    scaled to the batch's query tokens and reported per layer like the
    GPU figure."""
    import numpy as np
    import torch
    from oracle import indexer as OI, indexshare as OX, mla as OM
    bs = b.block_size
    n_layers = len(lays)

    def host(bi):
        L = b.seq_lens[bi]
        slots = torch.as_tensor(OI.physical_slots(b.block_table_host[bi], bs, L),
                                device=lays[0].kv_cache.device)
        t0 = int(b.cu_q_host[bi])
        per = []
        for i, lay in enumerate(lays):
            d = {"kv": lay.kv_cache[slots].cpu().float().numpy(),
                 "qm": lay.q_mla[t0:t0 + 1].float().cpu().numpy().astype(np.float64)}
            if src[i] == i:
                d["keys"] = lay.k_src[slots].cpu().view(torch.int16).numpy().view(np.uint16)
                d["q"] = lay.q_idx[t0:t0 + 1].float().cpu().numpy().astype(np.float64)
                d["w"] = lay.w[t0:t0 + 1].cpu().numpy().astype(np.float64)
            per.append(d)
        return L, per

    ident_of = lambda L: np.arange((L + bs - 1) // bs, dtype=np.int64)[None, :]
    pool, spent, tokens, runs = [], 0.0, 0, 0
    while spent < seconds:
        if len(pool) < min(8, b.num_reqs):
            pool.append(host(len(pool)))
        L, per = pool[runs % len(pool)]
        ident = ident_of(L)
        start = time.perf_counter()
        OX.forward(cfg.indexer_types, per,
                   lambda d: OI.indexer_topk([L], [0, 1], ident, bs, d["q"], d["w"],
                                             d["keys"], None, OI.BF16, cfg.topk),
                   lambda d, tk: OM.sparse_mla([L], [0, 1], ident, bs, d["qm"],
                                               lambda s: d["kv"][s], tk, cfg.kv_lora_rank,
                                               cfg.softmax_scale))
        spent += time.perf_counter() - start
        tokens += 1
        runs += 1
    us_layer = spent / tokens * b.num_q_tokens / n_layers * 1e6
    return {"value": us_layer, "unit": "us/layer", "cores": threads_used(), "kind": "oracle",
            "sample": "%d stack passes of one query token each (cycling over %d requests "
                      "of %d), float64 NumPy oracle through all %d layers, compute only, "
                      "%.1f s; scaled to the batch's %d query tokens and divided by the "
                      "layer count" % (runs, len(pool), b.num_reqs, n_layers, spent,
                                       b.num_q_tokens)}


if __name__ == "__main__":
    main()
