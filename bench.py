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

Prints one JSON line.  `value` is query tokens per second of the whole step.
`roofline` is for the dominant call (the indexer: score + top-k kernels),
algorithmic bytes / mean duration from HIP events on the launch stream.
`cpu_baseline` times the plain CPU oracle on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
METRIC = "decode query-tokens/s (indexer+top-k+sparse MLA) and % HBM roofline, 32K ctx"


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_32k_mtp",
                   choices=["decode_32k_mtp", "fp8_decode_varlen",
                            "indexshare_8layer", "prefill_16k"])
    p.add_argument("--no-cpu", action="store_true",
                   help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--pmc-run", action="store_true",
                   help="for rocprofv3 --pmc: one conversion of known size (calibration), "
                        "then the timed steps; prints nothing else")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 counter_collection.csv files "
                        "(FETCH_SIZE run, WRITE_SIZE run) into a traffic "
                        "summary (JSON on stdout); no GPU needed")
    return p.parse_args()


# ------------------------------------------------------------------ bytes
def indexer_bytes(b, cfg):
    """Algorithmic bytes of one indexer + top-k call: every causal key read
    once per request (+ its fp32 scale for an FP8 cache), queries and head
    weights read once, indices written once, block tables read once."""
    key_b = cfg.d_idx * (1 if cfg.idx_cache_dtype == "fp8" else 2)
    if cfg.idx_cache_dtype == "fp8":
        key_b += 4
    keys = sum(b.seq_lens) * key_b
    q = b.num_q_tokens * cfg.n_idx_heads * cfg.d_idx * 2
    w = b.num_q_tokens * cfg.n_idx_heads * 4
    out = b.num_q_tokens * cfg.topk * 4
    bt = b.num_reqs * b.max_blocks * 4
    return keys + q + w + out + bt


def mla_bytes(b, cfg):
    """One 1152-byte latent row per (query token, selected index), queries,
    indices, bf16 output and fp32 lse."""
    rows = 0
    for bi in range(b.num_reqs):
        for i in range(b.q_lens[bi]):
            pos = b.seq_lens[bi] - b.q_lens[bi] + i
            rows += min(cfg.topk, pos + 1)
    N, H = b.num_q_tokens, cfg.n_heads
    return (rows * cfg.d_latent * 2 + N * H * cfg.d_latent * 2 + N * cfg.topk * 4
            + N * H * cfg.kv_lora_rank * 2 + N * H * 4)


def cache_write_bytes(b, cfg):
    per = cfg.d_idx * (1 if cfg.idx_cache_dtype == "fp8" else 2)
    return b.num_q_tokens * (cfg.d_idx * 2 + per + 8)


# ------------------------------------------------------------------ traffic
CSRC = os.path.join(ROOT, "sparse_attention_topk_amd", "csrc")
# the dominant call's kernels, and the sources they are built from
INDEXER_KERNELS = ("k_score_dma", "k_topk")
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


def pmc_summary(fetch_csv, write_csv):
    """HBM bytes per launch of every library kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads for
    a conversion kernel of known size (1 GiB read, 512 MiB written) run in the
    same process."""
    import csv

    def read(path, counter):
        per, calib = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v, name = float(r["Counter_Value"]) * 1024.0, r["Kernel_Name"]
            if ("copy" in name and "dsa::" not in name
                    and int(r["Grid_Size"]) >= CALIB_ELEMS // 8):
                calib.append((v, name[:120]))
            if "dsa::" in name:
                key = name.split("::")[-1].split("(")[0]
                per.setdefault(key, []).append(v)
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
                "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc -o fetch --output-format csv"
                " -- python3 -u bench.py --pmc-run --steps 3 --warmup 1 --no-cpu",
                "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc -o write --output-format csv"
                " -- python3 -u bench.py --pmc-run --steps 3 --warmup 1 --no-cpu",
                "python3 bench.py --pmc-summary gpurun_out/pmc/fetch_counter_collection.csv"
                " gpurun_out/pmc/write_counter_collection.csv"],
            "note": "per-launch means; FETCH_SIZE and WRITE_SIZE scaled by the ratio of "
                    "known to counted bytes of the calibration kernel",
            "source_sha256": source_sha(), "sources": list(INDEXER_SRCS),
            "calibration": {"kernel": fcal[0][1], "read_bytes": CALIB_READ,
                            "write_bytes": CALIB_WRITE,
                            "fetch_counted_bytes": fcal[0][0],
                            "write_counted_bytes": wcal[0][0],
                            "fetch_scale": f_scale, "write_scale": w_scale},
            "indexer_call_traffic_bytes": call, "kernels": kernels}


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


# ------------------------------------------------------------------ cpu leg
def cpu_baseline(cfg, b, lay, k_cache, seconds):
    """Time the oracle (as it stands) on whole query tokens of the same
    workload until about `seconds` of compute have run."""
    import numpy as np
    import torch
    from oracle import indexer as OI, mla as OM
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    bs = b.block_size

    def host_inputs(bi):
        """Host copies of one request's inputs (not timed)."""
        L, ql = b.seq_lens[bi], b.q_lens[bi]
        slots = torch.as_tensor(OI.physical_slots(b.block_table_host[bi], bs, L),
                                device=k_cache.device)
        keys = k_cache[slots].cpu().view(torch.int16).numpy().view(np.uint16)
        kv = lay.kv_cache[slots].cpu().float().numpy()
        t0 = int(b.cu_q_host[bi])
        q = lay.q_idx[t0:t0 + ql].float().cpu().numpy().astype(np.float64)
        w = lay.w[t0:t0 + ql].cpu().numpy().astype(np.float64)
        qm = lay.q_mla[t0:t0 + ql].float().cpu().numpy().astype(np.float64)
        ident = np.arange((L + bs - 1) // bs, dtype=np.int64)[None, :]
        return L, ql, keys, kv, q, w, qm, ident

    # cycle over the first few requests until about `seconds` have run
    pool = [host_inputs(bi) for bi in range(min(b.num_reqs, 16))]
    spent, tokens, runs = 0.0, 0, 0
    while spent < seconds:
        L, ql, keys, kv, q, w, qm, ident = pool[runs % len(pool)]
        start = time.perf_counter()
        idx = OI.indexer_topk([L], [0, ql], ident, bs, q, w, keys, None,
                              OI.BF16, cfg.topk)
        OM.sparse_mla([L], [0, ql], ident, bs, qm, lambda s: kv[s], idx,
                      cfg.kv_lora_rank, cfg.softmax_scale)
        spent += time.perf_counter() - start
        tokens += ql
        runs += 1
    return {"value": tokens / spent, "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d request passes (cycling over %d requests of %d, %d query "
                      "tokens) of %s: float64 NumPy oracle, indexer+top-k+sparse MLA, "
                      "compute only, %.1f s" % (runs, len(pool), b.num_reqs, tokens,
                                                cfg.name, spent)}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.pmc_summary:
        print(json.dumps(pmc_summary(*args.pmc_summary), indent=1))
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

    if cfg.name == "indexshare_8layer":
        return bench_indexshare(args, cfg, b, bb, dsa, torch)
    if args.pmc_run:
        src = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
        dst = torch.empty(CALIB_ELEMS, dtype=torch.bfloat16, device=dev)
        dst.copy_(src)                     # the calibration kernel
        torch.cuda.synchronize()
        del src, dst

    lay = make_layer(cfg, b, dev)
    # the cache before this step: every slot populated through the cache write
    if cfg.idx_cache_dtype == "fp8":
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

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dsa.dsa_indexer_cache_write(k_new, b.slot_mapping_t, k_cache, k_scale)
        if ev is not None:
            ev[1].record(stream)
        dsa.dsa_indexer_topk(bb, lay.q_idx, lay.w, k_cache, k_scale, cfg.topk,
                             topk_idx=topk_idx, workspace=ws)
        if ev is not None:
            ev[2].record(stream)
        dsa.sparse_mla_attn(bb, lay.q_mla, lay.kv_cache, topk_idx, cfg.kv_lora_rank,
                            cfg.softmax_scale, out=out, lse=lse, workspace=ws)
        if ev is not None:
            ev[3].record(stream)

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Per-call durations: the same K steps once more, with events between the
    # calls.  Each event puts a marker into the queue that the GPU drains
    # before the next kernel starts, so this pass runs slower than the one
    # above and is kept apart from it.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(args.steps)]
    log("per-call breakdown over %d steps" % args.steps)
    tb = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    breakdown_ms_step = (time.perf_counter() - tb) * 1e3 / args.steps
    # Per-call durations without markers between calls: the same call K times
    # back to back, one event pair around the run (the kernels of one call
    # follow those of the previous one as they do inside a step).  The
    # dominant kernel's roofline uses this; it agrees with the rocprofv3
    # kernel durations, which a marker between calls inflates by ~3 us.
    def back_to_back(fn, k):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k
    log("back-to-back calls, %d each" % args.steps)
    ix_b2b = back_to_back(lambda: dsa.dsa_indexer_topk(
        bb, lay.q_idx, lay.w, k_cache, k_scale, cfg.topk, topk_idx=topk_idx,
        workspace=ws), args.steps)
    ml_b2b = back_to_back(lambda: dsa.sparse_mla_attn(
        bb, lay.q_mla, lay.kv_cache, topk_idx, cfg.kv_lora_rank, cfg.softmax_scale,
        out=out, lse=lse, workspace=ws), args.steps)
    # Cold caches: before each step, outside its events, a 1 GiB read evicts
    # L2 and the last-level cache (a read leaves no dirty lines behind), as
    # when other layers run between two steps of this one.
    junk = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for _ in range(min(args.steps, 50))]
    log("cold-cache pass over %d steps" % len(cold))
    for ev in cold:
        junk.sum()
        step(ev)
    torch.cuda.synchronize()
    del junk
    cw = [e[0].elapsed_time(e[1]) for e in evs]
    ix = [e[1].elapsed_time(e[2]) for e in evs]
    ml = [e[2].elapsed_time(e[3]) for e in evs]
    mean = lambda v: sum(v) / len(v)
    ms_step = elapsed * 1e3 / args.steps
    ib, mb, cb = indexer_bytes(b, cfg), mla_bytes(b, cfg), cache_write_bytes(b, cfg)
    ix_gbs = ib / (ix_b2b * 1e-3) / 1e9
    ml_gbs = mb / (ml_b2b * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.idx_cache_dtype != "fp8" else "bf16+fp8-cache",
        "data": "synthetic",
        "config": {"workload": cfg.name, "requests": b.num_reqs,
                   "max_context": b.max_seq_len, "total_context": int(sum(b.seq_lens)),
                   "query_tokens": N, "indexer_heads": cfg.n_idx_heads,
                   "d_idx": cfg.d_idx, "topk": cfg.topk, "mla_heads": cfg.n_heads,
                   "kv_lora_rank": cfg.kv_lora_rank, "rope_dim": cfg.rope_dim,
                   "idx_cache": cfg.idx_cache_dtype, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "dsa_indexer_topk (score + top-k)",
                     "achieved": ix_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ix_gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic(cfg.name),
                     "traffic_kernels": list(INDEXER_KERNELS),
                     "bytes_per_launch": ib, "mean_ms": ix_b2b},
        "calls": {
            "cache_write": {"mean_ms": mean(cw), "bytes": cb},
            "indexer_topk": {"mean_ms": ix_b2b, "bytes": ib, "GB/s": ix_gbs,
                             "frac_hbm": ix_gbs / HBM_PEAK_GBS,
                             "mean_ms_with_markers": mean(ix)},
            "sparse_mla_attn": {"mean_ms": ml_b2b, "bytes": mb, "GB/s": ml_gbs,
                                "frac_hbm": ml_gbs / HBM_PEAK_GBS,
                                "mean_ms_with_markers": mean(ml)},
            "step_frac_hbm": (ib + mb + cb) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "note": "mean_ms: the call run back to back, one event pair around the "
                    "run; mean_ms_with_markers: a second pass of the steps with an "
                    "event between calls (each marker idles the GPU ~3 us); neither "
                    "is the pass ms_per_step is taken from",
            "breakdown_pass_ms_per_step": breakdown_ms_step,
        },
        "calls_cold_cache": {
            "note": "per-call means with L2 and the last-level cache evicted (1 GiB "
                    "read) before each step",
            "indexer_topk_ms": mean([e[1].elapsed_time(e[2]) for e in cold]),
            "sparse_mla_attn_ms": mean([e[2].elapsed_time(e[3]) for e in cold]),
            "indexer_frac_hbm": ib / (mean([e[1].elapsed_time(e[2]) for e in cold]) * 1e-3)
                                / 1e9 / HBM_PEAK_GBS,
        },
        "cpu_baseline": None,
    }
    if args.pmc_run:
        return
    if not args.no_cpu and cfg.idx_cache_dtype != "fp8":
        log("cpu oracle baseline (~%.0f s)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(cfg, b, lay, k_cache, args.cpu_seconds)
    print(json.dumps(res))


def bench_indexshare(args, cfg, b, bb, dsa, torch):
    """IndexShare stack: 8 layers, amortised time per layer."""
    from synth import make_layer
    dev = "cuda"
    types = cfg.indexer_types
    src = []
    last = None
    for i, t in enumerate(types):
        last = i if t == "full" else last
        src.append(last)
    N = b.num_q_tokens
    layers = []
    for i in range(len(types)):
        full = src[i] == i
        lay = make_layer(cfg, b, dev, layer=i, with_indexer=full)
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
    codes = [dsa.DSA_LAYER_FULL if t == "full" else dsa.DSA_LAYER_SHARED for t in types]
    ws = torch.empty(max(256, dsa.indexshare_forward_workspace_size(bb, dims)),
                     dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        dsa.indexshare_forward(bb, codes, layers, dims, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dsa.indexshare_forward(bb, codes, layers, dims, workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    n_full = sum(1 for i in range(len(types)) if src[i] == i)
    by = n_full * indexer_bytes(b, cfg) + len(types) * mla_bytes(b, cfg)
    gbs = by / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "IndexShare stack ms and amortised us/layer", "value": ms * 1e3 / len(types),
        "unit": "us/layer", "higher_is_better": False, "ms_per_step": ms,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "config": {"workload": cfg.name, "layers": types, "requests": b.num_reqs,
                   "max_context": b.max_seq_len, "topk": cfg.topk},
        "stack_bytes": by, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
        "data": "synthetic", "dtype": "bf16"}))


if __name__ == "__main__":
    main()
