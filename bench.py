"""Benchmark of the paged KV-cache data plane on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch: the store of the step's
new tokens into the paged cache, then decode attention (decode workloads) or
varlen prefill attention (prefill workloads).  Inputs are seeded synthetic
tensors already resident in HBM.  Several identical copies of the inputs are
rotated between steps so that a step does not find the previous step's K/V in
L2 or the Infinity Cache.

Prints one JSON line.  Its headline is the long-context decode (batch 512,
contexts of 4k-32k tokens, 38.7 GB of K/V per step: the largest workload):
whole-step throughput (algorithmic HBM bytes per second) over K steps between
two HIP events, a roofline object for the attention call (its average launch
duration from K back-to-back launches between two HIP events on the launch
stream), the p10/p50/p90 of single steps, and the fp64 oracle timed on the
host's cores.  `sub` holds the same record for the other four workloads
(batch-256 decode, varlen and prefix-cached prefill in FLOP/s, the batch-4
edge decode), and `ceilings` what a plain copy and a library GEMM reach on
the same GPU.  With --workload NAME only that workload is timed.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode HBM GB/s (% peak) + decode tok/s; prefill TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


# ---- algorithmic work ------------------------------------------------------------------
def store_bytes(w) -> int:
    """Read k and v rows, write them into the cache, read the slot index."""
    row = w.num_kv_heads * w.head_dim * 2
    return int(w.num_new_tokens * (4 * row + 4))


def decode_bytes(w) -> int:
    """Each live K and V row of one kv head read once, plus Q, O, tables, lengths."""
    kv = int(w.lk.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * 2
    tables = sum(-(-int(n) // w.block_size) for n in w.lk) * 4 + 4 * w.num_seqs
    return kv + qo + tables


def prefill_flops(w) -> int:
    """4 * d flops per visible (query, key) pair per query head."""
    pairs = 0
    for lq, lk in zip(w.lq.tolist(), w.lk.tolist()):
        off = lk - lq
        pairs += lq * off + lq * (lq + 1) // 2 if w.causal else lq * lk
    return int(4 * w.head_dim * w.num_q_heads * pairs)


def prefill_bytes(w) -> int:
    qo = 2 * int(w.lq.sum()) * w.num_q_heads * w.head_dim * 2
    kv = int(w.lk.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    return qo + kv


# Source files whose change invalidates the counters of each call's kernels.
CALL_SOURCES = {
    "paged_decode_attention": ("paged_decode.hip",),
    "varlen_prefill_attention": ("varlen_prefill.hip",),
    "store_kvcache": ("store_kvcache.hip",),
    "topk_sample": ("sampling.hip",),
}
SHARED_SOURCES = ("common.h", "kernels.h")


def source_code_text(text: str) -> str:
    """C++ source without comments and blank lines (a comment edit keeps the hash)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_sources_sha(call: str, read=None) -> str:
    """Hash of the code (comments left out) of the sources that define one call's
    kernels; `read(name)` returns a source's text (default: the working tree)."""
    csrc = os.path.join(ROOT, "paged_kv_cache_419_amd", "csrc")
    if read is None:
        def read(name):
            with open(os.path.join(csrc, name), encoding="utf-8") as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in sorted(CALL_SOURCES[call] + SHARED_SOURCES):
        h.update(f.encode() + source_code_text(read(f)).encode())
    return h.hexdigest()[:16]


# Kernels that make up one call of each boundary entry point (rocprofv3 names).
CALL_KERNELS = {
    "paged_decode_attention": ("paged_decode_kernel", "paged_decode_combine_kernel"),
    "varlen_prefill_attention": ("varlen_prefill_kernel", "prefill_plan_kernel"),
    "store_kvcache": ("store_kvcache_kernel",),
    "topk_sample": ("topk_sample_kernel",),
}
COPY_PROBE_BYTES = 1 << 30  # plain device-to-device copy that calibrates the counters
COPY_KERNEL = "copyBuffer"


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def measured_traffic(workload: str, call: str):
    """HBM bytes per call from committed rocprofv3 counter runs, if still current."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get("calls", {}).get(call, {})
    if rec.get("kernel_sources_sha") != kernel_sources_sha(call):
        return None
    return rec.get("hbm_bytes_per_call")


def copy_probe(torch, dev):
    """The 1 GiB device copy that calibrates FETCH_SIZE and WRITE_SIZE (three dispatches)."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _counter_values(run_dir: str, counter: str):
    """{kernel name: [(dispatch id, value), ...]} for `counter` in a rocprofv3 csv run."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (name, did), v in per.items():
        by_kernel.setdefault(name, []).append((did, v))
    return by_kernel


def _copy_probe_kib(table) -> float:
    """Counter value of the calibration copy: the last three copy dispatches."""
    copies = sorted((did, v) for n, dv in table.items() if COPY_KERNEL in n for did, v in dv)
    if len(copies) < 3:
        raise SystemExit("no copy probe in the counter run (run bench.py with --copy-probe)")
    last = [v for _, v in copies[-3:]]
    if max(last) > 1.05 * min(last):
        raise SystemExit(f"inconsistent copy probe readings {last}")
    return sum(last) / 3.0


def summarize_counters(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """Per-call HBM traffic from a FETCH_SIZE run and a WRITE_SIZE run.

    Both counters read in KiB per dispatch; each is scaled by what it reads for
    the 1 GiB device copy that the profiled run ends with (the largest copy
    dispatch), so the result is in true bytes.  Writes profiles/traffic_<w>.json.
    """
    fetch = _counter_values(fetch_dir, "FETCH_SIZE")
    write = _counter_values(write_dir, "WRITE_SIZE")
    fetch_scale = COPY_PROBE_BYTES / (_copy_probe_kib(fetch) * 1024.0)
    write_scale = COPY_PROBE_BYTES / (_copy_probe_kib(write) * 1024.0)

    def mean(dv):
        return sum(v for _, v in dv) / len(dv)

    calls = {}
    for call, kernels in CALL_KERNELS.items():
        f = [(n, mean(dv)) for n, dv in fetch.items() if any(k in n for k in kernels)]
        w = [(n, mean(dv)) for n, dv in write.items() if any(k in n for k in kernels)]
        if not f:
            continue
        rb = sum(v for _, v in f) * 1024.0 * fetch_scale
        wb = sum(v for _, v in w) * 1024.0 * write_scale
        calls[call] = {"fetch_kib_per_call": sum(v for _, v in f),
                       "write_kib_per_call": sum(v for _, v in w),
                       "read_bytes_per_call": rb, "write_bytes_per_call": wb,
                       "hbm_bytes_per_call": rb + wb,
                       "kernels": sorted({k for n, _ in f for k in kernels if k in n}),
                       "kernel_sources_sha": kernel_sources_sha(call)}
    rec = {"workload": workload, "copy_probe_bytes": COPY_PROBE_BYTES,
           "fetch_scale": fetch_scale, "write_scale": write_scale, "calls": calls}
    with open(traffic_path(workload), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


# ---- CPU baseline: the fp64 oracle on the host's cores ---------------------------------
def _oracle_units(sub) -> float:
    """The metric's unit of work of a subset: decode bytes (store + attention) or flops."""
    return decode_bytes(sub) + store_bytes(sub) if sub.kind == "decode" else prefill_flops(sub)


def cpu_baseline(w, pool, budget_s: float):
    """The oracle as it stands, run per sequence over a process pool on the host's cores.

    A seeded random order of the workload's sequences is dealt to one task per
    worker process (one BLAS thread each); a task stops after ``budget_s``
    seconds of oracle time.  The batch's oracle wall time is the busiest
    process's oracle time (the processes run side by side); input generation
    is not timed.
    """
    order = np.random.Generator(np.random.PCG64(17)).permutation(w.num_seqs).tolist()
    done, busiest, total, procs = pool.timed(w, order, budget_s)
    units = _oracle_units(w.subset(done))
    if w.kind == "decode":
        value, unit, scale = units / busiest / 1e9, "GB/s", 1e9
    else:
        value, unit, scale = units / busiest / 1e12, "TFLOP/s", 1e12
    return {"value": value, "unit": unit, "cores": procs, "kind": "oracle",
            "per_core_value": units / total / scale,
            "sample": f"{len(done)} of {w.num_seqs} sequences (store + attention, fp64 NumPy), "
                      f"{procs} worker processes with one thread each, {total:.1f} s of oracle "
                      f"time in all, {busiest:.2f} s in the busiest process; input generation "
                      f"untimed"}


def cpu_baseline_one_core(w, budget_s: float):
    """The same oracle on one thread of this process (the small edge workload)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    done, t_work = [], 0.0
    for s in range(w.num_seqs):
        sub = w.subset([s])
        h = sub.host_inputs()
        t0 = time.perf_counter()
        kc, vc = oracle.store_kvcache(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"],
                                      h["slot_mapping"])
        oracle.paged_decode(h["q"], kc, vc, h["block_tables"], h["context_lens"], sub.block_size,
                            sub.scale)
        t_work += time.perf_counter() - t0
        done.append(s)
        if t_work >= budget_s:
            break
    if limiter is not None:
        limiter.unregister()
    units = _oracle_units(w.subset(done))
    return {"value": units / t_work / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} of {w.num_seqs} sequences, one thread, {t_work:.3f} s"}


# ---- sampling (the adjacent next-token step) ----------------------------------------------
SAMPLE_WORKLOAD = "sample_b256"


def sample_bytes(logits: np.ndarray, top_k: int) -> int:
    """Every logit read once, the noise of the candidates, one token id written per row."""
    rows, vocab = logits.shape
    return rows * (vocab * 4 + top_k * 4 + 4)


def run_sampling(args, torch, pkv, dev):
    from workload.sample import SAMPLE_ROWS, SAMPLE_TEMPERATURE, SAMPLE_TOP_K, SAMPLE_VOCAB, sample_inputs
    logits, gumbel = sample_inputs(SAMPLE_ROWS, SAMPLE_VOCAB, seed=4196)
    # 4 x 311 MB: between two uses of one copy the other three copies' 466 MB of logits
    # are read, more than the 256 MB Infinity Cache holds (with 2 copies, 155 MB in
    # between, a call ran ~3 % faster: some rows were still cached)
    reps = args.replicas or 4
    lg = [torch.from_numpy(logits).to(dev) for _ in range(reps)]
    gg = [torch.from_numpy(gumbel).to(dev) for _ in range(reps)]
    tok = [torch.empty(SAMPLE_ROWS, dtype=torch.int32, device=dev) for _ in range(reps)]
    for i in range(args.warmup):
        pkv.topk_sample(tok[i % reps], lg[i % reps], gg[i % reps], SAMPLE_TOP_K, SAMPLE_TEMPERATURE)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):  # the step is this one kernel, launched back to back
        pkv.topk_sample(tok[i % reps], lg[i % reps], gg[i % reps], SAMPLE_TOP_K, SAMPLE_TEMPERATURE)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    call_ms = ms
    import oracle.sampling as OS
    want = OS.topk_sample(logits, gumbel, SAMPLE_TOP_K, SAMPLE_TEMPERATURE)
    assert np.array_equal(tok[0].cpu().numpy(), want), "sampled tokens differ from the oracle"
    nbytes = sample_bytes(logits, SAMPLE_TOP_K)
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    rec = {
        "metric": "next-token sampling HBM GB/s (% peak)", "value": nbytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": SAMPLE_WORKLOAD, "rows": SAMPLE_ROWS, "vocab": SAMPLE_VOCAB,
                   "top_k": SAMPLE_TOP_K, "temperature": SAMPLE_TEMPERATURE,
                   "input_copies_rotated": reps, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(SAMPLE_WORKLOAD, "topk_sample"), "kernel": "topk_sample",
                     "kernel_ms": call_ms},
        "rows_per_s": SAMPLE_ROWS / (ms * 1e-3),
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        n = 0
        while n < SAMPLE_ROWS and time.perf_counter() - t0 < args.cpu_budget:
            OS.topk_sample(logits[n:n + 1], gumbel[n:n + 1], SAMPLE_TOP_K, SAMPLE_TEMPERATURE)
            n += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": n * (nbytes / SAMPLE_ROWS) / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} of {SAMPLE_ROWS} rows (NumPy, one thread), {dt:.1f} s"}
    if args.copy_probe:
        copy_probe(torch, dev)
    print(json.dumps(rec), flush=True)


# ---- decode steps replayed from captured graphs, against eager launches --------------------
GRAPH_SWEEP = "graph_sweep"
GRAPH_BATCHES = (1, 4, 16, 64, 256, 512)


def run_graph_sweep(args, torch, pkv, dev):
    """The decode step (the new tokens' store, then decode attention) at several batch
    sizes with the batch-256 decode's shape (Hq 16, Hkv 8, d 128, contexts U[100,1024]),
    four ways: two eager launches, the fused kernel eager, and each of those captured
    once per input copy as a HIP graph and replayed.  Each figure is the average ms per
    step over K back-to-back steps between two HIP events."""
    import workload as W
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_harness as H
    out = {}
    for b in GRAPH_BATCHES:
        seed = 4300 + b
        rng = np.random.Generator(np.random.PCG64(seed))
        ctx = rng.integers(100, 1024, size=b, endpoint=True)
        w = W.decode(ctx, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                     id_mode="choice", max_blocks_per_seq=4, seed=seed, rng=rng, name=f"decode_b{b}")
        reps = max(1, min(4, math.ceil(2.0e9 / unique_step_bytes(w))))
        copies = [w.materialize(dev) for _ in range(reps)]
        outs = [torch.full_like(c["q"], float("nan")) for c in copies]
        ws = torch.empty(max(16, pkv.decode_workspace_bytes(b, 16, 8, 128, w.max_context_len, 0)),
                         dtype=torch.uint8, device=dev)

        def two(i):
            c = copies[i % reps]
            pkv.store_kvcache(c["k_new"], c["v_new"], c["k_cache"], c["v_cache"], c["slot_mapping"])
            pkv.paged_decode_attention(outs[i % reps], c["q"], c["k_cache"], c["v_cache"],
                                       c["block_tables"], c["context_lens"], w.block_size,
                                       w.max_context_len, w.scale, 0, ws)

        def fused(i):
            c = copies[i % reps]
            pkv.store_and_decode(outs[i % reps], c["q"], c["k_new"], c["v_new"], c["k_cache"],
                                 c["v_cache"], c["slot_mapping"], c["block_tables"], c["context_lens"],
                                 w.block_size, w.max_context_len, w.scale, 0, ws)

        def capture(body):
            gs = []
            for i in range(reps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    body(i)
                gs.append(g)
            return gs

        def timed(body):
            for i in range(args.warmup):
                body(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(args.steps):
                body(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        rec = {"eager_ms": timed(two), "fused_ms": timed(fused)}
        g2 = capture(two)
        rec["graph_ms"] = timed(lambda i: g2[i % reps].replay())
        gf = capture(fused)
        rec["graph_fused_ms"] = timed(lambda i: gf[i % reps].replay())
        H.check_against_oracle(w, outs[0], [int(np.argmax(w.lk))])
        rec["input_copies_rotated"] = reps
        out[str(b)] = rec
        del copies, outs, ws, g2, gf
        torch.cuda.empty_cache()
    best = min(min(r["graph_ms"], r["graph_fused_ms"]) for r in out.values())
    rec = {"metric": "decode step ms (store + decode), eager vs graph replay", "value": best,
           "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": best, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": GRAPH_SWEEP, "batches": list(GRAPH_BATCHES), "num_q_heads": 16,
                      "num_kv_heads": 8, "head_dim": 128, "context": "U[100,1024]"},
           "sweep": out}
    print(json.dumps(rec), flush=True)


def summarize_graph_trace(trace_dir: str, per: int = 25) -> str:
    """Step time, kernel busy time and idle time per batch and launch kind, from a
    rocprofv3 kernel trace of `--workload graph_sweep` run with K + W = `per` steps."""
    import csv
    import glob
    import statistics as st
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += [r for r in csv.DictReader(open(f)) if "pkv" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    kinds = ["eager", "fused", "graph", "graph_fused"]
    dec = [i for i, r in enumerate(rows) if "paged_decode_kernel" in r["Kernel_Name"]]
    if len(dec) != per * len(kinds) * len(GRAPH_BATCHES):
        raise SystemExit(f"expected {per * len(kinds) * len(GRAPH_BATCHES)} decode dispatches, found {len(dec)}")
    us = lambda a, b: (int(b) - int(a)) / 1e3
    out = []
    for bi, b in enumerate(GRAPH_BATCHES):
        for ki, kind in enumerate(kinds):
            seg = dec[(bi * 4 + ki) * per:(bi * 4 + ki + 1) * per][5:]  # after the warm-up steps
            starts = [i - 1 if "store_kvcache" in rows[i - 1]["Kernel_Name"] else i for i in seg]
            busy, span = [], []
            for a, z in zip(starts, starts[1:]):
                busy.append(sum(us(r["Start_Timestamp"], r["End_Timestamp"]) for r in rows[a:z]))
                span.append(us(rows[a]["Start_Timestamp"], rows[z]["Start_Timestamp"]))
            dd = [us(rows[i]["Start_Timestamp"], rows[i]["End_Timestamp"]) for i in seg]
            out.append(f"B={b:4d} {kind:12s} step {st.mean(span):7.1f} us  kernels busy {st.mean(busy):7.1f} us  "
                       f"idle {st.mean(span) - st.mean(busy):6.1f} us  decode kernel {st.median(dd):6.1f} us  "
                       f"kernels/step {starts[1] - starts[0]}")
    return "\n".join(out)


# ---- GPU run ----------------------------------------------------------------------------
def unique_step_bytes(w) -> int:
    """Bytes one step touches, each distinct byte once: Q, O, the K/V of every distinct
    key position (a shared prefix once, not once per sequence) and the store's rows.
    Sizes the number of input copies rotated between steps."""
    kv_tokens = w.prefix_len + int((w.hist + w.lq).sum())
    kv = kv_tokens * w.num_kv_heads * w.head_dim * 2 * 2
    qo = 2 * w.num_q_rows * w.num_q_heads * w.head_dim * 2
    return kv + qo + store_bytes(w)


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def measure_ceilings(torch, dev, reps: int = 10) -> dict:
    """What plain library kernels reach on this machine, beside the published peaks: a
    2 GiB device-to-device copy (bytes read + written per second) and a bf16 GEMM of
    8192^3 through torch (rocBLAS and hipBLASLt, the faster kept), each the median of
    `reps` timed calls."""
    out = {}
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)

    def med_ms(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    ms = med_ms(lambda: dst.copy_(src))
    out["copy_gbs"] = 2 * n / (ms * 1e-3) / 1e9
    out["copy_frac_of_hbm_peak"] = out["copy_gbs"] / HBM_PEAK_GBS
    # both BLAS back ends torch can select on ROCm; the faster is the ceiling
    backends = {}
    prev = torch.backends.cuda.preferred_blas_library()
    for name, lib in (("rocblas", "cublas"), ("hipblaslt", "cublaslt")):
        try:
            torch.backends.cuda.preferred_blas_library(lib)
            ms = med_ms(lambda: torch.mm(a, b, out=c))
            backends[name] = 2 * 8192 ** 3 / (ms * 1e-3) / 1e12
        except RuntimeError as e:  # a back end this build lacks
            backends[name] = f"unavailable: {e}"
    torch.backends.cuda.preferred_blas_library(prev)
    timed = {k: v for k, v in backends.items() if isinstance(v, float)}
    best = max(timed, key=timed.get)
    out["gemm_bf16_tflops"] = timed[best]
    out["gemm_backend"] = best
    out["gemm_bf16_tflops_by_backend"] = backends
    out["gemm_frac_of_mfma_peak"] = out["gemm_bf16_tflops"] / MFMA_BF16_PEAK_TFLOPS
    out["how"] = ("median of 10 event-timed calls: torch copy_ of 2 GiB (read + write bytes), "
                  "torch.mm bf16 8192x8192x8192 under rocBLAS and hipBLASLt, the faster kept")
    del src, dst, a, b, c
    torch.cuda.empty_cache()
    return out


def measure(name, args, torch, pkv, dev, pool, cpu_budget):
    """Time one workload: K whole steps (store + attention) back to back, each call's
    own average launch duration, the spread of single steps, an oracle check of what
    was timed, and the oracle on the host's cores."""
    import workload as W
    w = W.make(name)
    decode = w.kind == "decode"
    reps = args.replicas or max(1, min(4, math.ceil(2.0e9 / unique_step_bytes(w))))
    copies = [w.materialize(dev) for _ in range(reps)]
    outs = [torch.full_like(c["q"], float("nan")) for c in copies]
    split = args.split_tokens
    ws_bytes = (pkv.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                           w.max_context_len, split) if decode else
                pkv.prefill_workspace_bytes(w.num_seqs, int(w.lq.sum()), w.num_q_heads,
                                            w.num_kv_heads))
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    max_q = int(w.lq.max())
    max_k = int(w.lk.max())

    def store(c):
        pkv.store_kvcache(c["k_new"], c["v_new"], c["k_cache"], c["v_cache"], c["slot_mapping"])

    def attend(c, out):
        if decode:
            pkv.paged_decode_attention(out, c["q"], c["k_cache"], c["v_cache"], c["block_tables"],
                                       c["context_lens"], w.block_size, w.max_context_len, w.scale,
                                       split, workspace)
        else:
            pkv.varlen_prefill_attention(out, c["q"], c["k_cache"], c["v_cache"], c["cu_seqlens_q"],
                                         c["cu_seqlens_k"], c["block_tables"], max_q, max_k,
                                         w.block_size, w.scale, w.causal, workspace)

    def step(i):
        store(copies[i % reps])
        attend(copies[i % reps], outs[i % reps])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(body) -> float:
        """Average ms per iteration of `body(i)` over the K steps, launched back to back."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            body(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def spread(body):
        """Per-iteration ms from an event between consecutive iterations (a separate pass)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(args.steps):
            body(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]

    # the timed region: K whole steps (store + attention); then the attention call's
    # own launch duration from K back-to-back launches of that call alone
    ms_step = timed(step)
    attn_ms = timed(lambda i: attend(copies[i % reps], outs[i % reps]))
    steps_ms = spread(step)
    attn_each = spread(lambda i: attend(copies[i % reps], outs[i % reps]))

    if decode:
        step_units = decode_bytes(w) + store_bytes(w)
        value, unit = step_units / (ms_step * 1e-3) / 1e9, "GB/s"
        achieved = decode_bytes(w) / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        kernel = "paged_decode_attention"
        roof["algorithmic_bytes"] = decode_bytes(w)
    else:
        value, unit = prefill_flops(w) / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        achieved = prefill_flops(w) / (attn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
        kernel = "varlen_prefill_attention"
        roof["algorithmic_flops"] = prefill_flops(w)
    roof["traffic"] = measured_traffic(name, kernel)
    roof["kernel"] = kernel
    roof["kernel_ms"] = attn_ms

    # correctness of what was timed: the longest sequence against the oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_harness as H
    probe = [int(np.argmax(w.lk if decode else w.lq))]
    H.check_against_oracle(w, outs[0], probe)

    rec = {
        "value": value, "unit": unit, "ms_per_step": ms_step,
        "step_ms_p10": _pct(steps_ms, 10), "step_ms_p50": _pct(steps_ms, 50),
        "step_ms_p90": _pct(steps_ms, 90),
        "attention_ms": attn_ms, "attention_ms_p10": _pct(attn_each, 10),
        "attention_ms_p90": _pct(attn_each, 90),
        "config": {
            "workload": name, "kind": w.kind, "sequences": w.num_seqs,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "num_blocks": w.num_blocks,
            "context_tokens": int(w.lk.sum()), "new_tokens": w.num_new_tokens,
            "split_tokens": (split or pkv.decode_split_tokens(w.num_seqs, w.num_q_heads,
                                                              w.num_kv_heads, w.head_dim,
                                                              w.max_context_len)) if decode else None,
            "input_copies_rotated": reps, "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    if decode:
        rec["decode_tok_per_s"] = w.num_seqs / (ms_step * 1e-3)
        rec["hbm_frac"] = value / HBM_PEAK_GBS
        if int(w.lq.min()) == 1 and w.pad_tokens == 0 and not args.copy_probe:
            # the same step as one fused kernel (store the new tokens and attend)
            def fused(i):
                c, out = copies[i % reps], outs[i % reps]
                pkv.store_and_decode(out, c["q"], c["k_new"], c["v_new"], c["k_cache"], c["v_cache"],
                                     c["slot_mapping"], c["block_tables"], c["context_lens"],
                                     w.block_size, w.max_context_len, w.scale, split, workspace)
            for i in range(args.warmup):
                fused(i)
            rec["fused_ms_per_step"] = timed(fused)
            H.check_against_oracle(w, outs[0], probe)
            rec["fused_decode_tok_per_s"] = w.num_seqs / (rec["fused_ms_per_step"] * 1e-3)
        if args.graph:
            # the same step (store + decode) captured once per input copy and replayed
            graphs = []
            for i, c in enumerate(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    store(c)
                    attend(c, outs[i])
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % reps].replay()
            rec["graph_ms_per_step"] = timed(lambda i: graphs[i % reps].replay())
            rec["graph_decode_tok_per_s"] = w.num_seqs / (rec["graph_ms_per_step"] * 1e-3)
    else:
        # the store of this step's tokens (36k tokens here: long enough to time on its own)
        store_ms = timed(lambda i: store(copies[i % reps]))
        rec["store_ms"] = store_ms
        rec["store_gbs"] = store_bytes(w) / (store_ms * 1e-3) / 1e9
        rec["mfma_frac"] = value / MFMA_BF16_PEAK_TFLOPS
    del copies, outs, workspace
    torch.cuda.empty_cache()
    if pool is not None:
        rec["cpu_baseline"] = cpu_baseline(w, pool, cpu_budget)
        if name == "decode_edge_b4":
            rec["cpu_baseline_one_core"] = cpu_baseline_one_core(w, cpu_budget)
    return rec


HEADLINE = "decode_long_b512"  # the largest single-GPU workload (38.7 GB of K/V per step)
# the other configurations, then one GPU's share of the headline under 8-way tensor parallelism
SUB_WORKLOADS = ("decode_b256", "prefill_varlen_s64", "prefill_prefix_s128", "decode_edge_b4",
                 "decode_long_b512_shard8")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help=f"time this workload alone (default: {HEADLINE} as the headline, with "
                         "the other data-plane workloads as sub-records)")
    ap.add_argument("--replicas", type=int, default=0, help="input copies rotated (0 = auto)")
    ap.add_argument("--split-tokens", type=int, default=0, help="decode split (0 = library's choice)")
    ap.add_argument("--cpu-budget", type=float, default=1.5,
                    help="seconds of oracle time per host worker process (headline workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="decode: also time the step replayed from a captured HIP graph")
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with a 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into profiles/traffic_<workload>.json")
    ap.add_argument("--graph-trace", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 kernel trace of --workload graph_sweep "
                         "(run with --steps 20 --warmup 5)")
    args = ap.parse_args()

    if args.counters:
        print(json.dumps(summarize_counters(args.workload, *args.counters)), flush=True)
        return
    if args.graph_trace:
        print(summarize_graph_trace(args.graph_trace, args.steps + args.warmup), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the data plane has no cross-GPU step in this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_419_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pkv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == SAMPLE_WORKLOAD:
        run_sampling(args, torch, pkv, dev)
        return
    if args.workload == GRAPH_SWEEP:
        run_graph_sweep(args, torch, pkv, dev)
        return
    single = args.workload is not None
    headline = args.workload or HEADLINE
    pool = None
    if not args.no_cpu_baseline:
        from oracle.pool import OraclePool
        pool = OraclePool()
    try:
        head = measure(headline, args, torch, pkv, dev, pool, args.cpu_budget)
        subs = {}
        if not single:
            for name in SUB_WORKLOADS:
                subs[name] = measure(name, args, torch, pkv, dev, pool, args.cpu_budget / 2)
    finally:
        if pool is not None:
            pool.close()
    rec = {
        "metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
    }
    rec.update(head)
    if subs:
        rec["sub"] = subs
    if not args.no_ceilings and not args.copy_probe:
        rec["ceilings"] = measure_ceilings(torch, dev)
    if args.copy_probe:
        copy_probe(torch, dev)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
