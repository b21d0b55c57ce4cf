"""The fp64 oracle run over many sequences on the host's cores.

TEST INFRASTRUCTURE ONLY: used by the GPU tests (every output row of a
full-size workload compared with the oracle) and by the benchmark's CPU
baseline (the oracle timed on all host cores).  Nothing in the product path
imports it.

Sequences of one workload are independent ("Nano-vLLM part 1", section 5.2:
prefill packs separate prompts by cumulative lengths; a decode batch is one
query per sequence), so the oracle of a batch is the oracle of each sequence on
its own.  Each worker process regenerates a sequence's inputs from the seeded
workload on a compact block pool (``Workload.subset``, the same logical tokens)
and runs ``oracle.fp64`` on it, one sequence at a time, with one BLAS thread.
Workers are spawned, not forked, so a parent that already drives the GPU hands
no device state to them.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import time
from typing import Optional, Sequence

import numpy as np

ATOL = 1e-2
RTOL = 1e-2
# A GPU machine grants one GPU's process 16 host cores, whatever the affinity mask shows.
MAX_WORKERS = 16


def host_cores() -> int:
    """Cores the pool uses: the affinity mask, capped at the per-GPU share."""
    return max(1, min(len(os.sched_getaffinity(0)), MAX_WORKERS))


def _init_worker():
    # one thread per worker for every library: BLAS, OpenMP and torch's own pool
    # (the input generator runs torch CPU ops), so the pool uses one core per process
    import torch
    torch.set_num_threads(1)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is installed here
        pass


def _ready():
    import torch
    return os.getpid(), torch.get_num_threads()


def _sequence_ref(w, s: int) -> np.ndarray:
    """fp64 oracle rows of sequence s (its store, then its attention)."""
    from oracle import fp64
    sub = w.subset([s])
    h = sub.host_inputs()
    kc, vc = fp64.store_kvcache(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"], h["slot_mapping"])
    if sub.kind == "decode":
        return fp64.paged_decode(h["q"], kc, vc, h["block_tables"], h["context_lens"],
                                 sub.block_size, sub.scale)
    return fp64.paged_prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["cu_seqlens_k"],
                              h["block_tables"], sub.block_size, sub.scale, sub.causal)


def _compare_task(w, seqs: Sequence[int], got_bits: Sequence[np.ndarray]):
    """Compare GPU rows (bf16 bits) of each sequence with the oracle's.

    Returns (rows checked, elements failing |gpu - ref| <= ATOL + RTOL |ref|,
    max abs error, max rel error, first failing sequence or -1).
    """
    from oracle import fp64
    rows = bad = 0
    ea = er = 0.0
    first_bad = -1
    for s, bits in zip(seqs, got_bits):
        ref = _sequence_ref(w, int(s))
        got = fp64.bf16_to_f64(bits).reshape(ref.shape)
        err = np.abs(got - ref)
        fail = ~(err <= ATOL + RTOL * np.abs(ref))  # NaN fails too
        nb = int(fail.sum())
        if nb and first_bad < 0:
            first_bad = int(s)
        bad += nb
        rows += ref.shape[0]
        if err.size:  # a NaN output counts as an infinite error
            err = np.where(np.isnan(err), np.inf, err)
            ea = max(ea, float(err.max()))
            er = max(er, float((err / np.maximum(np.abs(ref), 1e-30)).max()))
    return rows, bad, ea, er, first_bad


def _timed_task(w, seqs: Sequence[int], budget_s: float):
    """Run the oracle on seqs in order until budget_s of oracle time is spent
    (at least one sequence); input generation is not timed.  Returns (pid,
    oracle seconds, sequences done)."""
    from oracle import fp64
    done, t_work = [], 0.0
    for s in seqs:
        sub = w.subset([int(s)])
        h = sub.host_inputs()
        t0 = time.perf_counter()
        kc, vc = fp64.store_kvcache(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"],
                                    h["slot_mapping"])
        if sub.kind == "decode":
            fp64.paged_decode(h["q"], kc, vc, h["block_tables"], h["context_lens"], sub.block_size,
                              sub.scale)
        else:
            fp64.paged_prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["cu_seqlens_k"],
                               h["block_tables"], sub.block_size, sub.scale, sub.causal)
        t_work += time.perf_counter() - t0
        done.append(int(s))
        if t_work >= budget_s:
            break
    return os.getpid(), t_work, done


class OraclePool:
    """A pool of spawned worker processes running the oracle per sequence."""

    def __init__(self, workers: Optional[int] = None, log=None, timeout_s: float = 900.0):
        self.workers = workers or host_cores()
        self.log = log or (lambda msg: None)
        self.timeout_s = timeout_s
        self._ex = cf.ProcessPoolExecutor(max_workers=self.workers,
                                          mp_context=mp.get_context("spawn"),
                                          initializer=_init_worker)
        # start every worker now (the executor would otherwise start them one per
        # submitted task) and check that each came up with one thread
        t0 = time.perf_counter()
        futs = [self._ex.submit(_ready) for _ in range(self.workers)]
        ready = [f.result(timeout=self.timeout_s) for f in futs]
        self.log(f"oracle pool: {self.workers} workers up in {time.perf_counter() - t0:.1f} s, "
                 f"threads per worker {sorted({t for _, t in ready})}")

    def close(self):
        self._ex.shutdown(wait=True, cancel_futures=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def compare(self, w, seqs: Sequence[int], got_rows: Sequence[np.ndarray]):
        """Every row of the given sequences against the oracle.

        ``got_rows[i]`` holds the GPU output rows of ``seqs[i]`` as bf16 bits
        (uint16, [rows, Hq, d]).  Returns (rows, failing elements, max abs err,
        max rel err, first failing sequence or -1).
        """
        order = sorted(range(len(seqs)), key=lambda i: -int(w.lk[seqs[i]]) * max(1, int(w.lq[seqs[i]])))
        chunks = [order[k::self.workers * 2] for k in range(self.workers * 2)]  # cost-balanced
        futs = [self._ex.submit(_compare_task, w, [seqs[i] for i in c], [got_rows[i] for i in c])
                for c in chunks if c]
        rows = bad = 0
        ea = er = 0.0
        first_bad = -1
        t0 = time.perf_counter()
        for k, f in enumerate(cf.as_completed(futs, timeout=self.timeout_s)):
            r, b, a, e, fb = f.result()
            if (k + 1) % max(1, len(futs) // 4) == 0 or k + 1 == len(futs):
                self.log(f"oracle pool: {k + 1} of {len(futs)} chunks compared "
                         f"({time.perf_counter() - t0:.1f} s)")
            rows += r
            bad += b
            ea, er = max(ea, a), max(er, e)
            if fb >= 0 and (first_bad < 0 or fb < first_bad):
                first_bad = fb
        return rows, bad, ea, er, first_bad

    def timed(self, w, seqs: Sequence[int], budget_s: float):
        """Oracle throughput on the host's cores over a bounded sample.

        ``seqs`` is dealt round-robin to one task per worker; each task stops
        once it has spent ``budget_s`` seconds in the oracle.  Returns
        (sequences done, oracle seconds of the busiest worker process,
        total oracle seconds over all workers, worker processes used).  The
        workers run side by side, so the batch's oracle wall time is the
        busiest process's oracle time.
        """
        shares = [list(seqs[k::self.workers]) for k in range(self.workers)]
        futs = [self._ex.submit(_timed_task, w, sh, budget_s) for sh in shares if sh]
        per_pid, done, total = {}, [], 0.0
        for f in cf.as_completed(futs, timeout=self.timeout_s):
            pid, t, d = f.result()
            per_pid[pid] = per_pid.get(pid, 0.0) + t
            total += t
            done += d
        return done, max(per_pid.values()), total, len(per_pid)
