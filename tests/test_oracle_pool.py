"""The process pool that runs the oracle per sequence (CPU only).

The pool must agree with the oracle called directly: the oracle's own rows,
rounded to bf16, pass the attention tolerance, and a row moved by more than the
tolerance is reported in the sequence it belongs to.
"""
import numpy as np
import torch

import cases
import gpu_harness as H
from oracle.pool import OraclePool


def _bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_pool_matches_direct_oracle_and_catches_a_bad_row():
    with OraclePool(workers=2) as pool:
        for name in ("decode_b256[6]", "prefill_ragged_bs16"):
            w = cases.get(name)
            seqs = list(range(w.num_seqs))
            ref = cases.reference(name)
            bits = _bf16_round(ref)
            rows = [bits[H.rows_for(w, [s])] for s in seqs]
            n, bad, ea, _, first = pool.compare(w, seqs, rows)
            assert n == ref.shape[0] and bad == 0 and first == -1 and ea < 1e-2
            # one element of the last non-empty sequence pushed past the tolerance
            s_bad = max(s for s in seqs if rows[s].size)
            planted = [r.copy() for r in rows]
            planted[s_bad].reshape(-1)[0] = _bf16_round(
                np.array([H.to_f64(torch.from_numpy(rows[s_bad].view(np.int16)).view(torch.bfloat16))
                          .reshape(-1)[0] + 0.5]))[0]
            n, bad, _, _, first = pool.compare(w, seqs, planted)
            assert bad == 1 and first == s_bad


def test_pool_timing_reports_its_sample():
    w = cases.get("decode_b256[6]")
    with OraclePool(workers=2) as pool:
        done, busiest, total, procs = pool.timed(w, list(range(w.num_seqs)), budget_s=0.0)
    # a zero budget still runs one sequence per task
    assert sorted(done) == [0, 1]
    assert 0 < busiest <= total and 1 <= procs <= 2
