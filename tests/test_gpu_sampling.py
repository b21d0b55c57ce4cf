"""Sampling kernel vs the oracle: token ids bit-exact (integer work; every step
that decides them is fp32 on both sides), at small shapes with ties, -inf
entries and every top-k / temperature regime, and at the full bench size."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_419_amd as pkv
from oracle import sampling as S
from workload.sample import (SAMPLE_ROWS, SAMPLE_TEMPERATURE, SAMPLE_TOP_K, SAMPLE_VOCAB,
                             gumbel_noise, sample_inputs)

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(logits, gumbel, k, t):
    lg = torch.from_numpy(logits).cuda()
    gg = None if gumbel is None else torch.from_numpy(gumbel).cuda()
    tok = torch.empty(logits.shape[0], dtype=torch.int32, device="cuda")
    pkv.topk_sample(tok, lg, gg, k, t)
    torch.cuda.synchronize()
    return tok.cpu().numpy()


@pytest.mark.parametrize("vocab", [1, 7, 100, 1000, 5003])
@pytest.mark.parametrize("t", [0.0, 0.3, 1.0, 2.5])
def test_small(vocab, t):
    _note(f"sampling vocab {vocab} T {t}")
    rng = np.random.Generator(np.random.PCG64(vocab * 7 + int(t * 10)))
    rows = 9
    logits = (rng.standard_normal((rows, vocab)) * 2).astype(np.float32)
    logits[1] = np.round(logits[1])                  # many ties
    logits[2, ::3] = -np.inf                         # masked vocabulary entries
    logits[3] = 0.0
    logits[3, ::2] = -0.0                            # signed zeros only
    gumbel = gumbel_noise(rng, (rows, vocab))
    for k in sorted({0, 1, 2, 5, 50, max(vocab - 1, 1), vocab, vocab + 3}):
        got = _run(logits, gumbel if t > 0 else None, k, t)
        want = S.topk_sample(logits, gumbel, k, t)
        assert np.array_equal(got, want), f"k={k}: {got} vs {want}"


def test_full_size():
    _note("sampling full size")
    logits, gumbel = sample_inputs(SAMPLE_ROWS, SAMPLE_VOCAB, seed=4196)
    got = _run(logits, gumbel, SAMPLE_TOP_K, SAMPLE_TEMPERATURE)
    want = S.topk_sample(logits, gumbel, SAMPLE_TOP_K, SAMPLE_TEMPERATURE)
    assert np.array_equal(got, want)
    # every sampled token is among its row's 50 largest logits
    kth = np.sort(logits, axis=1)[:, -SAMPLE_TOP_K]
    assert np.all(logits[np.arange(SAMPLE_ROWS), got] >= kth)


def test_frequencies_follow_softmax():
    _note("sampling frequencies")
    z = np.array([1.2, -0.4, 2.0, 0.3, 2.0, -3.0], np.float32)
    n = 100_000
    g = gumbel_noise(np.random.Generator(np.random.PCG64(3)), (n, z.size))
    got = _run(np.ascontiguousarray(np.broadcast_to(z, (n, z.size))), g, 4, 0.7)
    freq = np.bincount(got, minlength=z.size) / n
    p = S.distribution(z, 4, 0.7)
    assert np.all(np.abs(freq - p) <= 5 * np.sqrt(p * (1 - p) / n) + 1e-12)
