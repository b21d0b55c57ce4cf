"""Seeded inputs of the sampling step: synthetic logits and Gumbel noise.

Holds no sampling arithmetic: logits are N(0, scale^2) draws rounded to fp32,
and the noise is the standard Gumbel transform -log(-log(u)) of uniform draws
u in (0, 1) (the random numbers a sampler draws, passed in as an input).
"""
from __future__ import annotations

import numpy as np

# Vocabulary of the synthetic sampling workload: the size of a Qwen-family
# tokenizer (the pages name Qwen among the model families); top_k and the
# temperature are in the ranges the pages suggest (top_k 50-100, T 0.7-1.0).
SAMPLE_VOCAB = 151936
SAMPLE_ROWS = 256
SAMPLE_TOP_K = 50
SAMPLE_TEMPERATURE = 0.8


def gumbel_noise(rng: np.random.Generator, shape) -> np.ndarray:
    u = (rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.float64) + 0.5) / 2.0 ** 32
    return (-np.log(-np.log(u))).astype(np.float32)


def sample_inputs(rows: int, vocab: int, seed: int, scale: float = 3.0):
    """(logits fp32 [rows, vocab], gumbel fp32 [rows, vocab])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = (rng.standard_normal((rows, vocab)) * scale).astype(np.float32)
    return logits, gumbel_noise(rng, (rows, vocab))
