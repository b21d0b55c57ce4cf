"""CPU oracle for next-token sampling with temperature and top-k.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports or calls this
module; only the tests and the benchmark's CPU-baseline leg do.  It shares no
code with the HIP library.

What it computes, and where the pages define it:

* The model's logits over the vocabulary become the next token by sampling
  from their distribution; the temperature T reshapes it as softmax(logits/T):
  near 0 the top token is almost always taken, a large T flattens it
  ["Nano-vLLM part 1", section 5.4 "Sampling: from logits to tokens"].
* top_k bounds the candidates considered at each step ["Nano-vLLM inference
  engine architecture" (blog.hotdry.top), configuration section, on
  SamplingParams].

Readings where the pages are silent (the same in the HIP kernel's contract):
candidates are the entries whose logit is >= the k-th largest (ties at that
value all kept), in the order of the fp32 bit patterns mapped to order-
preserving unsigned keys (so -0 < +0); the draw is the Gumbel-max identity,
argmax_i fl(fl(z_i * fl(1/T)) + g_i) over the candidates with the noise g
passed in, ties to the smallest index; T <= 0 takes the first maximum of the
logits.  Every step that decides the integer result is done in fp32, as the
GPU does it; the sampling distribution itself is pinned in the tests against
softmax(z/T) restricted to the candidates.
"""
from __future__ import annotations

import numpy as np


def order_keys(z: np.ndarray) -> np.ndarray:
    """Unsigned keys that sort like the fp32 values (-0 below +0)."""
    u = np.ascontiguousarray(z, dtype=np.float32).view(np.uint32)
    return np.where(u & np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def candidates(z: np.ndarray, top_k: int) -> np.ndarray:
    """Boolean mask of the top-k candidates of one row (ties at the k-th value kept)."""
    keys = order_keys(z)
    if top_k <= 0 or top_k >= keys.size:
        return np.ones(keys.size, dtype=bool)
    kth = np.sort(keys)[keys.size - top_k]
    return keys >= kth


def sample_row(z: np.ndarray, g: np.ndarray, top_k: int, temperature: float) -> int:
    z = np.asarray(z, dtype=np.float32)
    if temperature <= 0:
        return int(np.argmax(z))
    inv_t = np.float32(1.0) / np.float32(temperature)
    idx = np.nonzero(candidates(z, top_k))[0]
    y = (z[idx] * inv_t).astype(np.float32) + np.asarray(g, dtype=np.float32)[idx]
    return int(idx[int(np.argmax(y))])


def topk_sample(logits: np.ndarray, gumbel, top_k: int, temperature: float) -> np.ndarray:
    """One token id per row: int32 [rows]."""
    logits = np.asarray(logits, dtype=np.float32)
    out = np.empty(logits.shape[0], dtype=np.int32)
    for r in range(logits.shape[0]):
        out[r] = sample_row(logits[r], None if gumbel is None else gumbel[r], top_k, temperature)
    return out


def distribution(z: np.ndarray, top_k: int, temperature: float) -> np.ndarray:
    """fp64 probabilities the draw follows: softmax(z / T) over the candidates, 0 elsewhere."""
    z = np.asarray(z, dtype=np.float64)
    mask = candidates(np.asarray(z, dtype=np.float32), top_k)
    s = np.where(mask, z / temperature, -np.inf)
    p = np.exp(s - s.max())
    return p / p.sum()
