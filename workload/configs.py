"""The seeded workloads of the paged KV-cache data plane, by name: the five
configurations and one tensor-parallel shard of the long decode.

Draw order for every workload: lengths first, then physical block ids, from one
``numpy.random.Generator(PCG64(seed))``; Q/K/V values are counter-based
(``workload.synth.bf16_values``) and keyed by the same seed.
"""
from __future__ import annotations

import math

import numpy as np

from . import synth

BLOCK = 256  # default tokens per cache block ("Nano-vLLM part 1", section 4.1)

# name -> (default seed, one-line description)
WORKLOADS = {
    "decode_edge_b4": (4191, "decode, batch 4, context {1,255,256,700}, Hq 8 / Hkv 2, d 64, 16 blocks"),
    "decode_b256": (4192, "decode, batch 256, context U[100,1024], Hq 16 / Hkv 8, d 128, 2048 blocks"),
    "prefill_varlen_s64": (4193, "causal varlen prefill, 64 seqs, length U[100,1024], Hq 32 / Hkv 8, d 128"),
    "prefill_prefix_s128": (4194, "prefix-cached prefill, 128 seqs, 2048 shared + U[64,512], Hq 32 / Hkv 8, d 128"),
    "decode_long_b512": (4195, "long decode, batch 512, context U[4096,32768], Hq 64 / Hkv 8, d 128"),
    # one GPU's share of the long decode under tensor parallelism over its 8 kv heads: the same
    # seed, so the same context lengths and block tables, at Hq 8 / Hkv 1
    "decode_long_b512_shard8": (4195, "long decode at one of 8 tensor-parallel shards: batch 512, "
                                      "context U[4096,32768], Hq 8 / Hkv 1, d 128"),
}


def make(name: str, seed: int | None = None) -> synth.Workload:
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    seed = WORKLOADS[name][0] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "decode_edge_b4":
        ctx = np.array([1, 255, 256, 700])
        return synth.decode(ctx, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=BLOCK,
                            num_blocks=16, id_mode="choice", max_blocks_per_seq=3,
                            scale=1.0 / math.sqrt(64), seed=seed, rng=rng, name=name)
    if name == "decode_b256":
        ctx = rng.integers(100, 1024, size=256, endpoint=True)
        return synth.decode(ctx, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=BLOCK,
                            num_blocks=2048, id_mode="perm", max_blocks_per_seq=1024 // BLOCK,
                            seed=seed, rng=rng, name=name)
    if name == "prefill_varlen_s64":
        lens = rng.integers(100, 1024, size=64, endpoint=True)
        return synth.prefill(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=BLOCK,
                             id_mode="choice", max_blocks_per_seq=1024 // BLOCK, seed=seed,
                             rng=rng, name=name)
    if name == "prefill_prefix_s128":
        lens = rng.integers(64, 512, size=128, endpoint=True)
        return synth.prefill(lens, prefix_len=2048, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=BLOCK, id_mode="choice",
                             max_blocks_per_seq=2048 // BLOCK + 512 // BLOCK, seed=seed,
                             rng=rng, name=name)
    if name in ("decode_long_b512", "decode_long_b512_shard8"):
        ctx = rng.integers(4096, 32768, size=512, endpoint=True)
        hq, hkv = (64, 8) if name == "decode_long_b512" else (8, 1)
        return synth.decode(ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=BLOCK,
                            id_mode="choice", max_blocks_per_seq=32768 // BLOCK, seed=seed,
                            rng=rng, name=name)
    raise AssertionError(name)
