"""Shared workload cases for the tests (CPU side): inputs plus oracle results."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import workload as W


def small_workloads():
    """Cheap CPU cases covering every configuration's shape and the edge cases."""
    cases = {}
    cases["decode_edge_b4"] = W.make("decode_edge_b4")
    c2 = W.make("decode_b256")
    cases["decode_b256[6]"] = c2.subset([0, 1, 17, 100, 200, 255])
    c3 = W.make("prefill_varlen_s64")
    short = np.argsort(c3.lq)[:3].tolist() + [int(np.argmax(c3.lq))]
    cases["prefill_varlen_s64[4]"] = c3.subset(short)
    c4 = W.make("prefill_prefix_s128")
    cases["prefill_prefix_s128[3]"] = c4.subset([0, 5, 77])
    c5 = W.make("decode_long_b512")
    cases["decode_long_b512[2]"] = c5.subset([int(np.argmin(c5.lk)), 3])
    # edge cases: tiny blocks, empty and ragged contexts, every GQA group size
    cases["decode_tiny_bs16"] = W.decode([0, 1, 15, 16, 17, 33, 64], num_q_heads=4, num_kv_heads=1,
                                         head_dim=64, block_size=16, seed=11, name="decode_tiny_bs16")
    cases["decode_mha_bs32"] = W.decode([31, 32, 1, 97], num_q_heads=2, num_kv_heads=2,
                                        head_dim=128, block_size=32, seed=12, pad_tokens=3,
                                        name="decode_mha_bs32")
    cases["decode_g16"] = W.decode([5, 300], num_q_heads=16, num_kv_heads=1, head_dim=128,
                                   block_size=256, seed=13, name="decode_g16")
    cases["prefill_ragged_bs16"] = W.prefill([0, 1, 17, 40, 3], num_q_heads=4, num_kv_heads=2,
                                             head_dim=64, block_size=16, seed=14,
                                             name="prefill_ragged_bs16")
    cases["prefill_hist_bs32"] = W.prefill([5, 33, 1], hist=[7, 0, 40], num_q_heads=8,
                                           num_kv_heads=2, head_dim=128, block_size=32, seed=15,
                                           name="prefill_hist_bs32")
    cases["prefill_prefix_bs16"] = W.prefill([3, 20], prefix_len=32, num_q_heads=2,
                                             num_kv_heads=1, head_dim=64, block_size=16, seed=16,
                                             name="prefill_prefix_bs16")
    # scales the pages never use (negative, zero), full (non-causal) attention, GQA ratios
    # 1, 3 and 8, and enough query tiles that every prefill workgroup runs several items
    cases["prefill_negscale_g4"] = W.prefill([20, 70, 1], num_q_heads=8, num_kv_heads=2,
                                             head_dim=128, block_size=32, seed=17, scale=-0.3,
                                             name="prefill_negscale_g4")
    cases["prefill_scale0_mha"] = W.prefill([9, 150], num_q_heads=2, num_kv_heads=2,
                                            head_dim=64, block_size=16, seed=18, scale=0.0,
                                            name="prefill_scale0_mha")
    cases["prefill_full_g3"] = W.prefill([12, 40, 0, 5], hist=[30, 0, 0, 9], num_q_heads=6,
                                         num_kv_heads=2, head_dim=64, block_size=16, seed=19,
                                         causal=False, name="prefill_full_g3")
    lens = np.random.Generator(np.random.PCG64(20)).integers(1, 300, size=48, endpoint=True)
    cases["prefill_g8_many"] = W.prefill(lens.tolist(), num_q_heads=16, num_kv_heads=2,
                                         head_dim=64, block_size=64, seed=20,
                                         name="prefill_g8_many")
    cases["decode_negscale"] = W.decode([3, 40, 257], num_q_heads=8, num_kv_heads=4,
                                        head_dim=128, block_size=16, seed=22, scale=-0.5,
                                        name="decode_negscale")
    # a large scale: the scaled scores spread over tens of log2 units, so rows meet keys far
    # above the first tile's maximum and the kernels' lazy rescale of the running max runs
    cases["prefill_bigscale"] = W.prefill([190, 64, 129], hist=[0, 100, 0], num_q_heads=4,
                                          num_kv_heads=1, head_dim=128, block_size=32, seed=23,
                                          scale=3.0, name="prefill_bigscale")
    cases["decode_bigscale"] = W.decode([190, 700, 5], num_q_heads=4, num_kv_heads=2,
                                        head_dim=128, block_size=16, seed=24, scale=3.0,
                                        name="decode_bigscale")
    # blocks larger than the default: full (non-causal) prefill at head_dim 128 and GQA
    # ratio 8 over 128-token blocks, with history; decode over 1024-token blocks with
    # contexts on both sides of a block boundary
    cases["prefill_full_d128_g8_bs128"] = W.prefill(
        [70, 130, 1], hist=[0, 200, 50], num_q_heads=16, num_kv_heads=2, head_dim=128,
        block_size=128, seed=32, causal=False, name="prefill_full_d128_g8_bs128")
    cases["decode_bs1024"] = W.decode([1, 1023, 1024, 1025, 2500], num_q_heads=8, num_kv_heads=2,
                                      head_dim=128, block_size=1024, seed=33,
                                      name="decode_bs1024")
    # batches whose (sequence, kv head) items outnumber the resident workgroups several
    # times over: many equal contexts, empty contexts, head groups of 16 with two groups
    # per kv head, and batches of 512 and 513 sequences
    rng = np.random.Generator(np.random.PCG64(25))
    cases["decode_many_b300"] = W.decode(
        rng.choice([0, 1, 2, 37, 64, 100, 129, 160], size=300).tolist(), num_q_heads=8,
        num_kv_heads=4, head_dim=64, block_size=32, seed=25, name="decode_many_b300")
    cases["decode_many_g32"] = W.decode(
        rng.integers(0, 80, size=260, endpoint=True).tolist(), num_q_heads=32, num_kv_heads=1,
        head_dim=64, block_size=16, seed=26, name="decode_many_g32")
    cases["decode_many_b512"] = W.decode(
        rng.integers(1, 40, size=512, endpoint=True).tolist(), num_q_heads=16, num_kv_heads=8,
        head_dim=128, block_size=32, seed=27, name="decode_many_b512")
    cases["decode_b513"] = W.decode(
        rng.integers(1, 20, size=513, endpoint=True).tolist(), num_q_heads=1, num_kv_heads=1,
        head_dim=64, block_size=16, seed=28, name="decode_b513")
    # batches past 1024 sequences: the decode work order keeps at most four lengths per
    # thread in registers and reads the rest again (five per thread here, many equal
    # lengths), past 2048 decode keeps batch order; the prefill plan lists more than 1024
    # sequences in batch order
    cases["decode_b1100"] = W.decode(
        rng.choice([0, 1, 3, 16, 17, 40], size=1100).tolist(), num_q_heads=2, num_kv_heads=1,
        head_dim=64, block_size=16, seed=29, name="decode_b1100")
    cases["decode_b2100"] = W.decode(
        rng.choice([0, 1, 2, 5, 33], size=2100).tolist(), num_q_heads=1, num_kv_heads=1,
        head_dim=64, block_size=16, seed=31, name="decode_b2100")
    cases["prefill_s1030"] = W.prefill(
        rng.integers(0, 6, size=1030, endpoint=True).tolist(), num_q_heads=2, num_kv_heads=1,
        head_dim=64, block_size=16, seed=30, name="prefill_s1030")
    return cases


@functools.lru_cache(maxsize=None)
def _cases():
    return small_workloads()


def case_names():
    return list(_cases().keys())


def get(name):
    return _cases()[name]


@functools.lru_cache(maxsize=None)
def inputs(name):
    """Host inputs (uint16 bf16 bits) and the cache images after the oracle store."""
    w = get(name)
    h = w.host_inputs()
    kc, vc = oracle.store_kvcache(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"],
                                  h["slot_mapping"])
    h["k_cache_stored"], h["v_cache_stored"] = kc, vc
    return h


def run_oracle(w, h, k_cache=None, v_cache=None):
    kc = h["k_cache_stored"] if k_cache is None else k_cache
    vc = h["v_cache_stored"] if v_cache is None else v_cache
    if w.kind == "decode":
        return oracle.paged_decode(h["q"], kc, vc, h["block_tables"], h["context_lens"],
                                   w.block_size, w.scale)
    return oracle.paged_prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["cu_seqlens_k"],
                                h["block_tables"], w.block_size, w.scale, w.causal)


@functools.lru_cache(maxsize=None)
def reference(name):
    w = get(name)
    return run_oracle(w, inputs(name))
