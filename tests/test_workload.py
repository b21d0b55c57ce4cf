"""The seeded generator: valid control-plane outputs and device-independent values."""
import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload.synth import bf16_value_ref, bf16_values


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_metadata_valid(name):
    w = W.make(name)
    bs = w.block_size
    assert w.block_tables.dtype == np.int32
    live = w.block_tables[w.block_tables >= 0]
    assert live.max() < w.num_blocks
    # capacity: every sequence's context fits its allocated blocks and the row stride
    for s in range(w.num_seqs):
        n = int(w.lk[s])
        nb = oracle.blocks_for(n, bs)
        assert nb <= w.max_blocks_per_seq
        assert (w.block_tables[s, :nb] >= 0).all() and (w.block_tables[s, nb:] < 0).all()
    # distinct ids except the shared prefix, which every table lists
    ids, counts = np.unique(live, return_counts=True)
    npre = w.prefix_len // bs
    if npre:
        shared = w.block_tables[0, :npre]
        assert (w.block_tables[:, :npre] == shared[None, :]).all()
        assert set(ids[counts > 1].tolist()) == set(shared.tolist())
        assert (counts[np.isin(ids, shared)] == w.num_seqs).all()  # ref count = tables
    else:
        assert (counts == 1).all()
    sm = w.slot_mapping
    assert np.unique(sm[sm >= 0]).size == (sm >= 0).sum()
    oracle.check_store_targets(sm, w.block_tables, bs)  # never writes a shared block
    assert sm.shape[0] == w.num_new_tokens


def test_published_shapes():
    c1 = W.make("decode_edge_b4")
    assert c1.context_lens.tolist() == [1, 255, 256, 700] and c1.num_blocks == 16
    assert (c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.scale) == (8, 2, 64, 0.125)
    c2 = W.make("decode_b256")
    assert c2.num_seqs == 256 and c2.num_blocks == 2048
    assert 100 <= c2.lk.min() and c2.lk.max() <= 1024
    c3 = W.make("prefill_varlen_s64")
    assert c3.num_seqs == 64 and (c3.lk == c3.lq).all() and 100 <= c3.lq.min() <= c3.lq.max() <= 1024
    c4 = W.make("prefill_prefix_s128")
    assert c4.num_seqs == 128 and c4.prefix_len == 2048 and 64 <= c4.lq.min() <= c4.lq.max() <= 512
    c5 = W.make("decode_long_b512")
    assert c5.num_seqs == 512 and 4096 <= c5.lk.min() and c5.lk.max() <= 32768
    demand = sum(oracle.blocks_for(int(n), 256) for n in c5.lk)
    assert c5.num_blocks == int(np.ceil(1.1 * demand))
    # one tensor-parallel shard of c5: its lengths and tables, one kv head and its 8 query heads
    sh = W.make("decode_long_b512_shard8")
    assert (sh.lk == c5.lk).all() and (sh.block_tables == c5.block_tables).all()
    assert (sh.num_q_heads, sh.num_kv_heads, sh.head_dim) == (8, 1, 128)


def test_deterministic():
    a, b = W.make("decode_b256"), W.make("decode_b256")
    assert (a.block_tables == b.block_tables).all() and (a.lk == b.lk).all()
    c = W.make("decode_b256", seed=1)
    assert not (a.lk == c.lk).all()


def test_values_match_integer_reference():
    rng = np.random.Generator(np.random.PCG64(0))
    idx = np.concatenate([np.arange(70), rng.integers(0, 1 << 40, size=200),
                          [2**31 - 1, 2**31, 2**32 - 1, 2**32, 2**33 + 5]])
    got = bf16_values(3, 2, torch.from_numpy(idx.astype(np.int64)))
    got = got.view(torch.int16).numpy().view(np.uint16)
    assert got.tolist() == [bf16_value_ref(3, 2, int(i)) for i in idx]


def test_values_distribution():
    v = bf16_values(1, 2, torch.arange(1 << 20, dtype=torch.int64)).float()
    assert abs(v.mean().item()) < 0.01 and abs(v.std().item() - 1.0) < 0.01
    assert torch.isfinite(v).all()


def test_subset_keeps_values():
    w = W.make("prefill_prefix_s128")
    sub = w.subset([3, 9])
    for i, s in enumerate([3, 9]):
        a, b = w.dense(s), sub.dense(i)
        assert all((x == y).all() for x, y in zip(a, b))
    assert sub.num_blocks == 8 + sum(oracle.blocks_for(int(n), 256) for n in sub.lq)


def test_pool_exhaustion_raises():
    with pytest.raises(ValueError):
        W.decode([300, 300], num_q_heads=1, num_kv_heads=1, head_dim=64, block_size=256,
                 num_blocks=3, seed=1)


def test_cache_image_poisoned_outside_history():
    w = W.make("decode_edge_b4")
    h = w.host_inputs()
    rows, slots = w.history_tokens()
    mask = np.ones(w.num_slots, bool)
    mask[slots] = False
    assert (h["k_cache"][mask] == W.BF16_POISON).all() and (h["v_cache"][mask] == W.BF16_POISON).all()
    assert (h["k_cache"][slots] != W.BF16_POISON).any()
