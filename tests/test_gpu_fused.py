"""Fused decode step (store the new tokens and attend, one kernel).

The fused call must leave, bit for bit, the same cache image as the store
kernel, and its output must match the fp64 oracle to the attention tolerance
and the store-then-decode output to the same bound (the new token enters the
softmax state last instead of inside its tile, so fp32 rounding order
differs).
"""
import sys

import numpy as np
import pytest
import torch

import cases
import gpu_harness as H
import paged_kv_cache_419_amd as pkv
import workload as W

pytestmark = pytest.mark.gpu

DECODE = [n for n in cases.case_names() if cases.get(n).kind == "decode"]


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _per_sequence(w, t):
    """k_new / v_new / slot_mapping with one row per sequence: the store's rows for
    sequences with a new token, zeros and slot -1 for an empty context."""
    b = w.num_seqs
    has = torch.from_numpy(w.lq.astype(np.int64) > 0).cuda()
    tok = torch.cumsum(has.long(), 0) - 1  # store row of each sequence's token
    kn = torch.zeros((b,) + tuple(t["k_new"].shape[1:]), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros_like(kn)
    sm = torch.full((b,), -1, dtype=torch.int32, device="cuda")
    kn[has] = t["k_new"][tok[has]]
    vn[has] = t["v_new"][tok[has]]
    sm[has] = t["slot_mapping"][tok[has]]
    return kn.contiguous(), vn.contiguous(), sm


def _check(w, split, seqs):
    te = w.materialize("cuda")
    pkv.store_kvcache(te["k_new"], te["v_new"], te["k_cache"], te["v_cache"], te["slot_mapping"])
    ref = torch.full_like(te["q"], float("nan"))
    pkv.paged_decode_attention(ref, te["q"], te["k_cache"], te["v_cache"], te["block_tables"],
                               te["context_lens"], w.block_size, w.max_context_len, w.scale, split)
    torch.cuda.synchronize()
    ref_k, ref_v = te["k_cache"], te["v_cache"]
    del te
    tf = w.materialize("cuda")
    kn, vn, sm = _per_sequence(w, tf)
    out = torch.full_like(tf["q"], float("nan"))
    pkv.store_and_decode(out, tf["q"], kn, vn, tf["k_cache"], tf["v_cache"], sm, tf["block_tables"],
                         tf["context_lens"], w.block_size, w.max_context_len, w.scale, split)
    torch.cuda.synchronize()
    assert torch.equal(tf["k_cache"].view(torch.int16), ref_k.view(torch.int16))
    assert torch.equal(tf["v_cache"].view(torch.int16), ref_v.view(torch.int16))
    ok, ea, er = H.compare(H.to_f64(out), H.to_f64(ref))
    assert ok, f"fused vs store-then-decode: max abs diff {ea:.3e}"
    H.check_against_oracle(w, out, seqs)


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("name", DECODE)
def test_fused_matches_store_then_decode(name, split):
    _note(f"fused {name} split {split}")
    w = cases.get(name)
    _check(w, split, list(range(w.num_seqs)))


def test_fused_full_size_decode_b256():
    _note("fused full size decode_b256")
    w = W.make("decode_b256")
    rng = np.random.Generator(np.random.PCG64(12))
    seqs = sorted({0, int(np.argmax(w.lk))} | set(int(x) for x in rng.choice(w.num_seqs, 16, replace=False)))
    _check(w, 0, seqs)


def test_fused_last_split_holds_only_the_new_token():
    # context 257 with 256-token splits: the new token is alone in the second split
    _note("fused lone new token")
    w = W.decode([257, 33, 256, 1], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=256,
                 seed=31, name="fused_lone")
    _check(w, 256, list(range(w.num_seqs)))
