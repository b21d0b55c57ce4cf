"""Pins of the fp64 oracle to facts outside itself.

Each ``pin_*`` raises AssertionError when the oracle disagrees with what the
pages or the mathematics fix.  ``test_oracle.py`` runs them on the real oracle;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle (on the CPU)
and checks that some pin catches each one.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os

import numpy as np
import torch

import cases
import oracle
import oracle.fp64 as OA
from oracle import brute
import workload as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(bits):
    return oracle.bf16_to_f64(bits)


# ---- number format: bf16 bit patterns widened to fp64 ------------------------------
def _bf16_from_fields(bits: int) -> float:
    """bf16 value from its fields (1 sign, 8 exponent bits biased by 127, 7 fraction
    bits; exponent 0 is zero or subnormal, 255 is inf or NaN), in Python integers and
    math.ldexp: a decoding of the format's definition that shares nothing with the
    oracle's shift-and-reinterpret route."""
    sign = -1.0 if bits >> 15 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -126 - 7)
    return sign * math.ldexp(128 + frac, exp - 127 - 7)


def pin_bf16_widening():
    """All 65,536 bf16 bit patterns: the oracle's widening equals torch's bfloat16 ->
    float64 conversion and the field-by-field decoding, with the sign of zero kept
    and NaN exactly where the format puts it."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits)
    assert got.dtype == np.float64 and got.shape == bits.shape
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fields = np.array([_bf16_from_fields(int(b)) for b in bits], dtype=np.float64)
    for ref in (lib, fields):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
        assert np.array_equal(got[~nan], ref[~nan]), "values differ"
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signs differ"
    # a few patterns spelled out: 1, -2, the smallest subnormal, the largest finite, inf
    for b, v in ((0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133),
                 (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0xFF80, -math.inf)):
        assert oracle.bf16_to_f64(np.array([b], np.uint16))[0] == v, hex(b)


# ---- the pages' own worked example --------------------------------------------------
def pin_pages_block_example():
    """700 tokens in 256-token blocks: 3 blocks, 188 in the last, 68 idle."""
    g = json.load(open(os.path.join(GOLDEN, "block_fill_700.json")))
    n, last, idle = oracle.block_fill(g["num_tokens"], g["block_size"])
    assert (n, last, idle) == (g["blocks"], g["tokens_in_last_block"], g["idle_slots"])
    assert n - 1 == g["full_blocks"]
    # the last token (position 699) sits in the third block at its 188th slot
    lb, off = oracle.logical_block(g["num_tokens"] - 1, g["block_size"])
    assert (int(lb), int(off)) == (g["blocks"] - 1, g["tokens_in_last_block"] - 1)


def pin_slot_walk(name):
    """Positions of a sequence fill its listed blocks in order, one slot each."""
    w = cases.get(name)
    bs = w.block_size
    for s in range(w.num_seqs):
        n = int(w.lk[s])
        if n == 0:
            continue
        pos = np.arange(n)
        slots = oracle.slot_of(w.block_tables[s], pos, bs)
        assert np.unique(slots).size == n
        nb = oracle.blocks_for(n, bs)
        used = w.block_tables[s][:nb]
        assert ((slots // bs) == np.repeat(used, bs)[:n]).all()
        assert ((slots % bs) == np.tile(np.arange(bs), nb)[:n]).all()
        # the generator's control-plane slots for the new tokens agree
        new = np.arange(n - int(w.lq[s]), n)
        assert (oracle.slot_of(w.block_tables[s], new, bs) == w.slots(s, new)).all()


# ---- store -------------------------------------------------------------------------
def pin_store(name):
    """The store writes exactly the new tokens' rows; every other slot keeps its bits."""
    w = cases.get(name)
    h = cases.inputs(name)
    kc, vc = oracle.store_kvcache(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"],
                                  h["slot_mapping"])
    sm = h["slot_mapping"].astype(np.int64)
    live = sm >= 0
    assert (kc[sm[live]] == h["k_new"][live]).all() and (vc[sm[live]] == h["v_new"][live]).all()
    untouched = np.ones(kc.shape[0], bool)
    untouched[sm[live]] = False
    assert (kc[untouched] == h["k_cache"][untouched]).all()
    assert (vc[untouched] == h["v_cache"][untouched]).all()
    # the generator's new rows equal the dense token rows at those positions
    for s in range(w.num_seqs):
        if w.lq[s] == 0:
            continue
        _, kd, vd = w.dense(s)
        sl = w.slots(s, np.arange(w.lk[s] - w.lq[s], w.lk[s]))
        assert (kc[sl] == kd[-int(w.lq[s]):]).all() and (vc[sl] == vd[-int(w.lq[s]):]).all()
    oracle.check_store_targets(h["slot_mapping"], h["block_tables"], w.block_size)


def pin_store_rejects():
    kc = np.zeros((8, 1, 2), np.uint16)
    k = np.ones((2, 1, 2), np.uint16)
    for bad in ([3, 3], [0, 8]):
        try:
            oracle.store_kvcache(kc, kc, k, k, np.array(bad))
        except (ValueError, IndexError):
            continue
        raise AssertionError(f"store accepted slots {bad}")
    bt = np.array([[0, 1], [0, 2]])
    try:
        oracle.check_store_targets(np.array([1]), bt, block_size=4)  # slot 1 is in shared block 0
    except ValueError:
        pass
    else:
        raise AssertionError("store into a shared block accepted")


# ---- attention ----------------------------------------------------------------------
def _dense_rows(w, s):
    qd, kd, vd = w.dense(s)
    lq, lk = int(w.lq[s]), int(w.lk[s])
    causal = w.kind == "prefill" and w.causal
    return oracle.attention(_f64(qd), _f64(kd), _f64(vd), w.scale, causal, lk - lq)


def _rows_of(w, out, s):
    if w.kind == "decode":
        return out[s:s + 1]
    q0 = int(w.cu_seqlens_q[s])
    return out[q0:q0 + int(w.lq[s])]


def pin_paged_equals_dense(name):
    """Gathering through block tables gives exactly the contiguous tokens' result."""
    w = cases.get(name)
    out = cases.run_oracle(w, cases.inputs(name))
    for s in range(w.num_seqs):
        if w.kind == "decode" and w.lk[s] == 0:
            assert (out[s] == 0).all()
            continue
        assert np.array_equal(_rows_of(w, out, s), _dense_rows(w, s)), f"seq {s}"


def pin_block_permutation(name, seed=5):
    """Moving blocks to other physical ids changes nothing (bitwise)."""
    w = cases.get(name)
    base = cases.run_oracle(w, cases.inputs(name))
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(w.num_blocks)
    wp = w.permute_blocks(perm)
    h = wp.host_inputs()
    kc, vc = oracle.store_kvcache(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"],
                                  h["slot_mapping"])
    out = cases.run_oracle(wp, h, kc, vc)
    assert np.array_equal(out, base)


def pin_rows_sum_to_one(name):
    w = cases.get(name)
    for s in range(min(w.num_seqs, 3 if w.kind == "decode" else 1)):
        qd, kd, _ = w.dense(s)
        if w.lk[s] == 0 or qd.shape[0] == 0:
            continue
        causal = w.kind == "prefill" and w.causal
        p = oracle.softmax_weights(_f64(qd), _f64(kd), w.scale, causal,
                                   int(w.lk[s] - w.lq[s]))
        assert np.abs(p.sum(axis=2) - 1.0).max() < 1e-12
        assert (p >= 0).all()


def pin_single_key_returns_v(name):
    """A row that sees exactly one key returns that key's V row, exactly.

    Decode with context 1, and the first row of a causal prefill without cached
    history or prefix.
    """
    w = cases.get(name)
    h = cases.inputs(name)
    out = cases.run_oracle(w, h)
    g = w.num_q_heads // w.num_kv_heads
    hit = 0
    for s in range(w.num_seqs):
        sees_one = (w.kind == "decode" and w.lk[s] == 1) or \
                   (w.kind == "prefill" and w.causal and w.lq[s] > 0 and w.lk[s] == w.lq[s])
        if not sees_one:
            continue
        _, _, vd = w.dense(s)
        row = _rows_of(w, out, s)[0]
        for hq in range(w.num_q_heads):
            assert np.array_equal(row[hq], _f64(vd[0, hq // g]))
        hit += 1
    return hit


def pin_brute_force(name, rows_limit=6):
    """The scalar pure-Python route agrees within 1e-12 on tiny inputs."""
    w = cases.get(name)
    h = cases.inputs(name)
    out = cases.run_oracle(w, h)
    kc = _f64(h["k_cache_stored"]).tolist()
    vc = _f64(h["v_cache_stored"]).tolist()
    q = _f64(h["q"]).tolist()
    bt = h["block_tables"].tolist()
    if w.kind == "decode":
        ref = brute.decode(q, kc, vc, bt, h["context_lens"].tolist(), w.block_size, w.scale)
    else:
        ref = brute.prefill(q, kc, vc, h["cu_seqlens_q"].tolist(), h["cu_seqlens_k"].tolist(),
                            bt, w.block_size, w.scale, w.causal)
    ref = np.array(ref, dtype=np.float64).reshape(out.shape)
    assert np.abs(ref - out).max() < 1e-12, np.abs(ref - out).max()


def pin_torch_sdpa(name):
    """Where torch's fp64 CPU attention states the same problem, it agrees to 1e-12.

    torch maps query head h to KV head h // (Hq/Hkv) with ``enable_gqa`` and its
    causal mask is aligned top-left, which equals our alignment when Lq == Lk.
    """
    w = cases.get(name)
    out = cases.run_oracle(w, cases.inputs(name))
    checked = 0
    for s in range(w.num_seqs):
        lq, lk = int(w.lq[s]), int(w.lk[s])
        causal = w.kind == "prefill" and w.causal
        if lk == 0 or lq == 0 or (causal and lq != lk):
            continue
        if w.scale <= 0:
            # torch's math path scales the masked (-inf) scores too, so a non-positive
            # scale turns its mask into +inf / NaN; those cases have pins of their own
            continue
        qd, kd, vd = (torch.from_numpy(_f64(x)).transpose(0, 1)[None] for x in w.dense(s))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qd.contiguous(), kd.contiguous(), vd.contiguous(), is_causal=causal,
            scale=w.scale, enable_gqa=True)[0].transpose(0, 1).numpy()
        assert np.abs(ref - _rows_of(w, out, s)).max() < 1e-12
        checked += 1
    return checked


def pin_scale_zero_mean(name):
    """Scale 0: every visible key has the same score, so each row is the mean of
    the V rows it sees (causal limit included)."""
    w = cases.get(name)
    assert w.scale == 0.0
    out = cases.run_oracle(w, cases.inputs(name))
    g = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        lq, lk = int(w.lq[s]), int(w.lk[s])
        if lq == 0:
            continue
        _, _, vd = w.dense(s)
        v = _f64(vd)  # [Lk, Hkv, d]
        rows = _rows_of(w, out, s)
        for r in range(rows.shape[0]):
            n = (lk - lq + r + 1) if (w.kind == "prefill" and w.causal) else lk
            for h in range(w.num_q_heads):
                ref = v[:n, h // g].mean(axis=0) if n > 0 else np.zeros(w.head_dim)
                assert np.abs(rows[r, h] - ref).max() < 1e-12


def pin_negative_scale(name):
    """softmax(scale * q.k) with scale < 0 equals the attention of -q at -scale > 0
    (exact in fp64: negating q and the scale changes no magnitude)."""
    w = cases.get(name)
    assert w.scale < 0
    h = cases.inputs(name)
    out = cases.run_oracle(w, h)
    h2 = dict(h)
    h2["q"] = h["q"] ^ np.uint16(0x8000)
    out2 = cases.run_oracle(dataclasses.replace(w, scale=-w.scale), h2)
    assert np.array_equal(out, out2)
    # and it is not the attention at |scale| (the sign matters)
    out3 = cases.run_oracle(dataclasses.replace(w, scale=-w.scale), h)
    assert np.abs(out3 - out).max() > 1e-3


def pin_closed_forms():
    """Textbook special cases of softmax attention."""
    rng = np.random.Generator(np.random.PCG64(3))
    lk, hq, hkv, d = 9, 4, 2, 8
    k = rng.standard_normal((lk, hkv, d))
    v = rng.standard_normal((lk, hkv, d))
    q = rng.standard_normal((3, hq, d))
    g = hq // hkv
    # q = 0: uniform weights -> mean of V over the visible keys
    out = oracle.attention(np.zeros_like(q), k, v, 0.5)
    for h in range(hq):
        assert np.abs(out[:, h] - v[:, h // g].mean(axis=0)).max() < 1e-12
    # all keys equal: uniform weights again, for any q
    keq = np.repeat(k[:1], lk, axis=0)
    out = oracle.attention(q, keq, v, 0.7)
    for h in range(hq):
        assert np.abs(out[:, h] - v[:, h // g].mean(axis=0)).max() < 1e-12
    # causal with offset 2: row r sees keys 0..r+2, so with q = 0 it is their running mean
    out = oracle.attention(np.zeros_like(q), k, v, 1.0, causal=True, offset=2)
    for r in range(3):
        for h in range(hq):
            assert np.abs(out[r, h] - v[:r + 3, h // g].mean(axis=0)).max() < 1e-12
    # constant V rows c: the output is c whatever the weights
    c = rng.standard_normal((1, hkv, d))
    out = oracle.attention(q, k, np.repeat(c, lk, axis=0), 1.3)
    for h in range(hq):
        assert np.abs(out[:, h] - c[0, h // g]).max() < 1e-12
    # two keys whose scores differ by log(3): weights 1/4 and 3/4
    k2 = np.zeros((2, 1, 1))
    k2[1, 0, 0] = 1.0
    v2 = np.array([[[4.0]], [[8.0]]])
    out = oracle.attention(np.ones((1, 1, 1)), k2, v2, math.log(3.0))
    assert abs(out[0, 0, 0] - 7.0) < 1e-12


def pin_decode_is_last_prefill_row(name):
    """Prefill row r equals a decode of that query over keys 0 .. off + r (all Lk keys
    without the causal limit)."""
    w = cases.get(name)
    assert w.kind == "prefill"
    h = cases.inputs(name)
    out = cases.run_oracle(w, h)
    for s in range(w.num_seqs):
        lq, lk = int(w.lq[s]), int(w.lk[s])
        q0 = int(w.cu_seqlens_q[s])
        for r in sorted({0, lq // 2, lq - 1}) if lq else []:
            ctx = np.array([lk - lq + r + 1 if w.causal else lk], np.int32)
            dec = oracle.paged_decode(h["q"][q0 + r:q0 + r + 1], h["k_cache_stored"],
                                      h["v_cache_stored"], h["block_tables"][s:s + 1], ctx,
                                      w.block_size, w.scale)
            assert np.abs(dec[0] - out[q0 + r]).max() < 1e-12


def pin_prefix_rows_are_suffix_of_full_prefill(name):
    """With a cached prefix, the rows equal the tail of one causal prefill over all tokens."""
    w = cases.get(name)
    out = cases.run_oracle(w, cases.inputs(name))
    rng = np.random.Generator(np.random.PCG64(9))
    for s in range(w.num_seqs):
        qd, kd, vd = (_f64(x) for x in w.dense(s))
        lq, lk = int(w.lq[s]), int(w.lk[s])
        if lq == 0:
            continue
        head = rng.standard_normal((lk - lq,) + qd.shape[1:])  # queries for earlier positions
        full = oracle.attention(np.concatenate([head, qd]), kd, vd, w.scale, causal=True, offset=0)
        assert np.abs(full[lk - lq:] - _rows_of(w, out, s)).max() < 1e-12


def pin_split_merge(name, chunks=(256, 512, 2048, 16)):
    """Chunked partial softmax states merged by log-sum-exp equal the one-pass result.

    For chunk c of the keys: m_c = max score, l_c = sum exp(s - m_c),
    a_c = sum exp(s - m_c) v.  Then M = max m_c, out = sum e^(m_c-M) a_c / sum e^(m_c-M) l_c.
    """
    w = cases.get(name)
    assert w.kind == "decode"
    out = cases.run_oracle(w, cases.inputs(name))
    g = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        n = int(w.lk[s])
        if n == 0:
            continue
        qd, kd, vd = (_f64(x) for x in w.dense(s))
        for c in chunks:
            for h in range(w.num_q_heads):
                sc = (kd[:, h // g] @ qd[0, h]) * w.scale
                ms, ls, acc = [], [], []
                for j0 in range(0, n, c):
                    part = sc[j0:j0 + c]
                    m = part.max()
                    e = np.exp(part - m)
                    ms.append(m)
                    ls.append(e.sum())
                    acc.append(e @ vd[j0:j0 + c, h // g])
                M = max(ms)
                wts = np.exp(np.array(ms) - M)
                merged = (wts[:, None] * np.array(acc)).sum(0) / (wts * np.array(ls)).sum()
                assert np.abs(merged - out[s, h]).max() < 1e-12
