"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

A pin set that let one of these through would not be pinning the oracle.
"""
import numpy as np

import oracle.fp64 as OA
import oracle_pins as P


def _caught(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _any_caught(checks):
    return any(_caught(fn, *args) for fn, *args in checks)


def test_mutant_gqa_head_mapping(monkeypatch):
    # query head h reading KV head h % Hkv instead of h // (Hq/Hkv)
    monkeypatch.setattr(OA, "kv_head_of", lambda h, hq, hkv: h % hkv)
    assert _any_caught([(P.pin_torch_sdpa, "decode_edge_b4"),
                        (P.pin_brute_force, "decode_edge_b4")])


def test_mutant_causal_diagonal_dropped(monkeypatch):
    monkeypatch.setattr(OA, "visible_keys",
                        lambda r, off, lk, causal: lk if not causal else max(0, min(lk, off + r)))
    assert _any_caught([(P.pin_brute_force, "prefill_ragged_bs16"),
                        (P.pin_torch_sdpa, "prefill_ragged_bs16")])


def test_mutant_causal_top_left_alignment(monkeypatch):
    # ignoring the cached prefix when aligning the mask
    real = OA.attention
    monkeypatch.setattr(OA, "attention",
                        lambda q, k, v, scale, causal=False, offset=0: real(q, k, v, scale, causal, 0))
    assert _any_caught([(P.pin_brute_force, "prefill_prefix_bs16"),
                        (P.pin_decode_is_last_prefill_row, "prefill_hist_bs32")])


def test_mutant_scale_dropped(monkeypatch):
    real = OA.softmax_weights
    monkeypatch.setattr(OA, "softmax_weights",
                        lambda q, k, scale, causal=False, offset=0: real(q, k, 1.0, causal, offset))
    assert _any_caught([(P.pin_torch_sdpa, "decode_edge_b4"),
                        (P.pin_brute_force, "decode_tiny_bs16")])


def test_mutant_slot_without_block_offset(monkeypatch):
    # position added to the block base without taking it modulo the block size
    def bad_slot(row, position, bs):
        lb, _ = OA.logical_block(position, bs)
        return np.asarray(row, dtype=np.int64)[lb] * bs + np.asarray(position, dtype=np.int64)
    monkeypatch.setattr(OA, "slot_of", bad_slot)
    assert _any_caught([(P.pin_paged_equals_dense, "decode_edge_b4"),
                        (P.pin_slot_walk, "decode_edge_b4")])


def test_mutant_block_and_offset_swapped(monkeypatch):
    def bad_logical(position, bs):
        position = np.asarray(position, dtype=np.int64)
        return position % bs, position // bs
    monkeypatch.setattr(OA, "logical_block", bad_logical)
    assert _any_caught([(P.pin_pages_block_example,),
                        (P.pin_paged_equals_dense, "decode_tiny_bs16")])


def test_mutant_weights_applied_to_keys(monkeypatch):
    # the weighted sum taken over K rows instead of V rows
    real = OA.attention
    monkeypatch.setattr(OA, "attention",
                        lambda q, k, v, scale, causal=False, offset=0: real(q, k, k, scale, causal, offset))
    assert _any_caught([(P.pin_torch_sdpa, "decode_mha_bs32"),
                        (P.pin_brute_force, "decode_mha_bs32")])


def test_mutant_store_writes_padding(monkeypatch):
    # a padding entry (-1) written through, which lands on the last slot
    def bad_store(k_cache, v_cache, k, v, slot_mapping):
        kc = np.array(k_cache, copy=True)
        vc = np.array(v_cache, copy=True)
        for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
            kc[s] = k[i]
            vc[s] = v[i]
        return kc, vc
    monkeypatch.setattr(OA, "store_kvcache", bad_store)
    import oracle
    monkeypatch.setattr(oracle, "store_kvcache", bad_store)
    assert _any_caught([(P.pin_store, "decode_mha_bs32")])


def _patch_widening(monkeypatch, fn):
    import oracle
    monkeypatch.setattr(OA, "bf16_to_f64", fn)
    monkeypatch.setattr(oracle, "bf16_to_f64", fn)


def test_mutant_widening_shift(monkeypatch):
    # bf16 bits placed one position too low in the fp32 word
    def bad(bits):
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        return (b.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    _patch_widening(monkeypatch, bad)
    assert _any_caught([(P.pin_bf16_widening,)])


def test_mutant_widening_sign_dropped(monkeypatch):
    def bad(bits):
        b = np.ascontiguousarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _patch_widening(monkeypatch, bad)
    assert _any_caught([(P.pin_bf16_widening,)])


def test_mutant_widening_as_fp16(monkeypatch):
    # the bits read as IEEE half precision instead of bfloat16
    def bad(bits):
        return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    _patch_widening(monkeypatch, bad)
    assert _any_caught([(P.pin_bf16_widening,)])
