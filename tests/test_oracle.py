"""The fp64 oracle against its pins (CPU only)."""
import pytest

import cases
import oracle_pins as P

ALL = cases.case_names()
DECODE = [n for n in ALL if cases.get(n).kind == "decode"]
PREFILL = [n for n in ALL if cases.get(n).kind == "prefill"]
TINY = ["decode_edge_b4", "decode_tiny_bs16", "decode_mha_bs32", "prefill_ragged_bs16",
        "prefill_hist_bs32", "prefill_prefix_bs16"]


def test_bf16_widening():
    P.pin_bf16_widening()


def test_pages_block_example():
    P.pin_pages_block_example()


@pytest.mark.parametrize("name", ALL)
def test_slot_walk(name):
    P.pin_slot_walk(name)


@pytest.mark.parametrize("name", ALL)
def test_store(name):
    P.pin_store(name)


def test_store_rejects_bad_slots():
    P.pin_store_rejects()


@pytest.mark.parametrize("name", ALL)
def test_paged_equals_dense(name):
    P.pin_paged_equals_dense(name)


@pytest.mark.parametrize("name", ["decode_edge_b4", "decode_b256[6]", "prefill_prefix_s128[3]",
                                  "prefill_ragged_bs16", "decode_tiny_bs16"])
def test_block_permutation(name):
    P.pin_block_permutation(name)


@pytest.mark.parametrize("name", ALL)
def test_rows_sum_to_one(name):
    P.pin_rows_sum_to_one(name)


@pytest.mark.parametrize("name", ["decode_edge_b4", "decode_tiny_bs16", "prefill_varlen_s64[4]",
                                  "prefill_ragged_bs16"])
def test_single_key_returns_v(name):
    assert P.pin_single_key_returns_v(name) > 0


@pytest.mark.parametrize("name", TINY)
def test_brute_force(name):
    P.pin_brute_force(name)


@pytest.mark.parametrize("name", ALL)
def test_torch_sdpa(name):
    P.pin_torch_sdpa(name)


def test_closed_forms():
    P.pin_closed_forms()


def test_scale_zero_is_mean_of_visible_values():
    P.pin_scale_zero_mean("prefill_scale0_mha")


@pytest.mark.parametrize("name", ["prefill_negscale_g4", "decode_negscale"])
def test_negative_scale(name):
    P.pin_negative_scale(name)


@pytest.mark.parametrize("name", PREFILL)
def test_decode_is_last_prefill_row(name):
    P.pin_decode_is_last_prefill_row(name)


@pytest.mark.parametrize("name", ["prefill_prefix_bs16", "prefill_hist_bs32"])
def test_prefix_rows_are_suffix_of_full_prefill(name):
    P.pin_prefix_rows_are_suffix_of_full_prefill(name)


@pytest.mark.parametrize("name", ["decode_edge_b4", "decode_tiny_bs16", "decode_g16"])
def test_split_merge(name):
    P.pin_split_merge(name)
