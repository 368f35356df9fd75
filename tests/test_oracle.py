"""The CPU oracle against its pins (hand-derived examples, closed forms,
special cases, library routines, brute force).  No GPU needed."""
import pytest

import oracle
from tests import pins


def test_quant_golden():
    pins.pin_quant_golden(oracle)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quant_error_bound(bits):
    pins.pin_quant_error_bound(oracle, bits)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quant_on_grid(bits):
    pins.pin_quant_on_grid(oracle, bits)


def test_pack_exhaustive():
    pins.pin_pack_exhaustive(oracle)


def test_routing_golden():
    pins.pin_routing_golden(oracle)


def test_topk_bruteforce():
    pins.pin_topk_bruteforce(oracle)


def test_weights():
    pins.pin_weights(oracle)


def test_permute_bruteforce():
    pins.pin_permute_bruteforce(oracle)


def test_layer_bruteforce():
    pins.pin_layer_bruteforce(oracle)


def test_layer_special_cases():
    pins.pin_layer_special_cases(oracle)


def test_on_grid_layer():
    pins.pin_on_grid_layer(oracle)


def test_bf16_and_norm():
    pins.pin_bf16_and_norm(oracle)


def test_ffn_bf16_h():
    pins.pin_ffn_bf16_h(oracle)


def test_ffn_bf16_w():
    pins.pin_ffn_bf16_w(oracle)


def test_shrink_closed_form():
    pins.pin_shrink_closed_form(oracle)


def test_group_mean():
    pins.pin_group_mean(oracle)


def test_hqq_golden():
    pins.pin_hqq_golden(oracle)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_hqq_refine(bits):
    pins.pin_hqq_refine(oracle, bits)


def test_hqq_least_squares_round():
    pins.pin_hqq_least_squares_round(oracle)


def test_kv_codec():
    pins.pin_kv_codec(oracle)
