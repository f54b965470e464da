"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle as O
from rank_compressed_kv_lrkv_amd.workloads import DECODE_WORKLOADS, decode_inputs, as_f64
from tests import oracle_pins as P


def tiny_inputs():
    d = decode_inputs(DECODE_WORKLOADS["tiny_f32_T64"])
    f = lambda k: as_f64(d[k], d["dtype"])
    return (f("q"), f("k_s"), f("v_s"), f("z_k"), f("z_v"), f("b_k"), f("b_v"), d["seq_lens"])


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)


def test_brute_force_on_tiny_workload():
    P.pin_decode_brute_force(O, tiny_inputs())


def test_weight_level_on_tiny_workload():
    P.pin_weight_level_on_tiny_workload(O, tiny_inputs())


def test_brute_force_ragged_and_empty():
    q, k_s, v_s, z_k, z_v, b_k, b_v, _ = P._rand_cache(9, B=3, T=12, H=2, d_h=4, r=2)
    lens = np.array([12, 0, 5])
    P.pin_decode_brute_force(O, (q, k_s, v_s, z_k, z_v, b_k, b_v, lens))
