"""The CPU oracle against its pins (runs without a GPU)."""
import json
import os

import numpy as np
import pytest

import oracle_pins
from oracle.compare import (ABS_TOL, MAX_ULP, bf16_rne, bits_of_bf16_values, bits_to_f64,
                            compare, mismatch_offsets, ulp_dist)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", sorted(oracle_pins.PINS))
def test_pin(oracle, name):
    oracle_pins.PINS[name](oracle)


def test_oracle_is_unmutated(oracle):
    assert oracle.mutation == 0


def test_bf16_rne_closed_forms():
    # exact values stay; halfway cases go to even; carries across a binade
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-7, -0.0, 2.0 - 2**-9,
                  3.0 * 2**-130, 1.0 + 2**-8 + 2**-40])
    want = np.array([1.0, 1.0, 1.0 + 4 * 2**-8, 1.0 + 2**-7, -0.0, 2.0, 3.0 * 2**-130,
                     1.0 + 2**-7])
    assert np.array_equal(bf16_rne(x), want)
    # matches torch's float32 -> bf16 RNE wherever the value is a float32
    import torch
    rng = np.random.default_rng(0)
    f = rng.standard_normal(10000).astype(np.float32)
    t = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_rne(f.astype(np.float64)), t)


def test_comparator_selftest_matches_page():
    """Plant 1-ulp corruptions where the pages did; exactly those offsets are
    flagged and the bitwise share lands on the printed figure."""
    g = json.load(open(os.path.join(GOLDEN, "comparator_selftest.json")))
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(g["elements"]) * 0.05
    exact = bits_of_bf16_values(bf16_rne(ref))
    rep = compare(exact, ref)
    assert rep.ok and rep.bitwise_pct == g["bitwise_pct_before"]
    bad = exact.copy()
    for off in g["offsets"]:
        bad[off] = bad[off] + 1 if bad[off] & 0x7FFF != 0x7F7F else bad[off] - 1
    assert list(mismatch_offsets(bad, ref)) == g["offsets"]
    rep = compare(bad, ref)
    assert round(rep.bitwise_pct, 4) == g["bitwise_pct_after"]
    assert rep.max_ulp == 1 and rep.ok          # one step is inside the gate
    # three steps at one offset fail the gate, and only there
    worse = exact.copy()
    worse[700] = worse[700] + 3
    rep = compare(worse, ref)
    assert rep.n_fail == 1 and rep.worst[0] == 700


def test_comparator_rejects_nan_and_abs():
    ref = np.array([0.5, 0.25, 100.0])
    bits = bits_of_bf16_values(bf16_rne(ref))
    nanb = bits.copy()
    nanb[1] = 0x7FC0
    assert compare(nanb, ref).n_fail == 1
    # 100.0 +- 2 bf16 steps is 1.0 away: inside the ulp clause, outside 2e-2
    far = bits.copy()
    far[2] += 2
    rep = compare(far, ref)
    assert rep.max_ulp == 2 and rep.n_fail == 1 and ABS_TOL == 2e-2 and MAX_ULP == 2


def test_ulp_floor_and_signed_zero():
    a = np.array([0x0000, 0x8000, 0x3F80, 0xBF80], np.uint16)
    b = np.array([0x8000, 0x0000, 0x3F81, 0x3F80], np.uint16)
    assert list(ulp_dist(a, b)) == [0, 0, 1, 2 * 0x3F80]
    # a reference below 2^-16 may miss by many ulps but not by more than 2^-22
    ref = np.array([1e-7])
    g = bits_of_bf16_values(np.array([1e-7 + 2**-23]).astype(np.float32).astype(np.float64))
    g = bits_of_bf16_values(bf16_rne(bits_to_f64(g)))
    rep = compare(g, ref)
    assert rep.ok and rep.n_fail_unfloored == 1


def test_page_worst_row_is_one_step():
    """The pages' worst numerics row (6.104e-05 absolute) is exactly one bf16
    step for magnitudes in [2^-7, 2^-6)."""
    g = json.load(open(os.path.join(GOLDEN, "tiny_numerics_shape.json")))
    x = 2.0 ** -7
    step = bits_to_f64(bits_of_bf16_values(np.array([x])) + 1)[0] - x
    assert abs(step - g["worst_max_abs"]) / step < 1e-3


def test_f32_instantiation_close_to_f64(oracle):
    from paged_attention_decode_05_amd.workload import tiny
    case = tiny()
    a, la = oracle.decode(case, "f64")
    b, lb = oracle.decode(case, "f32")
    rep = compare(bits_of_bf16_values(bf16_rne(b)), a)
    assert rep.ok and rep.max_ulp <= 1, str(rep)
    assert np.abs(la - lb).max() < 1e-4


def test_thread_count_does_not_change_bits(oracle):
    from paged_attention_decode_05_amd.workload import tiny
    case = tiny()
    oracle.set_threads(1)
    a, la = oracle.decode(case, "f64")
    oracle.set_threads(max(2, os.cpu_count() or 2))
    b, lb = oracle.decode(case, "f64")
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_oracle_rejects_bad_page(oracle):
    from oracle.oracle import OracleError
    from paged_attention_decode_05_amd.workload import tiny
    case = tiny()
    case.block_table = case.block_table.clone()
    case.block_table[7, 3] = case.num_pages      # out of the pool
    with pytest.raises(OracleError):
        oracle.decode(case)
