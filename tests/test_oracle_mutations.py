"""RED-first: every planted mistake in the oracle must fail at least one pin.

The mistakes are compiled into copies of the oracle (ORACLE_MUTATION=k) on
the CPU; the shipped build carries none.  This is the pages' practice of
perturbing the code under test and showing the gate turns red [vllm.cpp
kernel matrix: RED-first mutation proofs in several rows].
"""
import os

import pytest

import oracle_pins
from oracle import build as obuild
from oracle.oracle import Oracle

MUTATIONS = {
    1: "window one key short",
    2: "interleaved GQA head map",
    3: "slot mirrored inside a page",
    4: "W_UK read as [j][d]",
    5: "lse without the max",
    6: "merge weight without l_j",
    7: "softmax scale dropped",
    8: "MLA value row shifted",
    9: "MLA rope term dropped",
    10: "split partitions counted from key 0",
    11: "KV insert with page and offset swapped",
    12: "MLA insert with the rope part first",
    13: "multi-query causal limit one key too far",
    14: "E4M3 exponent bias 8",
    15: "FP8 K and V scales swapped",
    16: "f32-pool V rows one token late",
    17: "FP8 MLA block exponent rounded down",
    18: "FP8 MLA block scale 2^(byte - 128)",
}


@pytest.mark.parametrize("k", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, k):
    lib = obuild.build(mutation=k, out=os.path.join(tmp_path, f"libpa_oracle_m{k}.so"))
    o = Oracle(lib)
    assert o.mutation == k
    res = oracle_pins.run_all(o)
    failed = [n for n, r in res.items() if r is not None]
    assert failed, f"mutation {k} ({MUTATIONS[k]}) passed every pin"


# Mistakes planted in the Python-level MLA multi-query composition: the
# method's source with one substitution, bound to the shipped oracle.
MULTI_MLA_MUTATIONS = {
    "causal limit one key short": ("(n - S + 1 + s).clamp", "(n - S + s).clamp"),
    "queries taken in reverse order": ("q4n[:, s]", "q4n[:, S - 1 - s]"),
    "mask applied when not causal": ("if causal:", "if True:"),
}


@pytest.mark.parametrize("name", sorted(MULTI_MLA_MUTATIONS))
def test_mla_multi_mutation_is_caught(oracle, name):
    import copy
    import inspect
    import textwrap
    import types

    import numpy as np
    import torch

    old, new = MULTI_MLA_MUTATIONS[name]
    src = inspect.getsource(Oracle.mla_multi)
    assert src.count(old) == 1
    ns = {"np": np, "torch": torch, "copy": copy}
    exec(textwrap.dedent(src.replace(old, new)), ns)   # noqa: S102 -- our own source
    o = copy.copy(oracle)
    o.mla_multi = types.MethodType(ns["mla_multi"], o)
    with pytest.raises(AssertionError):
        oracle_pins.mla_multi_bruteforce(o)
