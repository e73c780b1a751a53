"""The oracle is pinned to facts the pages and mathematics fix, not to itself.

Component pins (softmax, norms, GELU, SiLU, linear, attention, RoPE, argmax) and
model pins (KV-cached == stateless matrix form; closed forms for structured
weights). Every planted mistake in the oracle must break at least one pin.
"""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin_holds(check):
    oracle.set_mutation(0)
    check()


MUTATIONS = {
    1: "GELU without clamp (float exp overflow)",
    2: "GELU without cubic term",
    3: "LayerNorm without mean subtraction",
    4: "attention scale 1/hd",
    5: "cached attention drops the current position",
    6: "RoPE rotates the other way",
    7: "GQA head mapping h mod n_kv",
    8: "argmax ties to highest index",
    9: "stateless mask leaks one future position",
    10: "linear drops the bias",
    11: "bfloat16 K/V rounding truncates",
    12: "8-bit quantization truncates",
    13: "8-bit quantization scale max/128",
    14: "sampling ignores the temperature",
    15: "sampling keeps top_k + 1 candidates",
}


@pytest.mark.parametrize("mut", sorted(MUTATIONS), ids=lambda m: MUTATIONS[m])
def test_planted_mistake_is_caught(mut):
    failed = []
    try:
        oracle.set_mutation(mut)
        for check in P.ALL_CHECKS:
            try:
                check()
            except AssertionError:
                failed.append(check.__name__)
    finally:
        oracle.set_mutation(0)
    assert failed, f"mutation {mut} ({MUTATIONS[mut]}) broke no pin"


def test_gelu_naive_tanh_overflows_to_nan():
    """The page's bug: without the clamp, tanh via exp(2a) in float gives Inf/Inf = NaN."""
    import numpy as np
    oracle.set_mutation(1)
    try:
        g = oracle.gelu(np.array([10.0, 70.0], np.float32))
    finally:
        oracle.set_mutation(0)
    assert np.isnan(g[1])
