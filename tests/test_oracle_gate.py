"""Pins for the oracle's gate MLP (closed forms and invariants, no GPU)."""
import math

import numpy as np
import torch

from oracle import ref_gate
from tests._fixtures import load, sym


def test_gate_hand_derived_closed_form():
    fx = load("gate_closed_form.json")
    g, s = ref_gate(np.array(sym(fx["h"])), np.array(sym(fx["w1"])), np.array(sym(fx["b1"])),
                    np.array(sym(fx["w2"])), sym(fx["b2"]))
    np.testing.assert_allclose(s, sym(fx["expected_s"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(g, sym(fx["expected_g"]), rtol=0, atol=1e-15)


def test_gate_zero_weights_gives_sigmoid_of_output_bias():
    # W1 = 0 and b1 = 0 make every hidden unit 0 (SiLU(0) = 0), so s = b2 and
    # g = sigmoid(ln 3) = 3/4 for every token whatever h is.
    rng = np.random.default_rng(0)
    h = rng.standard_normal((7, 16))
    g, s = ref_gate(h, np.zeros((4, 16)), np.zeros(4), rng.standard_normal(4), math.log(3.0))
    np.testing.assert_allclose(s, math.log(3.0), atol=1e-15)
    np.testing.assert_allclose(g, 0.75, atol=1e-15)


def test_gate_single_unit_silu_values():
    # One hidden unit, identity-like weights: s = SiLU(x) with SiLU(x) = x*sigmoid(x).
    # SiLU(ln 3) = (3/4) ln 3, SiLU(-ln 3) = -(1/4) ln 3, SiLU(0) = 0.
    x = np.array([[math.log(3.0)], [-math.log(3.0)], [0.0]])
    _, s = ref_gate(x, np.ones((1, 1)), np.zeros(1), np.ones(1), 0.0)
    np.testing.assert_allclose(s, [0.75 * math.log(3.0), -0.25 * math.log(3.0), 0.0], atol=1e-15)


def test_gate_hidden_unit_permutation_invariance():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((9, 12))
    w1 = rng.standard_normal((5, 12))
    b1 = rng.standard_normal(5)
    w2 = rng.standard_normal(5)
    perm = rng.permutation(5)
    g0, s0 = ref_gate(h, w1, b1, w2, 0.3)
    g1, s1 = ref_gate(h, w1[perm], b1[perm], w2[perm], 0.3)
    np.testing.assert_allclose(s1, s0, rtol=1e-13, atol=1e-13)
    # A mis-paired output weight is caught: rolling w2 alone changes the score.
    _, s2 = ref_gate(h, w1, b1, np.roll(w2, 1), 0.3)
    assert np.max(np.abs(s2 - s0)) > 1e-3


def test_gate_token_permutation_equivariance():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((11, 8))
    w1 = rng.standard_normal((3, 8))
    w2 = rng.standard_normal(3)
    perm = rng.permutation(11)
    g0, _ = ref_gate(h, w1, None, w2, -0.1)
    g1, _ = ref_gate(h[perm], w1, None, w2, -0.1)
    np.testing.assert_array_equal(g1, g0[perm])


def test_gate_extreme_inputs_stay_finite_and_bounded():
    # SiLU tends to 0 for a -> -inf and to a for a -> +inf; sigmoid saturates.
    h = np.array([[1e4], [-1e4]])
    g, s = ref_gate(h, np.ones((1, 1)), np.zeros(1), np.ones(1), 0.0)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(s))
    np.testing.assert_allclose(s, [1e4, 0.0], atol=1e-12)
    np.testing.assert_allclose(g, [1.0, 0.5], atol=1e-15)


def test_gate_reads_bf16_tensors_exactly():
    t = torch.tensor([[1.5, -2.25]], dtype=torch.bfloat16)
    w1 = torch.tensor([[1.0, 1.0]], dtype=torch.bfloat16)
    _, s = ref_gate(t, w1, None, np.ones(1), 0.0)
    a = -0.75
    np.testing.assert_allclose(s, [a / (1.0 + math.exp(-a))], atol=1e-15)
