"""Pins for the oracle's upper-layer dense work: projections and the SwiGLU MLP (no GPU)."""
import json
import os

import numpy as np
import torch

from oracle import ref_linear, ref_mlp, ref_swiglu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_linear_equals_brute_force_sums_on_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-5, 6, (7, 5)).astype(np.float64)
    w = rng.integers(-5, 6, (4, 5)).astype(np.float64)
    r = rng.integers(-5, 6, (7, 4)).astype(np.float64)
    want = np.zeros((7, 4))
    for i in range(7):
        for j in range(4):
            acc = r[i, j]
            for t in range(5):
                acc += x[i, t] * w[j, t]
            want[i, j] = acc
    assert np.array_equal(ref_linear(x, w, r), want)  # small integers: exact
    assert np.array_equal(ref_linear(x, w), want - r)


def test_linear_identity_weight_and_bf16_inputs_read_exactly():
    x = torch.randn(9, 6).to(torch.bfloat16)
    y = ref_linear(x, np.eye(6))
    assert np.array_equal(y, x.double().numpy())


def test_swiglu_hand_derived_closed_form():
    with open(os.path.join(GOLDEN, "swiglu_closed_form.json")) as f:
        c = json.load(f)
    got = ref_swiglu(np.array(c["x"]), np.array(c["w_gate"]), np.array(c["w_up"]))
    np.testing.assert_allclose(got, np.array(c["out"]), rtol=1e-15, atol=0)


def test_swiglu_limits():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 8))
    wu = rng.standard_normal((3, 8))
    # SiLU(0) = 0: zero gate weights switch every unit off.
    assert np.all(ref_swiglu(x, np.zeros((3, 8)), wu) == 0.0)
    # SiLU(z) -> z for large z and -> 0 for very negative z.
    wg = np.zeros((3, 8))
    wg[:, 0] = 1.0
    xs = x.copy()
    xs[:, 0] = 60.0
    np.testing.assert_allclose(ref_swiglu(xs, wg, wu), 60.0 * (xs @ wu.T), rtol=1e-12)
    xs[:, 0] = -60.0
    assert np.max(np.abs(ref_swiglu(xs, wg, wu))) < 1e-20


def test_mlp_matches_torch_functional_in_fp64():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(11, 16, generator=g, dtype=torch.float64)
    wg = torch.randn(24, 16, generator=g, dtype=torch.float64)
    wu = torch.randn(24, 16, generator=g, dtype=torch.float64)
    wd = torch.randn(16, 24, generator=g, dtype=torch.float64)
    r = torch.randn(11, 16, generator=g, dtype=torch.float64)
    F = torch.nn.functional
    want = F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd) + r
    np.testing.assert_allclose(ref_mlp(x, wg, wu, wd, r), want.numpy(), rtol=1e-12, atol=1e-12)
