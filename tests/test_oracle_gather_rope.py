"""Pins for the oracle's gather and RoPE (closed forms and invariants, no GPU)."""
import math

import numpy as np
import torch

from oracle import ref_gather, ref_gather_varlen, ref_rope, ref_rope_kv


def test_gather_identity_and_positions():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((10, 6)).astype(np.float32)
    g = rng.random(10).astype(np.float32)
    hk, gk, pos = ref_gather(h, g, np.arange(10))
    np.testing.assert_array_equal(hk, h)
    np.testing.assert_array_equal(gk, g)
    np.testing.assert_array_equal(pos, np.arange(10))


def test_gather_rows_are_bit_copies_of_bf16():
    h = torch.randn(9, 4).to(torch.bfloat16).view(torch.int16).numpy()
    g = np.linspace(0.1, 0.9, 9).astype(np.float32)
    idx = np.array([1, 4, 8])
    hk, gk, pos = ref_gather(h, g, idx)
    np.testing.assert_array_equal(hk, h[[1, 4, 8]])
    np.testing.assert_array_equal(gk, g[[1, 4, 8]])
    np.testing.assert_array_equal(pos, idx)


def test_gather_varlen_offsets_by_prompt_start():
    h = np.arange(20).reshape(20, 1)
    g = np.arange(20, dtype=np.float32)
    hk, gk, pos = ref_gather_varlen(h, g, np.array([0, 3, 1, 2]), np.array([0, 5, 20]), np.array([0, 2, 4]))
    np.testing.assert_array_equal(hk[:, 0], [0, 3, 6, 7])
    np.testing.assert_array_equal(pos, [0, 3, 1, 2])


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((3, 2, 8))
    np.testing.assert_array_equal(ref_rope(x, np.zeros(3, np.int64), 1e6), x)


def test_rope_matches_complex_multiplication():
    # Rotate-half RoPE is multiplication of z_i = x_i + 1j*x_{i+Dh/2} by
    # exp(1j * pos * base**(-2i/Dh)).
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 16))
    pos = np.array([0, 1, 7, 1000, 131071])
    base = 10000.0
    z = x[..., :8] + 1j * x[..., 8:]
    freq = base ** (-np.arange(8) * 2.0 / 16.0)
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(ref_rope(x, pos, base), want, rtol=1e-12, atol=1e-12)


def test_rope_pairs_first_with_middle_dimension():
    # e_0 rotates within the plane (0, Dh/2) at angle pos * 1.
    x = np.zeros((1, 1, 8))
    x[0, 0, 0] = 1.0
    y = ref_rope(x, np.array([3]), 1e6)[0, 0]
    want = np.zeros(8)
    want[0], want[4] = math.cos(3.0), math.sin(3.0)
    np.testing.assert_allclose(y, want, atol=1e-15)


def test_rope_preserves_pair_norms_and_depends_on_relative_position():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    base = 1e6
    rq = ref_rope(q, np.array([900]), base)
    np.testing.assert_allclose(rq[..., :32] ** 2 + rq[..., 32:] ** 2, q[..., :32] ** 2 + q[..., 32:] ** 2,
                               rtol=1e-12)
    d1 = np.sum(ref_rope(q, np.array([900]), base) * ref_rope(k, np.array([850]), base))
    d2 = np.sum(ref_rope(q, np.array([50]), base) * k)
    d3 = np.sum(ref_rope(q, np.array([5050]), base) * ref_rope(k, np.array([5000]), base))
    np.testing.assert_allclose([d1, d3], [d2, d2], rtol=1e-9)


def test_rope_kv_copies_values_and_rotates_keys():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 4, 8))
    k = rng.standard_normal((4, 2, 8))
    v = rng.standard_normal((4, 2, 8))
    pos = np.array([2, 5, 6, 9])
    rq, kc, vc = ref_rope_kv(q, k, v, pos, 1e6)
    np.testing.assert_array_equal(vc, v)
    np.testing.assert_allclose(kc, ref_rope(k, pos, 1e6))
    np.testing.assert_allclose(rq, ref_rope(q, pos, 1e6))
