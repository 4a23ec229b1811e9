"""Property pins for the oracle, explored with hypothesis (no GPU).

Each property follows from the mathematics of the step, not from the
oracle's own formula, so that a dropped term, a wrong sign or a swapped index
in the oracle fails one of them:
  - select: the O(N^2) rank definition on score alphabets full of ties,
    NaNs, signed zeros and infinities;
  - RoPE: rotations compose additively in the position and keep every pair's
    norm;
  - attention: with the causal mask taken from position values, relabelling
    the tokens (a joint permutation of every row) only permutes the output.
"""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import ref_attn, ref_rope, ref_select
from tests.test_oracle_select import brute_force_select

ALPHABETS = {
    "ties": [0.0, 0.25, 0.5, 0.75, 1.0],
    "specials": [float("nan"), -0.0, 0.0, float("inf"), float("-inf"), 1.0, -1.0],
    "saturated": [1.0, 1.0, 1.0, 0.999, 0.5],
}


@settings(max_examples=150, deadline=None)
@given(data=st.data(), alphabet=st.sampled_from(sorted(ALPHABETS)))
def test_select_equals_the_rank_definition(data, alphabet):
    n = data.draw(st.integers(1, 48), label="n")
    q = data.draw(st.integers(0, n), label="q_len")
    k = data.draw(st.integers(q, n + 4), label="k")
    g = np.array(data.draw(st.lists(st.sampled_from(ALPHABETS[alphabet]), min_size=n, max_size=n)),
                 dtype=np.float32)
    np.testing.assert_array_equal(ref_select(g, k, q), brute_force_select(g, k, q))


@settings(max_examples=60, deadline=None)
@given(p1=st.integers(0, 70000), p2=st.integers(0, 70000), seed=st.integers(0, 2**31 - 1),
       half=st.sampled_from([4, 8, 32, 64]))
def test_rope_rotations_compose_and_keep_pair_norms(p1, p2, seed, half):
    dh = 2 * half
    x = np.random.default_rng(seed).standard_normal((1, 2, dh))
    base = 1e6
    once = ref_rope(ref_rope(x, np.array([p1]), base), np.array([p2]), base)
    direct = ref_rope(x, np.array([p1 + p2]), base)
    # Angles up to ~1.4e5 rad: fp64 keeps them to ~1e-11, so the rotated values agree to 1e-9.
    np.testing.assert_allclose(once, direct, rtol=0, atol=1e-9)
    def pair_norms(y):
        return np.hypot(y[..., :half], y[..., half:])
    np.testing.assert_allclose(pair_norms(direct), pair_norms(x), rtol=1e-12, atol=1e-12)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), n=st.integers(1, 20), heads=st.sampled_from([(2, 1), (4, 2), (2, 2)]))
def test_attn_relabelling_the_tokens_only_permutes_the_output(seed, n, heads):
    hq, hkv = heads
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, hq, 8))
    k = rng.standard_normal((n, hkv, 8))
    v = rng.standard_normal((n, hkv, 8))
    g = rng.uniform(1e-3, 1.0, n)
    pos = rng.choice(10 * n + 1, size=n, replace=False)  # distinct positions, in any order
    o, lse = ref_attn(q, k, v, g, pos)
    perm = rng.permutation(n)
    op, lp = ref_attn(q[perm], k[perm], v[perm], g[perm], pos[perm])
    np.testing.assert_allclose(op, o[perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lp, lse[:, perm], rtol=1e-12, atol=1e-12)
