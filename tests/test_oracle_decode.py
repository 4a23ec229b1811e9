"""Pins for the oracle's decode attention over the compact KV cache (no GPU)."""
import numpy as np
import torch

from oracle import ref_attn, ref_decode


def _cache(seed, lens, hq=4, hkv=2, dh=16):
    rng = np.random.default_rng(seed)
    total = int(sum(lens))
    q = rng.standard_normal((len(lens), hq, dh)) * 0.5
    k = rng.standard_normal((total, hkv, dh)) * 0.5
    v = rng.standard_normal((total, hkv, dh))
    g = rng.uniform(0.01, 1.0, total)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, g, cu


def test_decode_without_gate_is_torch_attention_of_one_query():
    q, k, v, _, cu = _cache(1, [37], hq=6, hkv=3)
    o, _ = ref_decode(q, k, v, None, cu)
    tq = torch.from_numpy(q).permute(1, 0, 2)                                   # [hq, 1, dh]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(2, dim=0)       # [hq, n, dh]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(2, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-12)


def test_decode_equals_the_last_row_of_gated_prefill_attention():
    # The new token's query against the cache of everything before it and itself
    # is the last row of the causal gated attention over the whole sequence.
    rng = np.random.default_rng(2)
    n, hq, hkv, dh = 29, 4, 2, 16
    q = rng.standard_normal((n, hq, dh)) * 0.5
    k = rng.standard_normal((n, hkv, dh)) * 0.5
    v = rng.standard_normal((n, hkv, dh))
    g = rng.uniform(0.01, 1.0, n)
    gain = np.array([1.0, 0.5, 2.0, 0.0])
    wo, wl = ref_attn(q, k, v, g, np.arange(n) * 2, head_gain=gain)
    o, lse = ref_decode(q[n - 1:n], k, v, g, np.array([0, n]), head_gain=gain)
    np.testing.assert_allclose(o[0], wo[n - 1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0], wl[:, n - 1], rtol=1e-12, atol=1e-12)


def test_decode_single_key_returns_its_value_and_empty_cache_gives_zero():
    q, k, v, g, cu = _cache(3, [1, 0, 5], hq=2, hkv=1)
    o, lse = ref_decode(q, k, v, g, cu)
    np.testing.assert_array_equal(o[0], np.repeat(v[0:1, 0, :], 2, axis=0))
    np.testing.assert_array_equal(o[1], 0.0)
    assert np.all(lse[1] == -np.inf)


def test_decode_gain_two_equals_squared_gate():
    q, k, v, g, cu = _cache(4, [17, 9])
    o2, l2 = ref_decode(q, k, v, g, cu, head_gain=np.full(4, 2.0))
    osq, lsq = ref_decode(q, k, v, g * g, cu)
    np.testing.assert_allclose(o2, osq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, lsq, rtol=1e-12, atol=1e-12)
