"""Pins for the oracle's token-gated causal GQA attention (no GPU)."""
import numpy as np
import pytest
import torch

from oracle import FLT_MIN, ref_attn, ref_attn_varlen
from tests._fixtures import load, sym


def _rand(seed, n=24, hq=4, hkv=2, dh=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, hq, dh)) * 0.5
    k = rng.standard_normal((n, hkv, dh)) * 0.5
    v = rng.standard_normal((n, hkv, dh))
    g = rng.uniform(0.05, 1.0, n)
    return q, k, v, g, np.arange(n)


def test_attn_hand_derived_closed_form():
    fx = load("attn_closed_form.json")
    o, lse = ref_attn(np.array(sym(fx["q"])), np.array(sym(fx["k"])), np.array(sym(fx["v"])),
                      np.array(sym(fx["g"])), np.array(fx["pos"]))
    np.testing.assert_allclose(o, sym(fx["expected_o"]), atol=1e-14)
    np.testing.assert_allclose(lse, sym(fx["expected_lse"]), atol=1e-14)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (6, 1)])
def test_attn_with_unit_gates_is_standard_causal_gqa_attention(hq, hkv):
    q, k, v, _, pos = _rand(1, hq=hq, hkv=hkv)
    o, _ = ref_attn(q, k, v, np.ones(len(pos)), pos)
    group = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attn_equals_weights_multiplied_by_gate_then_renormalised():
    # The paper's Figure 1(c) form: causal softmax weights, each multiplied by
    # its key's g_j, renormalised per query.
    q, k, v, g, pos = _rand(2)
    o, _ = ref_attn(q, k, v, g, pos)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    n, hq, dh = q.shape
    group = hq // k.shape[1]
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    tg = torch.from_numpy(g)
    for h in range(hq):
        s = (tq[:, h] @ tk[:, h // group].T) / dh ** 0.5
        a = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=1)
        a = a * tg[None, :]
        a = a / a.sum(dim=1, keepdim=True)
        np.testing.assert_allclose(o[:, h], (a @ tv[:, h // group]).numpy(), rtol=1e-12, atol=1e-12)


def test_attn_zero_queries_give_gate_weighted_prefix_means():
    # With q = 0 every logit is 0, so o_i = sum_{j<=i} g_j v_j / sum_{j<=i} g_j
    # and lse_i = ln(sum_{j<=i} g_j); GQA heads 0,1 read KV head 0, heads 2,3 KV head 1.
    _, k, v, g, pos = _rand(3)
    q = np.zeros((len(pos), 4, 16))
    o, lse = ref_attn(q, k, v, g, pos)
    cg = np.cumsum(g)
    for h in range(4):
        want = np.cumsum(g[:, None] * v[:, h // 2], axis=0) / cg[:, None]
        np.testing.assert_allclose(o[:, h], want, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[h], np.log(cg), rtol=1e-12, atol=1e-12)


def test_attn_constant_gate_is_shift_invariant():
    q, k, v, _, pos = _rand(4)
    o1, lse1 = ref_attn(q, k, v, np.ones(len(pos)), pos)
    o2, lse2 = ref_attn(q, k, v, np.full(len(pos), 0.37), pos)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse1 + np.log(0.37), rtol=1e-12, atol=1e-12)


def test_attn_first_query_returns_its_own_value_and_single_token():
    q, k, v, g, pos = _rand(5)
    o, _ = ref_attn(q, k, v, g, pos)
    np.testing.assert_array_equal(o[0], v[0, [0, 0, 1, 1]])
    o1, lse1 = ref_attn(q[:1], k[:1], v[:1], g[:1], pos[:1])
    np.testing.assert_array_equal(o1[0], v[0, [0, 0, 1, 1]])


def test_attn_gate_at_flt_min_removes_the_key():
    q, k, v, g, pos = _rand(6)
    g = g.copy()
    g[3] = FLT_MIN
    o, _ = ref_attn(q, k, v, g, pos)
    keep = np.array([i for i in range(len(pos)) if i != 3])
    o_drop, _ = ref_attn(q[keep], k[keep], v[keep], g[keep], pos[keep])
    np.testing.assert_allclose(o[keep], o_drop, rtol=1e-12, atol=1e-12)


def test_attn_zero_gate_is_clamped_not_nan():
    q, k, v, g, pos = _rand(7)
    g0 = g.copy()
    g0[0] = 0.0
    gm = g.copy()
    gm[0] = FLT_MIN
    o0, l0 = ref_attn(q, k, v, g0, pos)
    om, lm = ref_attn(q, k, v, gm, pos)
    assert np.all(np.isfinite(o0)) and np.all(np.isfinite(l0))
    np.testing.assert_array_equal(o0, om)


def test_attn_causal_on_original_positions():
    # Kept tokens sit at scattered, ascending prompt positions: the mask on
    # positions equals the causal mask on the compacted index.
    q, k, v, g, _ = _rand(8)
    pos = np.sort(np.random.default_rng(8).choice(10000, size=24, replace=False))
    o1, l1 = ref_attn(q, k, v, g, pos)
    o2, l2 = ref_attn(q, k, v, g, np.arange(24))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_attn_varlen_is_per_prompt():
    q, k, v, g, _ = _rand(9, n=30)
    cu = np.array([0, 11, 12, 30])
    pos = np.concatenate([np.arange(11) * 3, [5], np.arange(18) + 100])
    o, lse = ref_attn_varlen(q, k, v, g, pos, cu)
    for b in range(3):
        a, e = cu[b], cu[b + 1]
        ob, lb = ref_attn(q[a:e], k[a:e], v[a:e], g[a:e], pos[a:e])
        np.testing.assert_array_equal(o[a:e], ob)
        np.testing.assert_array_equal(lse[:, a:e], lb)


def test_attn_row_subset_equals_full_rows():
    q, k, v, g, pos = _rand(10, n=40)
    o, lse = ref_attn(q, k, v, g, pos)
    rows = np.array([0, 7, 39, 12])
    os_, ls = ref_attn(q, k, v, g, pos, rows=rows)
    np.testing.assert_array_equal(os_, o[rows])
    np.testing.assert_array_equal(ls, lse[:, rows])


def _sdpa_causal(q, k, v, hq, hkv):
    group = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(1, 0, 2).numpy()


def test_attn_without_gate_is_standard_causal_gqa_attention():
    # Full-context layers: no gate at all is torch's causal attention.
    q, k, v, _, pos = _rand(11, hq=6, hkv=2)
    o, _ = ref_attn(q, k, v, None, pos)
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, 6, 2), rtol=1e-12, atol=1e-12)


def test_attn_zero_head_gain_switches_the_gate_off_per_head():
    q, k, v, g, pos = _rand(12, hq=4, hkv=2)
    gain = np.array([0.0, 1.0, 0.0, 1.0])
    o, lse = ref_attn(q, k, v, g, pos, head_gain=gain)
    plain = _sdpa_causal(q, k, v, 4, 2)
    gated, gated_lse = ref_attn(q, k, v, g, pos)
    for h in (0, 2):
        np.testing.assert_allclose(o[:, h], plain[:, h], rtol=1e-12, atol=1e-12)
    for h in (1, 3):
        np.testing.assert_allclose(o[:, h], gated[:, h], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[h], gated_lse[h], rtol=1e-13, atol=1e-13)


def test_attn_head_gain_two_equals_squared_gate():
    # gamma * ln g = ln g^gamma: gain 2 on g is gain 1 on g^2 (g^2 stays above FLT_MIN here).
    q, k, v, g, pos = _rand(13, hq=4, hkv=4)
    o2, lse2 = ref_attn(q, k, v, g, pos, head_gain=np.full(4, 2.0))
    osq, lsesq = ref_attn(q, k, v, g * g, pos)
    np.testing.assert_allclose(o2, osq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lsesq, rtol=1e-12, atol=1e-12)


def test_attn_varlen_passes_gain_and_missing_gate_per_prompt():
    q, k, v, g, _ = _rand(14, n=30, hq=2, hkv=1)
    cu = np.array([0, 11, 11, 30])
    pos = np.concatenate([np.arange(11), np.arange(19)])
    gain = np.array([0.5, 1.5])
    o, lse = ref_attn_varlen(q, k, v, None, pos, cu, head_gain=gain)
    for a, e in ((0, 11), (11, 30)):
        ob, lb = ref_attn(q[a:e], k[a:e], v[a:e], np.ones(e - a), pos[a:e])
        np.testing.assert_allclose(o[a:e], ob, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:e], lb, rtol=1e-13, atol=1e-13)
