"""GPU parity: every stage of the HIP path against the fp64 oracle on the same
seeded inputs (stage by stage, each stage fed the same bytes on both sides).

Bars: select and gather bit-exact; gate g within 1e-2 relative (bf16) and
1e-5 (fp32); attention within 2e-2 max-abs (bf16, fp32 accumulation) and
1e-4 (fp32); RoPE output within one bf16 rounding of the fp64 rotation.
"""
import math

import numpy as np
import pytest
import torch

import learned_token_pruning_03_amd.workloads as W
from oracle import ref_attn, ref_attn_varlen, ref_decode, ref_gate, ref_linear, ref_mlp, ref_swiglu, ref_gather, ref_rope, ref_select, ref_select_varlen

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30)))


# ----------------------------------------------------------------------------- gate
def _gate_case(tg, n, d, hidden, dtype, seed, planted=0.0):
    h = W.hidden_states(n, d, dtype, seed, planted_frac=planted)
    w1, b1, w2, b2 = W.gate_weights(d, hidden, dtype, seed)
    b1 = b1 + torch.linspace(-0.5, 0.5, hidden)  # non-zero bias exercises the b1 path
    g_ref, s_ref = ref_gate(h, w1, b1, w2, 0.25)
    g, s = tg.tg_gate_score(h.to(DEV), w1.to(DEV), b1.to(DEV), w2.to(DEV), 0.25, want_scores=True)
    torch.cuda.synchronize()
    return g.cpu().numpy(), s.cpu().numpy(), g_ref, s_ref


def test_gate_tiny_fp32(gpu_lib):
    sh = W.SHAPES["tiny"]
    _say("gate tiny fp32", sh.n, sh.d, sh.hidden)
    g, s, g_ref, s_ref = _gate_case(gpu_lib, sh.n, sh.d, sh.hidden, torch.float32, W.SEEDS["tiny"])
    assert _rel_err(g, g_ref) <= 1e-5
    np.testing.assert_allclose(s, s_ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("n,d,hidden", [(1000, 256, 64), (777, 512, 128), (300, 2048, 256), (129, 64, 256),
                                        (1, 128, 256), (128, 192, 64)])
def test_gate_bf16_shapes(gpu_lib, n, d, hidden):
    _say("gate bf16", n, d, hidden)
    g, s, g_ref, s_ref = _gate_case(gpu_lib, n, d, hidden, torch.bfloat16, 7 + n)
    err = _rel_err(g, g_ref)
    _say("  max rel err g", err)
    assert err <= 1e-2
    np.testing.assert_allclose(s, s_ref, rtol=1e-3, atol=1e-3)


def test_gate_bf16_qwen_32k_full(gpu_lib):
    sh = W.SHAPES["qwen1p7b_32k"]
    _say("gate bf16 32k full", sh.n, sh.d, sh.hidden)
    g, s, g_ref, s_ref = _gate_case(gpu_lib, sh.n, sh.d, sh.hidden, torch.bfloat16, W.SEEDS["qwen1p7b_32k"],
                                    planted=sh.planted_frac)
    err = _rel_err(g, g_ref)
    _say("  max rel err g", err)
    assert err <= 1e-2


def test_gate_fp32_ragged(gpu_lib):
    _say("gate fp32 ragged")
    g, s, g_ref, s_ref = _gate_case(gpu_lib, 333, 100, 37, torch.float32, 5)
    assert _rel_err(g, g_ref) <= 1e-5


# ----------------------------------------------------------------------------- select
def _sel(tg, g_cpu, k, q, entry="one"):
    """entry "one": tg_select_topk (one workgroup per prompt); "ws": tg_select_topk_ws
    (several workgroups, caller workspace)."""
    g = g_cpu.to(DEV)
    idx = tg.tg_select_topk(g, k, q) if entry == "one" else tg.tg_select_topk_ws(g, k, q)
    torch.cuda.synchronize()
    return idx.cpu().numpy().astype(np.int64)


def _score_vector(kind, n, seed):
    if kind == "uniform":
        return W.random_scores(n, seed)
    if kind == "wide":
        return W.gate_values_wide(n, seed)
    if kind == "tie8":
        return W.tie_storm_scores(n, 8, seed)
    if kind == "equal":
        return torch.full((n,), 0.5, dtype=torch.float32)
    if kind == "saturated":
        g = W.random_scores(n, seed)
        g[torch.arange(n) % 3 == 0] = 1.0
        return g
    if kind == "special":
        g = W.random_scores(n, seed) - 0.5
        g[::7] = float("nan")
        g[1::11] = -0.0
        g[2::11] = 0.0
        g[3::13] = float("-inf")
        g[4::17] = float("inf")
        return g
    raise ValueError(kind)


@pytest.mark.parametrize("entry", ["one", "ws"])
@pytest.mark.parametrize("kind", ["uniform", "wide", "tie8", "equal", "saturated", "special"])
@pytest.mark.parametrize("n,k,q", [(512, 128, 32), (1000, 300, 17), (5000, 999, 0), (4097, 4096, 64),
                                   (70, 64, 64), (64, 100, 10), (3, 2, 1), (2049, 5, 1), (20001, 7000, 5)])
def test_select_bit_exact(gpu_lib, kind, n, k, q, entry):
    g = _score_vector(kind, n, n + k)
    got = _sel(gpu_lib, g, k, q, entry)
    want = ref_select(g.numpy(), k, q)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name,n,k,q,kind", [("qwen1p7b_32k", 32768, 4096, 64, "uniform"),
                                             ("qwen1p7b_32k", 32768, 4096, 64, "tie8"),
                                             ("stack19", 65536, 4096, 64, "uniform"),
                                             ("qwen1p7b_128k", 131072, 8192, 64, "wide"),
                                             ("qwen1p7b_128k", 131072, 8192, 64, "tie8"),
                                             ("long", 200003, 20000, 100, "uniform")])
@pytest.mark.parametrize("entry", ["one", "ws"])
def test_select_full_sizes(gpu_lib, name, n, k, q, kind, entry):
    _say("select", entry, name, n, k, q, kind)
    g = _score_vector(kind, n, 3)
    np.testing.assert_array_equal(_sel(gpu_lib, g, k, q, entry), ref_select(g.numpy(), k, q))


@pytest.mark.parametrize("entry", ["one", "ws"])
def test_select_budget_covers_prompt_and_tail_only(gpu_lib, entry):
    g = W.random_scores(300, 1)
    np.testing.assert_array_equal(_sel(gpu_lib, g, 300, 20, entry), np.arange(300))
    np.testing.assert_array_equal(_sel(gpu_lib, g, 1000, 20, entry), np.arange(300))
    np.testing.assert_array_equal(_sel(gpu_lib, g, 20, 20, entry), np.arange(280, 300))


@pytest.mark.parametrize("doc_extra", [0, 1])
def test_select_ws_at_its_largest_document(gpu_lib, doc_extra):
    """2^24 document tokens: the most the multi-workgroup path takes (8192 chunks,
    each summing up to 8191 chunk counts for its offset); one token more falls back
    to the one-workgroup kernel.  Tie-heavy scores, so the last radix pass and the
    equal-key rule both matter."""
    q = 64
    n = (1 << 24) + doc_extra + q
    _say("select ws largest document", n)
    g = W.tie_storm_scores(n, 8, 5 + doc_extra)
    k = (1 << 20) + q
    got = _sel(gpu_lib, g, k, q, "ws")
    np.testing.assert_array_equal(got, ref_select(g.numpy(), k, q))


def test_select_ws_dirty_workspace_and_unaligned_scores(gpu_lib):
    """The multi-workgroup select clears what it uses: a workspace full of garbage, or
    left over from a longer call, gives the same answer; scores that start off a
    16-byte boundary take the scalar loads."""
    _say("select ws dirty workspace")
    n_big = 40000
    ws = torch.full((gpu_lib.tg_select_topk_workspace_size(n_big),), 0xAB, dtype=torch.uint8, device=DEV)
    for n, k, q, kind, seed in [(40000, 5000, 64, "wide", 1), (9000, 1000, 8, "tie8", 2), (40000, 5000, 64, "uniform", 3)]:
        g = _score_vector(kind, n, seed)
        idx = gpu_lib.tg_select_topk_ws(g.to(DEV), k, q, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_select(g.numpy(), k, q))
    base = _score_vector("uniform", 30001, 4)
    gd = base.to(DEV)[1:]  # 4-byte offset from the allocation
    idx = gpu_lib.tg_select_topk_ws(gd, 3000, 16, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_select(base[1:].numpy(), 3000, 16))


@pytest.mark.parametrize("dirty", [False, True])
@pytest.mark.parametrize("n,k,q", [(4097, 3600, 64), (30001, 27000, 1), (2113, 2000, 0)])
def test_select_ws_nan_threshold_in_a_partial_chunk(gpu_lib, n, k, q, dirty):
    """The kd-th largest document score is a NaN (so T is the key of NaN, 0) and
    the document ends inside a 64-token chunk: the ranking treats the keys past
    the document's end as that same key and must take them back out of every
    count of it (histogram bin 0 of a zero prefix, and the count equal to T).
    The workspace starts clean or full of garbage (this entry clears its
    histogram itself), and the second call reuses what the first left."""
    _say("select ws NaN threshold", n, k, q, "dirty" if dirty else "clean")
    g = W.random_scores(n, 21)
    g[::3] = float("nan")
    g[1::10] = float("nan")
    doc, kd = n - q, k - q
    assert doc % 64 != 0 and int(torch.isnan(g[:doc]).logical_not().sum()) < kd  # the threshold is a NaN
    size = gpu_lib.tg_select_topk_workspace_size(n)
    ws = (torch.full((size,), 0xAB, dtype=torch.uint8, device=DEV) if dirty
          else torch.zeros(size, dtype=torch.uint8, device=DEV))
    for _ in range(2):  # the second call starts from the workspace the first left behind
        idx = gpu_lib.tg_select_topk_ws(g.to(DEV), k, q, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_select(g.numpy(), k, q))


def test_select_varlen_ragged_batch(gpu_lib):
    ns, qs = W.ragged_lengths(8, W.SEEDS["ragged8"])
    ns = ns[:6] + [100, 0]
    qs = qs[:6] + [100, 0]
    k = 256
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    g = W.random_scores(int(cu[-1]), 9)
    want, want_cu = ref_select_varlen(g.numpy(), cu, qs, k)
    idx, cu_kept = gpu_lib.tg_select_topk_varlen(g.to(DEV), torch.from_numpy(cu).to(DEV),
                                                 torch.tensor(qs, dtype=torch.int32, device=DEV), max(ns), k,
                                                 int(want_cu[-1]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cu_kept.cpu().numpy(), want_cu)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


# ----------------------------------------------------------------------------- gate + select in one call
def _gate_select_case(tg, h, w1, b1, w2, b2, k, q, ws=None):
    """tg_gate_select and tg_gate_select_gather against the plain gate on the
    same input (the same g, bit for bit), the oracle's selection on the g they
    wrote (bit-exact) and the oracle's gather of those rows (bit-exact)."""
    hd, w1d, b1d, w2d = h.to(DEV), w1.to(DEV), b1.to(DEV), w2.to(DEV)
    g, idx = tg.tg_gate_select(hd, w1d, b1d, w2d, b2, k, q, workspace=ws)
    g2, idx2, hk, gk, pos = tg.tg_gate_select_gather(hd, w1d, b1d, w2d, b2, k, q, workspace=ws)
    g_plain = tg.tg_gate_score(hd, w1d, b1d, w2d, b2)
    torch.cuda.synchronize()
    g_cpu = g.cpu().numpy()
    np.testing.assert_array_equal(g_cpu.view(np.uint32), g_plain.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(g2.cpu().numpy().view(np.uint32), g_cpu.view(np.uint32))
    want = ref_select(g_cpu, k, q)
    np.testing.assert_array_equal(idx.cpu().numpy().astype(np.int64), want)
    np.testing.assert_array_equal(idx2.cpu().numpy().astype(np.int64), want)
    bits = h.view(torch.int16).numpy() if h.dtype == torch.bfloat16 else h.view(torch.int32).numpy()
    wh, wg, wp = ref_gather(bits, g_cpu, want)
    np.testing.assert_array_equal(hk.cpu().view(torch.int16 if h.dtype == torch.bfloat16 else torch.int32).numpy(), wh)
    np.testing.assert_array_equal(gk.cpu().numpy().view(np.uint32), np.asarray(wg, dtype=np.float32).view(np.uint32))
    np.testing.assert_array_equal(pos.cpu().numpy(), wp)
    return g_cpu


def _counts_clean(ws):
    """The histogram and the arrival counter (first 2049 words) are zero."""
    return int(ws[:2049 * 4].count_nonzero()) == 0


@pytest.mark.parametrize("n,d,hidden,k,q,planted", [
    (1000, 256, 64, 300, 17, 0.0), (5000, 512, 128, 999, 0, 0.05), (4097, 2048, 256, 4096, 64, 0.05),
    (129, 64, 256, 100, 1, 0.0), (300, 2048, 256, 300, 20, 0.0), (300, 2048, 256, 1000, 20, 0.0),
    (300, 2048, 256, 20, 20, 0.0), (3, 64, 64, 2, 1, 0.0), (40000, 256, 256, 5000, 64, 0.05),
    (70001, 128, 256, 4096, 64, 0.05), (32832, 256, 256, 4096, 64, 0.0), (32833, 256, 256, 4096, 64, 0.0),
    (18464, 128, 64, 2000, 32, 0.05), (18465, 128, 64, 2000, 32, 0.05), (24608, 128, 128, 3000, 32, 0.0),
    (24609, 128, 128, 3000, 32, 0.0)])
def test_gate_select_parity(gpu_lib, n, d, hidden, k, q, planted):
    """Ragged row counts against the 128-row gate tiles, budgets that keep the
    whole prompt or only the tail, and documents on both sides of what the
    gate's last workgroup ranks itself (32768, 24576 and 18432 document tokens
    at hidden 256, 128 and 64); longer documents (40000 and 70001 tokens too)
    take the gate and the six-kernel selection."""
    _say("gate_select", n, d, hidden, k, q)
    h = W.hidden_states(n, d, torch.bfloat16, 31 + n, planted_frac=planted)
    w1, b1, w2, _ = W.gate_weights(d, hidden, torch.bfloat16, 31 + n)
    g = _gate_select_case(gpu_lib, h, w1, b1, w2, 0.25, k, q)
    g_ref, _ = ref_gate(h, w1, b1, w2, 0.25)
    assert _rel_err(g, g_ref) <= 1e-2


@pytest.mark.parametrize("b2,dup", [(0.0, 8), (40.0, 1), (-200.0, 1)])
def test_gate_select_ties(gpu_lib, b2, dup):
    """Equal scores: every row repeated `dup` times (equal g), or an output bias
    that saturates the sigmoid to 1.0f, or drives it to 0 -- the lower index
    wins every tie."""
    n, d, hidden, k, q = 8192, 256, 256, 1000, 32
    _say("gate_select ties", b2, dup)
    base = W.hidden_states(n // dup, d, torch.bfloat16, 41)
    h = base.repeat_interleave(dup, dim=0).contiguous() if dup > 1 else base
    w1, b1, w2, _ = W.gate_weights(d, hidden, torch.bfloat16, 41)
    g = _gate_select_case(gpu_lib, h, w1, b1, w2, b2, k, q)
    assert len(np.unique(g)) < n  # ties present


def test_gate_select_reuses_its_workspace(gpu_lib):
    """One workspace across calls of different lengths and budgets: each call
    leaves its counts and arrival counter zero, as the next one needs."""
    _say("gate_select workspace reuse")
    ws = gpu_lib.select_workspace(50000, DEV)
    for n, d, k, q, seed in [(40000, 256, 5000, 64, 1), (1000, 128, 300, 8, 2), (32768, 2048, 4096, 64, 3),
                             (2048, 64, 2048, 16, 4), (9000, 256, 77, 5, 5)]:
        h = W.hidden_states(n, d, torch.bfloat16, seed, planted_frac=0.05)
        w1, b1, w2, _ = W.gate_weights(d, 256, torch.bfloat16, seed)
        _gate_select_case(gpu_lib, h, w1, b1, w2, 0.0, k, q, ws=ws)
        torch.cuda.synchronize()
        assert _counts_clean(ws), "counts and counter not left zero"


def test_gate_select_recounts_a_histogram_that_does_not_add_up(gpu_lib):
    """A workspace whose histogram holds stale counts (arrival counter zero):
    the last workgroup finds that the counts do not add up to the document
    length, counts the keys itself, and still selects exactly."""
    _say("gate_select stale histogram")
    ws = gpu_lib.select_workspace(20000, DEV)
    ws[:8192] = 7  # stale histogram words; the counter (word 2048, bytes 8192..8195) stays zero
    n, d, k, q = 20000, 256, 3000, 40
    h = W.hidden_states(n, d, torch.bfloat16, 51, planted_frac=0.05)
    w1, b1, w2, _ = W.gate_weights(d, 256, torch.bfloat16, 51)
    _gate_select_case(gpu_lib, h, w1, b1, w2, 0.0, k, q, ws=ws)
    torch.cuda.synchronize()
    assert _counts_clean(ws)


def test_gate_select_nan_threshold_with_a_stale_histogram(gpu_lib):
    """Hidden states with NaN rows score NaN, the lowest rank.  With fewer finite
    document scores than the budget, the threshold T is the key of NaN (0), the
    key the ranking also gives to the positions past the document's end in its
    last chunk (the document here ends 56 tokens into it).  A stale histogram
    makes the last workgroup count the top digit from the keys itself; every
    count of key 0 must leave those positions out."""
    n, d, k, q = 20000, 256, 15000, 40
    h = W.hidden_states(n, d, torch.bfloat16, 52)
    h[::2] = float("nan")
    w1, b1, w2, _ = W.gate_weights(d, 256, torch.bfloat16, 52)
    for stale in (False, True):
        _say("gate_select NaN threshold", "stale" if stale else "clean")
        ws = gpu_lib.select_workspace(n, DEV)
        if stale:
            ws[:8192] = 7  # stale histogram words; the arrival counter stays zero
        g = _gate_select_case(gpu_lib, h, w1, b1, w2, 0.0, k, q, ws=ws)
        doc, kd = n - q, k - q
        assert doc % 64 != 0 and int(np.isfinite(g[:doc]).sum()) < kd  # the threshold is a NaN
        torch.cuda.synchronize()
        assert _counts_clean(ws)


def test_gate_select_fp32_tiny(gpu_lib):
    sh = W.SHAPES["tiny"]
    _say("gate_select tiny fp32")
    h = W.hidden_states(sh.n, sh.d, torch.float32, W.SEEDS["tiny"])
    w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, torch.float32, W.SEEDS["tiny"])
    g = _gate_select_case(gpu_lib, h, w1, b1, w2, b2, sh.k, sh.q_len)
    g_ref, _ = ref_gate(h, w1, b1, w2, b2)
    assert _rel_err(g, g_ref) <= 1e-5


@pytest.mark.parametrize("name", ["qwen1p7b_32k", "stack19", "qwen1p7b_128k"])
def test_gate_select_full_sizes(gpu_lib, name):
    """The bench workloads' gate + select at full size: g on every row within
    1e-2 of the oracle's gate (so the 131072-token gate, 1024 workgroups, is
    checked too), idx bit-exact on the g the call wrote."""
    sh = W.SHAPES[name]
    seed = W.SEEDS[name]
    _say("gate_select full size", name, sh.n, sh.k)
    h = W.hidden_states(sh.n, sh.d, sh.dtype, seed, planted_frac=sh.planted_frac)
    w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, sh.dtype, seed)
    g = _gate_select_case(gpu_lib, h, w1, b1, w2, b2, sh.k, sh.q_len)
    g_ref, _ = ref_gate(h, w1, b1, w2, b2)
    err = _rel_err(g, g_ref)
    _say("  max rel err g", err)
    assert err <= 1e-2


# ----------------------------------------------------------------------------- gather
@pytest.mark.parametrize("dtype,n,d,nk", [(torch.bfloat16, 1000, 2048, 333), (torch.float32, 512, 256, 128),
                                          (torch.bfloat16, 32768, 2048, 4096), (torch.bfloat16, 50, 8, 50)])
def test_gather_bit_exact(gpu_lib, dtype, n, d, nk):
    _say("gather", dtype, n, d, nk)
    h = W.hidden_states(n, d, dtype, 11)
    g = W.random_scores(n, 12)
    idx = torch.from_numpy(np.sort(np.random.default_rng(n).choice(n, nk, replace=False)).astype(np.int32))
    hk, gk, pos = gpu_lib.tg_gather(h.to(DEV), g.to(DEV), idx.to(DEV))
    torch.cuda.synchronize()
    wh, wg, wp = ref_gather(h.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(), g.numpy(),
                            idx.numpy())
    np.testing.assert_array_equal(hk.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(),
                                  wh)
    np.testing.assert_array_equal(gk.cpu().numpy(), wg)
    np.testing.assert_array_equal(pos.cpu().numpy(), wp)


def test_gather_out_of_range_index_gives_zero_row(gpu_lib):
    h = W.hidden_states(10, 64, torch.bfloat16, 1).to(DEV)
    g = W.random_scores(10, 1).to(DEV)
    idx = torch.tensor([3, 10, -1, 9], dtype=torch.int32, device=DEV)
    hk, gk, pos = gpu_lib.tg_gather(h, g, idx)
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [3, -1, -1, 9]
    assert torch.all(hk[1:3].float() == 0).item() and gk[1].item() == 0.0
    assert torch.equal(hk[0], h[3]) and torch.equal(hk[3], h[9])


def test_gather_varlen(gpu_lib):
    ns = [700, 5, 1300]
    qs = [10, 5, 64]
    k = 256
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    g = W.random_scores(int(cu[-1]), 4)
    h = W.hidden_states(int(cu[-1]), 2048, torch.bfloat16, 4)
    idx_local, cu_kept = ref_select_varlen(g.numpy(), cu, qs, k)
    hk, gk, pos = gpu_lib.tg_gather_varlen(h.to(DEV), g.to(DEV), torch.from_numpy(idx_local.astype(np.int32)).to(DEV),
                                           torch.from_numpy(cu).to(DEV),
                                           torch.from_numpy(cu_kept.astype(np.int32)).to(DEV), k)
    torch.cuda.synchronize()
    rows = np.concatenate([cu[b] + idx_local[cu_kept[b]:cu_kept[b + 1]] for b in range(3)])
    np.testing.assert_array_equal(hk.cpu().view(torch.int16).numpy(), h.view(torch.int16).numpy()[rows])
    np.testing.assert_array_equal(gk.cpu().numpy(), g.numpy()[rows])
    np.testing.assert_array_equal(pos.cpu().numpy(), idx_local)


# ----------------------------------------------------------------------------- rope
@pytest.mark.parametrize("dtype,n,hq,hkv,dh", [(torch.bfloat16, 4096, 16, 8, 128), (torch.bfloat16, 77, 4, 2, 64),
                                               (torch.float32, 128, 4, 2, 64), (torch.bfloat16, 33, 2, 1, 16)])
def test_rope_kv_parity(gpu_lib, dtype, n, hq, hkv, dh):
    _say("rope", dtype, n, hq, hkv, dh)
    base = 1e6
    max_pos = 131072
    q, k, v = W.qkv(n, hq, hkv, dh, 1.0 / dh, dtype, 21)
    pos = torch.from_numpy(np.sort(np.random.default_rng(n).choice(max_pos, n, replace=False)).astype(np.int32))
    pos[0] = 0
    pos[-1] = max_pos - 1
    table = gpu_lib.tg_rope_table(max_pos, dh, base, DEV)
    qd = q.to(DEV)
    _, kc, vc = gpu_lib.tg_rope_kv(qd, k.to(DEV), v.to(DEV), pos.to(DEV), table)
    torch.cuda.synchronize()
    wq = ref_rope(q, pos.numpy(), base)
    wk = ref_rope(k, pos.numpy(), base)
    tol = 2.0 ** -8 if dtype == torch.bfloat16 else 1e-6
    for got, want in ((qd, wq), (kc, wk)):
        got = got.cpu().double().numpy()
        assert np.all(np.abs(got - want) <= tol * np.abs(want) + 1e-6), float(np.max(np.abs(got - want)))
    assert torch.equal(vc.cpu(), v)


def test_rope_table_matches_fp64_angles(gpu_lib):
    dh, base, max_pos = 128, 1e6, 131072
    t = gpu_lib.tg_rope_table(max_pos, dh, base, DEV).cpu().double().numpy()
    rows = np.array([0, 1, 2, 1000, 65535, 131071])
    theta = np.power(base, -2.0 * np.arange(dh // 2) / dh)
    phi = rows[:, None] * theta[None, :]
    want = np.concatenate([np.cos(phi), np.sin(phi)], axis=1).astype(np.float32).astype(np.float64)
    assert np.max(np.abs(t[rows] - want)) <= 1.2e-7


# ----------------------------------------------------------------------------- attention
def _attn_inputs(n, hq, hkv, dh, dtype, seed, gkind="uniform", pos_kind="sparse"):
    q, k, v = W.qkv(n, hq, hkv, dh, 1.0 / dh, dtype, seed)
    if gkind == "uniform":
        g = W.random_scores(n, seed)
    elif gkind == "wide":
        g = W.gate_values_wide(n, seed)
    elif gkind == "edge":
        g = W.random_scores(n, seed)
        g[::5] = 0.0
        g[1::5] = 1.0
        g[2::7] = 1e-30
    else:
        raise ValueError(gkind)
    if pos_kind == "sparse":
        pos = np.sort(np.random.default_rng(seed).choice(max(4 * n, 1), n, replace=False)).astype(np.int32)
    else:
        pos = np.arange(n, dtype=np.int32)
    return q, k, v, g, torch.from_numpy(pos)


def _run_attn(tg, q, k, v, g, pos):
    o, lse = tg.tg_gated_attn(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), pos.to(DEV), want_lse=True)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def test_attn_tiny_fp32(gpu_lib):
    sh = W.SHAPES["tiny"]
    _say("attn tiny fp32")
    q, k, v, g, pos = _attn_inputs(sh.k, sh.hq, sh.hkv, sh.dh, torch.float32, W.SEEDS["tiny"])
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    wo, wl = ref_attn(q, k, v, g, pos.numpy())
    assert np.max(np.abs(o - wo)) <= 1e-4
    assert np.max(np.abs(lse - wl)) <= 1e-4


@pytest.mark.parametrize("n,hq,hkv,dh,gkind", [(300, 4, 2, 64, "uniform"), (300, 16, 8, 128, "wide"),
                                               (1, 4, 4, 128, "uniform"), (63, 8, 1, 128, "edge"),
                                               (129, 2, 2, 64, "edge"), (640, 6, 3, 128, "uniform"),
                                               (257, 16, 8, 128, "uniform")])
def test_attn_bf16_shapes(gpu_lib, n, hq, hkv, dh, gkind):
    _say("attn bf16", n, hq, hkv, dh, gkind)
    q, k, v, g, pos = _attn_inputs(n, hq, hkv, dh, torch.bfloat16, n + hq, gkind)
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    wo, wl = ref_attn(q, k, v, g, pos.numpy())
    err = float(np.max(np.abs(o - wo)))
    _say("  max abs err o", err, "lse", float(np.max(np.abs(lse - wl))))
    assert err <= 2e-2
    assert np.max(np.abs(lse - wl)) <= 1e-3


def _rising_logit_inputs(n, hq, hkv, dh, seed, jump_at, jump=250.0):
    """Q/K whose logits spread over several units and grow along the prompt
    (key j scaled by 1 + 3j/n), plus one key at jump_at sharing a direction
    with every query so that its logit is about `jump` (natural units) for
    all later queries.  jump = 250 puts it more than 128 base-2 units above
    every earlier key (past the fp32 range of 2^x); jump = 90 puts it 64 to
    128 units above them (weights finite but past 2^64).  Either way the
    kernel's reference maximum must move."""
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(n, hq, dh, generator=gen, dtype=torch.float64) * 2.0
    k = torch.randn(n, hkv, dh, generator=gen, dtype=torch.float64) * 2.0
    v = torch.randn(n, hkv, dh, generator=gen, dtype=torch.float64) / dh ** 0.5
    k *= (1.0 + 3.0 * torch.arange(n, dtype=torch.float64) / n)[:, None, None]
    u = torch.zeros(dh, dtype=torch.float64)
    u[: dh // 2] = 1.0
    q += 2.0 * u
    k[jump_at] = jump * dh ** 0.5 / (2.0 * float(u @ u)) * u
    pos = torch.arange(n, dtype=torch.int32)
    bf = lambda x: x.to(torch.bfloat16).contiguous()
    return bf(q), bf(k), bf(v), W.random_scores(n, seed), pos


@pytest.mark.parametrize("n,hq,hkv,dh,jump_at,jump", [(1000, 4, 2, 128, 517, 250.0), (700, 4, 4, 64, 130, 250.0),
                                                    (1000, 4, 2, 128, 517, 90.0)])
def test_attn_bf16_rising_logits(gpu_lib, n, hq, hkv, dh, jump_at, jump):
    _say("attn bf16 rising logits", n, hq, hkv, dh, jump_at, jump)
    q, k, v, g, pos = _rising_logit_inputs(n, hq, hkv, dh, 77 + n, jump_at, jump)
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    wo, wl = ref_attn(q, k, v, g, pos.numpy())
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err = float(np.max(np.abs(o - wo)))
    _say("  max abs err o", err, "lse", float(np.max(np.abs(lse - wl))))
    assert err <= 2e-2
    # lse reaches ~400 here: fp32 keeps it to a few 1e-5.
    assert np.max(np.abs(lse - wl)) <= 1e-3


def test_attn_bf16_rising_logits_streamed_bias(gpu_lib):
    """The same redo path in the streamed-bias form (8300 keys, past the LDS
    bias table at head dim 128), on sampled query rows that include the rows
    around the planted key."""
    n, jump_at = 8300, 5003
    _say("attn bf16 rising logits, streamed bias", n)
    q, k, v, g, pos = _rising_logit_inputs(n, 2, 1, 128, 91, jump_at)
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    rows = np.unique(np.concatenate([_sample_rows(n, 9, count=40), np.arange(jump_at - 2, jump_at + 3)]))
    wo, wl = ref_attn(q, k, v, g, pos.numpy(), rows=rows)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err = float(np.max(np.abs(o[rows] - wo)))
    _say("  max abs err o", err)
    assert err <= 2e-2
    assert np.max(np.abs(lse[:, rows] - wl)) <= 1e-3


@pytest.mark.parametrize("n,hq,hkv,dh", [(200, 4, 2, 64), (77, 2, 1, 128)])
def test_attn_fp32_shapes(gpu_lib, n, hq, hkv, dh):
    q, k, v, g, pos = _attn_inputs(n, hq, hkv, dh, torch.float32, n, "edge")
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    wo, wl = ref_attn(q, k, v, g, pos.numpy())
    assert np.max(np.abs(o - wo)) <= 1e-4
    assert np.max(np.abs(lse - wl)) <= 1e-4


def _sample_rows(n, seed, count=192):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, n // 2, n - 129, n - 128, n - 65, n - 64, n - 2, n - 1]
    rows = np.unique(np.concatenate([[r for r in fixed if 0 <= r < n], rng.choice(n, count, replace=False)]))
    return rows


@pytest.mark.parametrize("name,gkind", [("qwen1p7b_32k", "uniform"), ("qwen1p7b_128k", "wide")])
def test_attn_bf16_full_size_sampled_rows(gpu_lib, name, gkind):
    sh = W.SHAPES[name]
    _say("attn full size", name, sh.k)
    q, k, v, g, pos = _attn_inputs(sh.k, sh.hq, sh.hkv, sh.dh, torch.bfloat16, W.SEEDS[name], gkind)
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    rows = _sample_rows(sh.k, 5)
    wo, wl = ref_attn(q, k, v, g, pos.numpy(), rows=rows)
    err = float(np.max(np.abs(o[rows] - wo)))
    _say("  max abs err o", err)
    assert err <= 2e-2
    assert np.max(np.abs(lse[:, rows] - wl)) <= 1e-3
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("n,dh", [(8300, 128), (16500, 64)])
def test_attn_bf16_past_the_lds_bias_table(gpu_lib, n, dh):
    """Kept counts above the LDS bias table (8192 keys at head dim 128, 16384 at
    64) take the kernel's streamed-bias form (gate values copied tile by tile)."""
    _say("attn long prompt", n, dh)
    q, k, v, g, pos = _attn_inputs(n, 2, 1, dh, torch.bfloat16, 31, "wide")
    o, lse = _run_attn(gpu_lib, q, k, v, g, pos)
    rows = _sample_rows(n, 6, count=48)
    wo, wl = ref_attn(q, k, v, g, pos.numpy(), rows=rows)
    err = float(np.max(np.abs(o[rows] - wo)))
    _say("  max abs err o", err)
    assert err <= 2e-2
    assert np.max(np.abs(lse[:, rows] - wl)) <= 1e-3


def _gains(hq, seed):
    gain = np.random.default_rng(seed).uniform(0.0, 2.0, hq).astype(np.float32)
    gain[0] = 0.0  # one head with the gate switched off
    return torch.from_numpy(gain)


@pytest.mark.parametrize("dtype,n,hq,hkv,dh", [(torch.bfloat16, 300, 16, 8, 128), (torch.bfloat16, 777, 4, 2, 64),
                                               (torch.float32, 200, 4, 2, 64)])
def test_attn_head_gain(gpu_lib, dtype, n, hq, hkv, dh):
    """Per-head gain on the gate bias (tg_gated_attn_ex)."""
    _say("attn head gain", dtype, n, hq, hkv, dh)
    q, k, v, g, pos = _attn_inputs(n, hq, hkv, dh, dtype, 41, "wide")
    gain = _gains(hq, 41)
    o, lse = gpu_lib.tg_gated_attn(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), pos.to(DEV), want_lse=True,
                                   head_gain=gain.to(DEV))
    torch.cuda.synchronize()
    wo, wl = ref_attn(q, k, v, g, pos.numpy(), head_gain=gain.numpy())
    tol_o, tol_l = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-4, 1e-4)
    assert np.max(np.abs(o.cpu().double().numpy() - wo)) <= tol_o
    assert np.max(np.abs(lse.cpu().double().numpy() - wl)) <= tol_l


def test_attn_head_gain_on_the_streamed_bias_form(gpu_lib):
    n = 8300  # past the LDS bias table at head dim 128
    q, k, v, g, pos = _attn_inputs(n, 2, 1, 128, torch.bfloat16, 42, "wide")
    gain = torch.tensor([0.5, 1.75], dtype=torch.float32)
    o, lse = gpu_lib.tg_gated_attn(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), pos.to(DEV), want_lse=True,
                                   head_gain=gain.to(DEV))
    torch.cuda.synchronize()
    rows = _sample_rows(n, 7, count=48)
    wo, wl = ref_attn(q, k, v, g, pos.numpy(), rows=rows, head_gain=gain.numpy())
    assert np.max(np.abs(o.cpu().double().numpy()[rows] - wo)) <= 2e-2
    assert np.max(np.abs(lse.cpu().double().numpy()[:, rows] - wl)) <= 1e-3


@pytest.mark.parametrize("n,dtype", [(300, torch.bfloat16), (32768, torch.bfloat16), (150, torch.float32)])
def test_attn_without_gate_full_context(gpu_lib, n, dtype):
    """g=None: plain causal GQA attention, as in the layers at or below the selection layer; at
    32768 tokens the full-context shape of the 32k workload."""
    _say("attn no gate", n, dtype)
    hq, hkv, dh = (16, 8, 128) if dtype == torch.bfloat16 else (4, 2, 64)
    q, k, v, _, pos = _attn_inputs(n, hq, hkv, dh, dtype, 43, "uniform", pos_kind="dense")
    o, lse = gpu_lib.tg_gated_attn(q.to(DEV), k.to(DEV), v.to(DEV), None, pos.to(DEV), want_lse=True)
    torch.cuda.synchronize()
    rows = _sample_rows(n, 8, count=64) if n > 4096 else np.arange(n)
    wo, wl = ref_attn(q, k, v, None, pos.numpy(), rows=rows)
    tol_o, tol_l = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-4, 1e-4)
    assert np.max(np.abs(o.cpu().double().numpy()[rows] - wo)) <= tol_o
    assert np.max(np.abs(lse.cpu().double().numpy()[:, rows] - wl)) <= tol_l


def test_attn_varlen_with_head_gain(gpu_lib):
    lens = [256, 1, 100, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    q, k, v, g, _ = _attn_inputs(total, 4, 2, 128, torch.bfloat16, 44, "wide")
    pos = torch.from_numpy(np.concatenate([np.arange(m) * 3 for m in lens]).astype(np.int32))
    gain = _gains(4, 44)
    o, lse = gpu_lib.tg_gated_attn_varlen(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), pos.to(DEV),
                                          torch.from_numpy(cu).to(DEV), max(lens), want_lse=True,
                                          head_gain=gain.to(DEV))
    torch.cuda.synchronize()
    wo, wl = ref_attn_varlen(q, k, v, g, pos.numpy(), cu, head_gain=gain.numpy())
    assert np.max(np.abs(o.cpu().double().numpy() - wo)) <= 2e-2
    assert np.max(np.abs(lse.cpu().double().numpy() - wl)) <= 1e-3


def test_attn_varlen_streamed_bias_with_head_gain(gpu_lib):
    """A packed batch whose longest prompt passes the LDS bias table (9000 keys at
    head dim 128) runs every prompt in the streamed-bias form: ragged lengths, an
    empty prompt, per-head gains; the long prompt on sampled rows."""
    lens = [9000, 300, 0, 77]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    _say("attn varlen streamed bias", lens)
    q, k, v, g, _ = _attn_inputs(total, 4, 2, 128, torch.bfloat16, 46, "wide")
    pos = torch.from_numpy(np.concatenate([np.arange(m) * 2 for m in lens]).astype(np.int32))
    gain = _gains(4, 46)
    o, lse = gpu_lib.tg_gated_attn_varlen(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), pos.to(DEV),
                                          torch.from_numpy(cu).to(DEV), max(lens), want_lse=True,
                                          head_gain=gain.to(DEV))
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    for b, m in enumerate(lens):
        if m == 0:
            continue
        s0 = int(cu[b])
        sl = slice(s0, s0 + m)
        rows = _sample_rows(m, 7 + b, count=40) if m > 2000 else np.arange(m)
        wo, wl = ref_attn(q[sl], k[sl], v[sl], g[sl], pos[sl].numpy(), rows=rows, head_gain=gain.numpy())
        assert np.max(np.abs(o[s0 + rows] - wo)) <= 2e-2, f"prompt {b}"
        assert np.max(np.abs(lse[:, s0 + rows] - wl)) <= 1e-3, f"prompt {b}"


def test_attn_varlen_ragged(gpu_lib):
    lens = [256, 1, 100, 256, 129, 0, 256]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    q, k, v = W.qkv(total, 16, 8, 128, 1.0 / 128, torch.bfloat16, 31)
    g = W.random_scores(total, 31)
    pos = np.concatenate([np.sort(np.random.default_rng(b).choice(40000, n, replace=False)) for b, n in
                          enumerate(lens)]).astype(np.int32)
    o, lse = gpu_lib.tg_gated_attn_varlen(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV),
                                          torch.from_numpy(pos).to(DEV), torch.from_numpy(cu).to(DEV),
                                          max(lens), want_lse=True)
    torch.cuda.synchronize()
    wo, wl = ref_attn_varlen(q, k, v, g, pos, cu)
    assert np.max(np.abs(o.cpu().double().numpy() - wo)) <= 2e-2
    assert np.max(np.abs(lse.cpu().double().numpy() - wl)) <= 1e-3


def test_attn_first_query_is_its_own_value(gpu_lib):
    q, k, v, g, pos = _attn_inputs(200, 4, 2, 128, torch.bfloat16, 3)
    o, _ = _run_attn(gpu_lib, q, k, v, g, pos)
    np.testing.assert_array_equal(o[0], v[0, [0, 0, 1, 1]].double().numpy())


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
def test_attn_masks_by_kept_index_not_position_values(gpu_lib, dtype, tol):
    """Positions that break the strictly increasing precondition (repeats,
    descents, -1 as gather writes for an out-of-range index) do not change the
    output: both dtypes mask by kept index, which the oracle computes with
    positions 0..n-1.  The outputs are bit-identical to a call with those."""
    n = 200
    q, k, v, g, _ = _attn_inputs(n, 4, 2, 64, dtype, 11, "uniform")
    rng = np.random.default_rng(11)
    bad = rng.integers(-1, 50, n).astype(np.int32)
    bad[10:20] = 7
    bad[0] = -1
    o_bad, lse_bad = _run_attn(gpu_lib, q, k, v, g, torch.from_numpy(bad))
    o_idx, lse_idx = _run_attn(gpu_lib, q, k, v, g, torch.arange(n, dtype=torch.int32))
    np.testing.assert_array_equal(o_bad, o_idx)
    np.testing.assert_array_equal(lse_bad, lse_idx)
    wo, wl = ref_attn(q, k, v, g, np.arange(n))
    assert np.max(np.abs(o_bad - wo)) <= tol
    assert np.max(np.abs(lse_bad - wl)) <= 1e-3


def test_binding_refuses_host_buffers_next_to_device_ones(gpu_lib):
    """A host tensor among device tensors is refused before any launch: the C
    ABI takes raw pointers and would hand the kernel a host address."""
    q, k, v, g, pos = _attn_inputs(64, 4, 2, 64, torch.bfloat16, 3)
    qd, kd, vd, gd, pd = (t.to(DEV) for t in (q, k, v, g, pos))
    with pytest.raises(ValueError):
        gpu_lib.tg_gated_attn(qd, kd, vd, g, pd)  # gate values on the host
    with pytest.raises(ValueError):
        gpu_lib.tg_gated_attn(qd, kd, vd, gd, pos)  # positions on the host
    with pytest.raises(ValueError):
        gpu_lib.tg_gated_attn(qd, kd, vd, gd, pd, o=torch.empty_like(q))  # output on the host
    with pytest.raises(ValueError):
        gpu_lib.tg_gated_attn(qd, k, vd, gd, pd)  # keys on the host


# ----------------------------------------------------------------------------- end to end
def test_end_to_end_qwen_32k(gpu_lib):
    """The full path at the 32k workload: each stage checked against the oracle
    with that stage's input taken from the previous GPU stage (shared bytes)."""
    tg = gpu_lib
    sh = W.SHAPES["qwen1p7b_32k"]
    seed = W.SEEDS["qwen1p7b_32k"]
    _say("end-to-end 32k")
    h = W.hidden_states(sh.n, sh.d, sh.dtype, seed, planted_frac=sh.planted_frac)
    w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, sh.dtype, seed)
    hd = h.to(DEV)
    g = tg.tg_gate_score(hd, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2)
    idx = tg.tg_select_topk(g, sh.k, sh.q_len)
    hk, gk, pos = tg.tg_gather(hd, g, idx)
    q, k, v = W.qkv(sh.k, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, seed)
    table = tg.tg_rope_table(sh.n, sh.dh, sh.rope_base, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    _, kc, vc = tg.tg_rope_kv(qd, kd, vd, pos, table)
    o, lse = tg.tg_gated_attn(qd, kc, vc, gk, pos, want_lse=True)
    torch.cuda.synchronize()

    g_ref, _ = ref_gate(h, w1, b1, w2, b2)
    assert _rel_err(g.cpu().numpy(), g_ref) <= 1e-2
    g_cpu = g.cpu().numpy()
    idx_ref = ref_select(g_cpu, sh.k, sh.q_len)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    overlap = len(np.intersect1d(idx_ref, ref_select(g_ref.astype(np.float32), sh.k, sh.q_len))) / sh.k
    _say("  kept-set overlap with the oracle's own gate values:", overlap)
    wh, wg, wp = ref_gather(h.view(torch.int16).numpy(), g_cpu, idx_ref)
    np.testing.assert_array_equal(hk.cpu().view(torch.int16).numpy(), wh)
    np.testing.assert_array_equal(gk.cpu().numpy(), wg)
    np.testing.assert_array_equal(pos.cpu().numpy(), wp)
    assert np.all(np.abs(qd.cpu().double().numpy() - ref_rope(q, wp, sh.rope_base)) <=
                  2.0 ** -8 * np.abs(ref_rope(q, wp, sh.rope_base)) + 1e-6)
    rows = _sample_rows(sh.k, 8)
    wo, wl = ref_attn(qd.cpu(), kc.cpu(), vc.cpu(), wg, wp, rows=rows)
    assert np.max(np.abs(o.cpu().double().numpy()[rows] - wo)) <= 2e-2
    assert np.max(np.abs(lse.cpu().double().numpy()[:, rows] - wl)) <= 1e-3


def test_end_to_end_stack19_fused_calls(gpu_lib):
    """The 19-layer stack workload through the calls of its timed step: the
    fused gate + select + gather on the 65536-token prompt, then for each of
    the 19 upper layers RoPE + KV and gated attention with that layer's own
    q, k, v (drawn from seed * 1000 + layer).  The kept rows, gate values and
    positions are bit-exact against the oracle's select and gather on the g the
    call wrote; every layer's rotated q and its attention (sampled query rows,
    all heads) are checked against the oracle."""
    tg = gpu_lib
    sh = W.SHAPES["stack19"]
    seed = W.SEEDS["stack19"]
    _say("end-to-end stack19", sh.n, sh.k, sh.layers)
    h = W.hidden_states(sh.n, sh.d, sh.dtype, seed, planted_frac=sh.planted_frac)
    w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, sh.dtype, seed)
    ws = tg.select_workspace(sh.n, DEV)
    g, idx, hk, gk, pos = tg.tg_gate_select_gather(h.to(DEV), w1.to(DEV), b1.to(DEV), w2.to(DEV), b2, sh.k,
                                                   sh.q_len, workspace=ws)
    table = tg.tg_rope_table(sh.n, sh.dh, sh.rope_base, DEV)
    torch.cuda.synchronize()
    g_cpu = g.cpu().numpy()
    idx_ref = ref_select(g_cpu, sh.k, sh.q_len)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    wh, wg, wp = ref_gather(h.view(torch.int16).numpy(), g_cpu, idx_ref)
    np.testing.assert_array_equal(hk.cpu().view(torch.int16).numpy(), wh)
    np.testing.assert_array_equal(gk.cpu().numpy(), wg)
    np.testing.assert_array_equal(pos.cpu().numpy(), wp)
    rows = _sample_rows(sh.k, 19, count=24)
    worst = 0.0
    for layer in range(sh.layers):
        q, k, v = W.qkv(sh.k, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, seed * 1000 + layer)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        _, kc, vc = tg.tg_rope_kv(qd, kd, vd, pos, table)
        o, lse = tg.tg_gated_attn(qd, kc, vc, gk, pos, want_lse=True)
        torch.cuda.synchronize()
        rq = ref_rope(q, wp, sh.rope_base)
        assert np.all(np.abs(qd.cpu().double().numpy() - rq) <= 2.0 ** -8 * np.abs(rq) + 1e-6), layer
        wo, wl = ref_attn(qd.cpu(), kc.cpu(), vc.cpu(), wg, wp, rows=rows)
        err = float(np.max(np.abs(o.cpu().double().numpy()[rows] - wo)))
        worst = max(worst, err)
        assert err <= 2e-2, (layer, err)
        assert np.max(np.abs(lse.cpu().double().numpy()[:, rows] - wl)) <= 1e-3, layer
    _say("  worst max abs err o over 19 layers", worst)


def test_repeat_runs_are_bitwise_identical(gpu_lib):
    """Ten runs of every stage on the same inputs give the same bytes: the gate,
    both selects (the multi-workgroup one builds its histograms with device
    atomics, whose order must not matter), gather, RoPE + KV, attention, decode
    and a dense product."""
    tg = gpu_lib
    _say("repeat runs")
    n, d, hidden, k, q_len = 32768, 2048, 256, 4096, 64
    h = W.hidden_states(n, d, torch.bfloat16, 12, planted_frac=0.05).to(DEV)
    w1, b1, w2, b2 = W.gate_weights(d, hidden, torch.bfloat16, 12)
    w1, b1, w2 = w1.to(DEV), b1.to(DEV), w2.to(DEV)
    g = W.random_scores(n, 2).to(DEV)
    ws = torch.empty(tg.tg_select_topk_workspace_size(n), dtype=torch.uint8, device=DEV)
    q, kk, vv, gk, pos = _attn_inputs(1000, 16, 8, 128, torch.bfloat16, 4)
    q, kk, vv, gk, pos = (t.to(DEV) for t in (q, kk, vv, gk, pos))
    table = tg.tg_rope_table(4096, 128, 1e6, DEV)
    cu = torch.tensor([0, 600, 1000], dtype=torch.int32, device=DEV)
    qn = W.qkv(2, 16, 8, 128, 1.0 / 128, torch.bfloat16, 13)[0].to(DEV)
    x = W.hidden_states(300, 2048, torch.bfloat16, 14).to(DEV)
    wl = W.linear_weight(512, 2048, torch.bfloat16, 14).to(DEV)
    first = None
    for _ in range(10):
        gg = tg.tg_gate_score(h, w1, b1, w2, b2)
        idx = tg.tg_select_topk(g, k, q_len)
        idx_ws = tg.tg_select_topk_ws(g, k, q_len, workspace=ws)
        hk, gk2, pk = tg.tg_gather(h, gg, idx)
        qr = q.clone()
        _, kc, vc = tg.tg_rope_kv(qr, kk, vv, pos, table)
        o = tg.tg_gated_attn(q, kk, vv, gk, pos)
        od = tg.tg_decode_attn(qn, kk, vv, gk, cu, 600)
        y = tg.tg_linear(x, wl)
        torch.cuda.synchronize()
        cur = [t.cpu().view(torch.int16) if t.dtype == torch.bfloat16 else t.cpu()
               for t in (gg, idx, idx_ws, hk, gk2, pk, qr, kc, vc, o, od, y)]
        if first is None:
            first = cur
            assert torch.equal(idx, idx_ws)
        else:
            for a, b in zip(cur, first):
                assert torch.equal(a, b)


# ----------------------------------------------------------------------------- decode
def _decode_case(tg, lens, hq, hkv, dh, dtype, seed, gkind="uniform", gain=False):
    B, total = len(lens), int(sum(lens))
    q, _, _ = W.qkv(B, hq, hkv, dh, 1.0 / dh, dtype, seed)
    _, k, v = W.qkv(total, hq, hkv, dh, 1.0 / dh, dtype, seed + 1)
    g = None
    if gkind == "uniform":
        g = W.random_scores(total, seed)
    elif gkind == "wide":
        g = W.gate_values_wide(total, seed)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    hg = _gains(hq, seed) if gain else None
    o_ref, lse_ref = ref_decode(q, k, v, g, cu, head_gain=hg)
    o, lse = tg.tg_decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), None if g is None else g.to(DEV), cu.to(DEV),
                               max(lens), head_gain=None if hg is None else hg.to(DEV), want_lse=True)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref


@pytest.mark.parametrize("dtype,lens,hq,hkv,dh,gkind,gain", [
    (torch.bfloat16, [0, 1, 37, 1000, 4099], 16, 8, 128, "uniform", True),
    (torch.bfloat16, [513, 2048, 64], 32, 4, 64, "wide", False),
    (torch.bfloat16, [300, 7], 4, 2, 128, None, False),
    (torch.bfloat16, [4096 + 37] * 3, 16, 16, 64, "uniform", True),
    (torch.float32, [5, 300, 1025], 4, 4, 128, None, False),
    (torch.float32, [0, 2, 777], 8, 2, 64, "wide", True),
    # (sequence, KV head) pairs >= 256 with 1-2 heads per KV head: one block per pair, no combine pass
    (torch.bfloat16, [0, 1, 300, 64, 1000, 5, 129, 2] * 4, 8, 8, 64, "uniform", True),
    (torch.float32, [700, 0, 65, 1] * 4, 32, 16, 128, None, False),
])
def test_decode_parity(gpu_lib, dtype, lens, hq, hkv, dh, gkind, gain):
    _say("decode", dtype, lens, hq, hkv, dh, gkind, gain)
    o, lse, o_ref, lse_ref = _decode_case(gpu_lib, lens, hq, hkv, dh, dtype, 31 + sum(lens), gkind, gain)
    tol_o, tol_l = (2e-2, 1e-3) if dtype == torch.bfloat16 else (1e-4, 1e-4)
    err_o = float(np.max(np.abs(o - o_ref)))
    live = np.isfinite(lse_ref)
    err_l = float(np.max(np.abs(lse[live] - lse_ref[live])))
    _say("  max abs err o", err_o, "lse", err_l)
    assert err_o <= tol_o and err_l <= tol_l
    assert np.array_equal(np.isfinite(lse), live)  # empty caches: lse = -inf
    assert np.all(o[~live] == 0.0)


def test_decode_bench_shape_sampled(gpu_lib):
    # 32 sequences with 4096-key compact caches (the 32k prompt's budget) plus
    # a few generated tokens each; the oracle checks a sample of sequences.
    rng = np.random.default_rng(5)
    lens = [4096 + int(x) for x in rng.integers(0, 256, 32)]
    hq, hkv, dh = 16, 8, 128
    q, _, _ = W.qkv(32, hq, hkv, dh, 1.0 / dh, torch.bfloat16, 77)
    _, k, v = W.qkv(sum(lens), hq, hkv, dh, 1.0 / dh, torch.bfloat16, 78)
    g = W.random_scores(sum(lens), 79)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    o, lse = gpu_lib.tg_decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), cu.to(DEV), max(lens),
                                    want_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    for b in (0, 13, 31):
        a, e = int(cu[b]), int(cu[b + 1])
        o_ref, lse_ref = ref_decode(q[b:b + 1], k[a:e], v[a:e], g[a:e], np.array([0, e - a]))
        assert np.max(np.abs(o[b] - o_ref[0])) <= 2e-2
        assert np.max(np.abs(lse[b] - lse_ref[0])) <= 1e-3


def test_decode_reuses_a_dirty_workspace(gpu_lib):
    # The workspace needs no clearing: a second call over the same (dirty)
    # buffer with other lengths gives the oracle's result.
    hq, hkv, dh = 16, 8, 128
    ws = torch.full((gpu_lib.tg_decode_attn_workspace_size(3, 5000, hq, hkv, dh),), 255, dtype=torch.uint8,
                    device=DEV)
    for lens in ([5000, 4000, 1], [17, 0, 2500]):
        q, _, _ = W.qkv(3, hq, hkv, dh, 1.0 / dh, torch.bfloat16, 90 + lens[0])
        _, k, v = W.qkv(sum(lens), hq, hkv, dh, 1.0 / dh, torch.bfloat16, 91 + lens[0])
        g = W.random_scores(sum(lens), 92)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
        o = gpu_lib.tg_decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), cu.to(DEV), 5000, workspace=ws)
        torch.cuda.synchronize()
        o_ref, _ = ref_decode(q, k, v, g, cu)
        assert np.max(np.abs(o.cpu().double().numpy() - o_ref)) <= 2e-2


# ----------------------------------------------------------------------------- dense (upper layers)
def _dense_ok(got, want, slack=1e-3):
    """One bf16 rounding of the fp32-accumulated result: |got - want| <= 2^-8 |want|
    plus `slack` times the output's rms for values near zero."""
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want ** 2))) + 1e-30
    excess = np.abs(got - want) - (2.0 ** -8 * np.abs(want) + slack * rms)
    _say("  max abs err", float(np.max(np.abs(got - want))), "rms", rms, "worst excess", float(np.max(excess)))
    return bool(np.all(excess <= 0))


@pytest.mark.parametrize("m,n,k", [(1, 256, 32), (300, 256, 64), (129, 512, 2048), (4133, 4096, 256),
                                   (1000, 2048, 6144)])
def test_linear_parity(gpu_lib, m, n, k):
    _say("linear", m, n, k)
    x = W.hidden_states(m, k, torch.bfloat16, m + k)
    w = W.linear_weight(n, k, torch.bfloat16, n + k)
    y = gpu_lib.tg_linear(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    assert _dense_ok(y.cpu().double().numpy(), ref_linear(x, w))


@pytest.mark.parametrize("m,n,k,inplace", [(300, 256, 64, False), (4133, 4096, 256, True), (777, 2048, 512, True)])
def test_linear_residual_parity(gpu_lib, m, n, k, inplace):
    _say("linear + residual", m, n, k, "in place" if inplace else "")
    x = W.hidden_states(m, k, torch.bfloat16, 5 + m)
    w = W.linear_weight(n, k, torch.bfloat16, 6 + n)
    r = W.hidden_states(m, n, torch.bfloat16, 7 + k)
    want = ref_linear(x, w, r)
    rd = r.to(DEV)
    y = gpu_lib.tg_linear(x.to(DEV), w.to(DEV), residual=rd, y=rd if inplace else None)
    torch.cuda.synchronize()
    assert _dense_ok(y.cpu().double().numpy(), want)


@pytest.mark.parametrize("m,f,k", [(300, 128, 64), (129, 256, 2048), (4133, 6144, 256), (64, 768, 96)])
def test_swiglu_parity(gpu_lib, m, f, k):
    _say("swiglu", m, f, k)
    x = W.hidden_states(m, k, torch.bfloat16, 9 + m)
    wg = W.linear_weight(f, k, torch.bfloat16, 10 + f)
    wu = W.linear_weight(f, k, torch.bfloat16, 11 + f)
    y = gpu_lib.tg_swiglu(x.to(DEV), wg.to(DEV), wu.to(DEV))
    torch.cuda.synchronize()
    assert _dense_ok(y.cpu().double().numpy(), ref_swiglu(x, wg, wu))


def test_linear_strided_operands(gpu_lib):
    # Row strides of x, w and y larger than the logical widths (views into
    # wider buffers), as when q, k and v are column slices of one projection.
    m, n, k = 300, 256, 128
    xb = W.hidden_states(m, k + 64, torch.bfloat16, 21)
    wb = W.linear_weight(n, k + 32, torch.bfloat16, 22)
    x, w = xb[:, 32:32 + k], wb[:, :k]
    yb = torch.zeros(m, n + 256, dtype=torch.bfloat16, device=DEV)
    gpu_lib.tg_linear(xb.to(DEV)[:, 32:32 + k], wb.to(DEV)[:, :k], y=yb[:, 256:])
    torch.cuda.synchronize()
    assert _dense_ok(yb[:, 256:].cpu().double().numpy(), ref_linear(x, w))
    assert torch.all(yb[:, :256] == 0)  # nothing written outside y


def test_mlp_block_qwen_shape_sampled_rows(gpu_lib):
    # The MLP block of one upper layer at the bench shape: 4096 kept tokens,
    # d = 2048, F = 6144: SwiGLU, then the down projection onto the residual
    # stream in place.  The oracle checks 48 sampled rows (first, last, tile
    # boundaries and random ones).
    m, d, f = 4096, 2048, 6144
    x = W.hidden_states(m, d, torch.bfloat16, 31)
    wg = W.linear_weight(f, d, torch.bfloat16, 32)
    wu = W.linear_weight(f, d, torch.bfloat16, 33)
    wd = W.linear_weight(d, f, torch.bfloat16, 34)
    res = W.hidden_states(m, d, torch.bfloat16, 35)
    xd, resd = x.to(DEV), res.to(DEV)
    a = gpu_lib.tg_swiglu(xd, wg.to(DEV), wu.to(DEV))
    gpu_lib.tg_linear(a, wd.to(DEV), residual=resd, y=resd)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, m - 1],
                                     np.random.default_rng(36).choice(m, 42, replace=False)]))
    want = ref_mlp(x[rows], wg, wu, wd, res[rows])
    # The hidden activation is stored in bf16 between the two products (as the
    # layer stores it); its rounding (2^-9 relative per element) reaches the
    # output as noise of ~1e-3 of the output's rms, hence the wider slack.
    assert _dense_ok(resd.cpu()[rows].double().numpy(), want, slack=1e-2)
    # The hidden activation itself, on the same rows.
    assert _dense_ok(a.cpu()[rows].double().numpy(), ref_swiglu(x[rows], wg, wu))


@pytest.mark.parametrize("m,hq,hkv,dh,k", [(300, 16, 8, 128, 256), (4133, 16, 8, 128, 128), (77, 8, 4, 64, 64)])
def test_qkv_proj_parity(gpu_lib, m, hq, hkv, dh, k):
    _say("qkv_proj", m, hq, hkv, dh, k)
    x = W.hidden_states(m, k, torch.bfloat16, 41 + m)
    w = W.linear_weight((hq + 2 * hkv) * dh, k, torch.bfloat16, 42 + k)
    q, kk, vv = gpu_lib.tg_qkv_proj(x.to(DEV), w.to(DEV), hq, hkv, dh)
    torch.cuda.synchronize()
    want = ref_linear(x, w)
    nq, nkv = hq * dh, hkv * dh
    assert _dense_ok(q.cpu().reshape(m, nq).double().numpy(), want[:, :nq])
    assert _dense_ok(kk.cpu().reshape(m, nkv).double().numpy(), want[:, nq:nq + nkv])
    assert _dense_ok(vv.cpu().reshape(m, nkv).double().numpy(), want[:, nq + nkv:])


# ----------------------------------------------------------------------------- position check
def test_check_positions(gpu_lib):
    def run(pos, cu=None):
        p = torch.tensor(pos, dtype=torch.int32, device=DEV)
        c = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=DEV)
        return int(gpu_lib.tg_check_positions(p, c).item())

    sparse = np.sort(np.random.default_rng(3).choice(40000, 5000, replace=False)).tolist()
    assert run(sparse) == 5000  # select + gather order: valid
    bad = list(sparse)
    bad[3001] = bad[3000]  # repeated position
    bad[4000] = -1
    assert run(bad) == 3001
    assert run([0, 5, 5]) == 2
    assert run([3, 2, 1]) == 1
    assert run([-4]) == 0
    assert run([]) == 0
    # Packed sequences: each restarts its positions; the order is checked within each.
    assert run([0, 4, 9, 1, 2, 0, 7], cu=[0, 3, 5, 5, 7]) == 7
    assert run([0, 4, 9, 1, 1, 0, 7], cu=[0, 3, 5, 5, 7]) == 4
    assert run([0, 4, 9, 1, 2, 0, 0], cu=[0, 3, 5, 5, 7]) == 6


# ----------------------------------------------------------------------------- HIP graph replay
def test_path_replayed_from_a_hip_graph(gpu_lib):
    # The whole path (gate -> select -> gather -> RoPE + KV -> attention, plus
    # decode over the cache it built) captured once into a HIP graph and
    # replayed three times, with eager work and synchronisation between the
    # replays.  Every replay must reproduce the eager outputs bit for bit.
    tg = gpu_lib
    n, q_len, d, hidden, k, hq, hkv, dh = 4096, 64, 2048, 256, 1024, 16, 8, 128
    h = W.hidden_states(n, d, torch.bfloat16, 51, planted_frac=0.05).to(DEV)
    w1, b1, w2, b2 = W.gate_weights(d, hidden, torch.bfloat16, 51)
    w1, b1, w2 = w1.to(DEV), b1.to(DEV), w2.to(DEV)
    q0, kk, vv = (t.to(DEV) for t in W.qkv(k, hq, hkv, dh, 1.0 / dh, torch.bfloat16, 52))
    qn = W.qkv(1, hq, hkv, dh, 1.0 / dh, torch.bfloat16, 53)[0].to(DEV)
    table = tg.tg_rope_table(n, dh, 1e6, DEV)
    cu = torch.tensor([0, k], dtype=torch.int32, device=DEV)
    ws = torch.empty(tg.tg_decode_attn_workspace_size(1, k, hq, hkv, dh), dtype=torch.uint8, device=DEV)
    sws = torch.empty(tg.tg_select_topk_workspace_size(n), dtype=torch.uint8, device=DEV)

    def buffers():
        return {"g": torch.empty(n, device=DEV), "idx": torch.empty(k, dtype=torch.int32, device=DEV),
                "idx_ws": torch.empty(k, dtype=torch.int32, device=DEV),
                "hk": torch.empty(k, d, dtype=torch.bfloat16, device=DEV), "gk": torch.empty(k, device=DEV),
                "pos": torch.empty(k, dtype=torch.int32, device=DEV), "q": torch.empty_like(q0),
                "kc": torch.empty_like(kk), "vc": torch.empty_like(vv), "o": torch.empty_like(q0),
                "lse": torch.empty(hq, k, device=DEV), "od": torch.empty_like(qn)}

    def path(b):
        b["q"].copy_(q0)  # RoPE rotates q in place: start every run from the same q
        tg.tg_gate_score(h, w1, b1, w2, b2, g=b["g"])
        tg.tg_select_topk(b["g"], k, q_len, idx=b["idx"])
        tg.tg_select_topk_ws(b["g"], k, q_len, idx=b["idx_ws"], workspace=sws)  # its zero kernel, too
        tg.tg_gather(h, b["g"], b["idx"], h_out=b["hk"], g_out=b["gk"], pos_out=b["pos"])
        tg.tg_rope_kv(b["q"], kk, vv, b["pos"], table, k_cache=b["kc"], v_cache=b["vc"])
        tg.tg_gated_attn(b["q"], b["kc"], b["vc"], b["gk"], b["pos"], o=b["o"], lse=b["lse"])
        tg.tg_decode_attn(qn, b["kc"], b["vc"], b["gk"], cu, k, o=b["od"], workspace=ws)

    eager = buffers()
    path(eager)
    torch.cuda.synchronize()
    want = {name: t.clone() for name, t in eager.items()}
    assert torch.equal(want["idx"], want["idx_ws"])

    graphed = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path(graphed)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path(graphed)
    for rep in range(3):
        for t in graphed.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say("graph replay", rep)
        for name, t in graphed.items():
            a, b = t.view(torch.uint8) if t.dtype != torch.bfloat16 else t.view(torch.int16), want[name]
            b = b.view(torch.uint8) if b.dtype != torch.bfloat16 else b.view(torch.int16)
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"
        path(eager)  # eager work between replays
        torch.cuda.synchronize()


def test_end_to_end_ragged_batch_of_eight_prompts(gpu_lib):
    """The packed-batch path at its configuration: 8 prompts of 4096-32768
    tokens with 32-128-token question tails, K = 256 kept per prompt, each
    stage checked against the oracle on the previous GPU stage's bytes."""
    tg = gpu_lib
    sh = W.SHAPES["ragged8"]
    seed = W.SEEDS["ragged8"]
    ns, qs = W.ragged_lengths(8, seed)
    _say("end-to-end ragged8", ns, qs)
    cu = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    total = int(cu[-1])
    h = W.hidden_states(total, sh.d, sh.dtype, seed)
    w1, b1, w2, b2 = W.gate_weights(sh.d, sh.hidden, sh.dtype, seed)
    hd = h.to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    g = tg.tg_gate_score(hd, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2)
    kept_total = sum(min(sh.k, n) for n in ns)
    idx, cu_kept = tg.tg_select_topk_varlen(g, cud, torch.tensor(qs, dtype=torch.int32, device=DEV), max(ns), sh.k,
                                            kept_total)
    hk, gk, pos = tg.tg_gather_varlen(hd, g, idx, cud, cu_kept, sh.k)
    q, k, v = W.qkv(kept_total, sh.hq, sh.hkv, sh.dh, sh.qkv_var, sh.dtype, seed)
    table = tg.tg_rope_table(max(ns), sh.dh, sh.rope_base, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    _, kc, vc = tg.tg_rope_kv(qd, kd, vd, pos, table)
    o, lse = tg.tg_gated_attn_varlen(qd, kc, vc, gk, pos, cu_kept, sh.k, want_lse=True)
    torch.cuda.synchronize()

    # Gate on 2048 sampled rows (the oracle on all ~150k rows would take minutes).
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, np.random.default_rng(seed).choice(total, 2000,
                                                                                          replace=False)]))
    g_ref, _ = ref_gate(h[rows], w1, b1, w2, b2)
    g_cpu = g.cpu().numpy()
    assert _rel_err(g_cpu[rows], g_ref) <= 1e-2
    idx_ref, cu_kept_ref = ref_select_varlen(g_cpu, cu, qs, sh.k)
    np.testing.assert_array_equal(cu_kept.cpu().numpy(), cu_kept_ref)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    grow = np.concatenate([cu[b] + idx_ref[cu_kept_ref[b]:cu_kept_ref[b + 1]] for b in range(8)])
    np.testing.assert_array_equal(hk.cpu().view(torch.int16).numpy(), h.view(torch.int16).numpy()[grow])
    np.testing.assert_array_equal(gk.cpu().numpy(), g_cpu[grow])
    np.testing.assert_array_equal(pos.cpu().numpy(), idx_ref)
    wq = ref_rope(q, idx_ref, sh.rope_base)
    assert np.all(np.abs(qd.cpu().double().numpy() - wq) <= 2.0 ** -8 * np.abs(wq) + 1e-6)
    wo, wl = ref_attn_varlen(qd.cpu(), kc.cpu(), vc.cpu(), g_cpu[grow], idx_ref, cu_kept_ref)
    assert np.max(np.abs(o.cpu().double().numpy() - wo)) <= 2e-2
    assert np.max(np.abs(lse.cpu().double().numpy() - wl)) <= 1e-3
