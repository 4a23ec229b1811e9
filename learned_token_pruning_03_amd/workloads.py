"""Seeded synthetic workloads for the TokenGate gated-prefill path.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic.  It is shared by the tests, the benchmark and the
oracle's callers, so that the GPU path and the oracle are fed the very same
bytes.  Every tensor is produced on the CPU by a seeded ``torch.Generator``
and rounded to its storage dtype with round-to-nearest-even (``Tensor.to``).

The pages measure on long-context QA, summarisation, code-completion and
needle-in-a-haystack prompts with Qwen3-1.7B (TokenGate paper page,
thelatestinai.com, Figure 3 and Table 3).  Those datasets and the trained gate
are not available, so these generators stand in for them with the shapes of
Qwen3-1.7B's layer (hidden 2048, 16 query heads, 8 KV heads, head dim 128) and
random values of the stated distributions.

Workloads (the seed of workload ``c`` is ``1000 + c``):

* ``tiny``   fp32: N=512 (last 32 are the question), d=256, gate 256->64->1,
  K=128, 4 query / 2 KV heads, head dim 64, Q/K/V ~ N(0, 1/64); no RoPE.
* ``qwen1p7b_32k`` bf16: N=32768 (64-token question), d=2048 ~ N(0,1) with 5%
  of the rows (chosen by the seed) scaled by 8, gate 2048->256->1, K=4096,
  16/8 heads, head dim 128, Q/K/V ~ N(0, 1/128), RoPE base 1e6.
* ``qwen1p7b_128k`` bf16: as above with N=131072, K=8192, no planted rows, and
  an attention/select gate vector drawn as sigmoid(N(0, variance 2)).
* ``ragged8`` bf16: 8 prompts, N_b ~ U{4096..32768}, q_b ~ U{32..128}, K=256
  kept per prompt, packed along the token axis with ``cu_seqlens``.
* ``stack19`` bf16: N=65536, K=4096, gate once, then 19 upper layers, each with
  its own Q/K/V (seed ``1000*4 + layer``).

The second argument of N(0, x) is a variance.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "WorkloadShape",
    "SHAPES",
    "gate_weights",
    "hidden_states",
    "qkv",
    "gate_values_wide",
    "ragged_lengths",
    "tie_storm_scores",
]


@dataclass(frozen=True)
class WorkloadShape:
    name: str
    dtype: torch.dtype
    n: int            # tokens in the prompt, question tail included
    q_len: int        # trailing question tokens that are never pruned
    d: int            # hidden size of the selection layer's residual stream
    hidden: int       # gate MLP hidden width
    k: int            # kept-token budget (question included)
    hq: int
    hkv: int
    dh: int
    rope: bool
    rope_base: float = 1.0e6
    planted_frac: float = 0.0
    planted_scale: float = 8.0
    qkv_var: float = 1.0 / 128.0
    layers: int = 1
    batch: int = 1
    extra: dict = field(default_factory=dict)


SHAPES = {
    "tiny": WorkloadShape("tiny", torch.float32, n=512, q_len=32, d=256, hidden=64, k=128,
                          hq=4, hkv=2, dh=64, rope=False, qkv_var=1.0 / 64.0),
    "qwen1p7b_32k": WorkloadShape("qwen1p7b_32k", torch.bfloat16, n=32768, q_len=64, d=2048,
                                  hidden=256, k=4096, hq=16, hkv=8, dh=128, rope=True,
                                  planted_frac=0.05),
    "qwen1p7b_128k": WorkloadShape("qwen1p7b_128k", torch.bfloat16, n=131072, q_len=64, d=2048,
                                   hidden=256, k=8192, hq=16, hkv=8, dh=128, rope=True),
    "ragged8": WorkloadShape("ragged8", torch.bfloat16, n=0, q_len=0, d=2048, hidden=256, k=256,
                             hq=16, hkv=8, dh=128, rope=True, batch=8),
    "stack19": WorkloadShape("stack19", torch.bfloat16, n=65536, q_len=64, d=2048, hidden=256,
                             k=4096, hq=16, hkv=8, dh=128, rope=True, layers=19),
}

SEEDS = {"tiny": 1000, "qwen1p7b_32k": 1001, "qwen1p7b_128k": 1002, "ragged8": 1003,
         "stack19": 1004}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def gate_weights(d: int, hidden: int, dtype: torch.dtype, seed: int):
    """Xavier-uniform (gain 1) weights, zero biases.

    Returns ``W1`` [hidden, d] in ``dtype`` (nn.Linear layout), ``b1`` [hidden]
    fp32, ``w2`` [hidden] fp32 holding values representable in ``dtype``, and
    ``b2`` (a Python float).
    """
    g = _gen(seed * 7919 + 1)
    w1 = torch.empty(hidden, d, dtype=torch.float32)
    torch.nn.init.xavier_uniform_(w1, gain=1.0, generator=g)
    w2 = torch.empty(1, hidden, dtype=torch.float32)
    torch.nn.init.xavier_uniform_(w2, gain=1.0, generator=g)
    w1 = w1.to(dtype).contiguous()
    w2 = w2.to(dtype).to(torch.float32).reshape(hidden).contiguous()
    b1 = torch.zeros(hidden, dtype=torch.float32)
    return w1, b1, w2, 0.0


def linear_weight(n_out: int, n_in: int, dtype: torch.dtype, seed: int):
    """A random-init projection weight [n_out, n_in] (nn.Linear layout),
    N(0, 1/n_in) so that outputs of N(0, 1) inputs stay O(1)."""
    g = _gen(seed * 7919 + 11)
    w = torch.randn(n_out, n_in, generator=g, dtype=torch.float32) / math.sqrt(n_in)
    return w.to(dtype).contiguous()


def hidden_states(n: int, d: int, dtype: torch.dtype, seed: int,
                  planted_frac: float = 0.0, planted_scale: float = 8.0):
    """h [n, d] ~ N(0, 1); ``round(planted_frac * n)`` rows, chosen by the seed
    among all n rows, are multiplied by ``planted_scale`` (a power of two, so
    the rounding of the base values is unchanged)."""
    g = _gen(seed * 7919 + 2)
    h = torch.randn(n, d, generator=g, dtype=torch.float32)
    n_planted = int(round(planted_frac * n))
    if n_planted:
        rows = torch.randperm(n, generator=g)[:n_planted]
        h[rows] *= planted_scale
    return h.to(dtype).contiguous()


def qkv(n: int, hq: int, hkv: int, dh: int, var: float, dtype: torch.dtype, seed: int):
    """q [n, hq, dh], k and v [n, hkv, dh] ~ N(0, var)."""
    g = _gen(seed * 7919 + 3)
    std = math.sqrt(var)
    q = torch.randn(n, hq, dh, generator=g) * std
    k = torch.randn(n, hkv, dh, generator=g) * std
    v = torch.randn(n, hkv, dh, generator=g) * std
    return q.to(dtype).contiguous(), k.to(dtype).contiguous(), v.to(dtype).contiguous()


def gate_values_wide(n: int, seed: int, var: float = 2.0):
    """fp32 gate values sigmoid(z), z ~ N(0, var): a widely spread g vector."""
    g = _gen(seed * 7919 + 4)
    z = torch.randn(n, generator=g, dtype=torch.float64) * math.sqrt(var)
    return torch.sigmoid(z).to(torch.float32).contiguous()


def ragged_lengths(batch: int, seed: int, n_lo=4096, n_hi=32768, q_lo=32, q_hi=128):
    """Per-prompt lengths N_b ~ U{n_lo..n_hi} and question tails q_b ~ U{q_lo..q_hi}."""
    g = _gen(seed * 7919 + 5)
    ns = torch.randint(n_lo, n_hi + 1, (batch,), generator=g)
    qs = torch.randint(q_lo, q_hi + 1, (batch,), generator=g)
    return [int(x) for x in ns], [int(x) for x in qs]


def tie_storm_scores(n: int, levels: int, seed: int):
    """fp32 scores taking only ``levels`` distinct values in (0, 1)."""
    g = _gen(seed * 7919 + 6)
    lv = torch.randint(0, levels, (n,), generator=g).to(torch.float32)
    return ((lv + 1.0) / (levels + 1.0)).contiguous()


def random_scores(n: int, seed: int):
    """fp32 scores uniform in (0, 1)."""
    g = _gen(seed * 7919 + 7)
    return torch.rand(n, generator=g, dtype=torch.float32).clamp_min(1e-7).contiguous()
