"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random tensors and applies the input transforms that define each
workload (scaling, per-token L2 normalisation of q and k, the decay and write-strength
parametrisations).  It holds none of the recurrence's arithmetic.  Both sides receive
exactly the same arrays: the device tensors go to the library, their host copies go to
the oracle.

Recipes (one torch.Generator per tensor, seeded with ``seed * 1000 + tensor_id``;
tensor ids q=0, k=1, v=2, a=3, beta-logit=4, state=5, warm-up=6):

* additive  : q, k, v ~ N(0,1)/sqrt(d)                       (float32 or bfloat16)
* based     : q, k ~ N(0,1)/sqrt(d'), v ~ N(0,1)
* gated     : as gated_delta without the key normalisation requirement
* gated_delta: q, k ~ N(0,1) then L2-normalised per token (in float32), v ~ N(0,1),
              alpha = exp(-softplus(a)), a ~ U(-2, 4), beta = sigmoid(N(0,1))
Every tensor is generated in float32 and rounded once (round-to-nearest-even) to the
requested dtype.  State tensors are float32.
"""

from __future__ import annotations

import math

import torch

Q, K, V, A, BETA, STATE, WARMUP = range(7)


def _gen(device, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(tid))
    return g


def randn(shape, seed, tid, device="cpu"):
    return torch.randn(shape, generator=_gen(device, seed, tid), device=device, dtype=torch.float32)


def rand(shape, seed, tid, device="cpu"):
    return torch.rand(shape, generator=_gen(device, seed, tid), device=device, dtype=torch.float32)


def _l2norm_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def additive_inputs(B, H, T, d, dtype=torch.float32, seed=0, device="cpu"):
    s = 1.0 / math.sqrt(d)
    return dict(
        q=(randn((B, H, T, d), seed, Q, device) * s).to(dtype),
        k=(randn((B, H, T, d), seed, K, device) * s).to(dtype),
        v=(randn((B, H, T, d), seed, V, device) * s).to(dtype),
    )


def based_inputs(B, H, T, dp, dv, dtype=torch.bfloat16, seed=0, device="cpu"):
    s = 1.0 / math.sqrt(dp)
    return dict(
        q=(randn((B, H, T, dp), seed, Q, device) * s).to(dtype),
        k=(randn((B, H, T, dp), seed, K, device) * s).to(dtype),
        v=randn((B, H, T, dv), seed, V, device).to(dtype),
    )


def decay_and_strength(shape, seed=0, device="cpu", a_lo=-2.0, a_hi=4.0):
    """alpha = exp(-softplus(a)), a ~ U(a_lo, a_hi);  beta = sigmoid(N(0,1)); both float32."""
    a = a_lo + (a_hi - a_lo) * rand(shape, seed, A, device)
    alpha = torch.exp(-torch.nn.functional.softplus(a))
    beta = torch.sigmoid(randn(shape, seed, BETA, device))
    return alpha, beta


def gdn_inputs(B, H, T, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu", normalize=True):
    q = randn((B, H, T, dk), seed, Q, device)
    k = randn((B, H, T, dk), seed, K, device)
    if normalize:
        q, k = _l2norm_rows(q), _l2norm_rows(k)
    v = randn((B, H, T, dv), seed, V, device)
    alpha, beta = decay_and_strength((B, H, T), seed, device)
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), alpha=alpha.to(dtype),
                beta=beta.to(dtype))


def gdn_state(shape, seed=0, device="cpu"):
    """A seeded N(0,1) float32 state (e.g. [N, d_v, d_k])."""
    return randn(shape, seed, STATE, device)


def gdn_decode_inputs(steps, N, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Per-step decode inputs with the gated-delta recipe: q, k [steps, N, d_k] etc."""
    d = gdn_inputs(1, steps, N, dk, dv, dtype=dtype, seed=seed, device=device)
    return {n: t[0] for n, t in d.items()}


def based_decode_inputs(steps, N, dp, dv, dtype=torch.bfloat16, seed=0, device="cpu"):
    d = based_inputs(1, steps, N, dp, dv, dtype=dtype, seed=seed, device=device)
    return {n: t[0] for n, t in d.items()}


def based_warmup_inputs(N, T_warm, dp, dv, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Warm-up tokens whose end state serves as a seeded, consistent BASED start state."""
    d = based_inputs(1, N, T_warm, dp, dv, dtype=dtype, seed=seed * 7 + WARMUP, device=device)
    return {n: t[0] for n, t in d.items()}
