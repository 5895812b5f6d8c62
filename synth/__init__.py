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

Regimes beyond the configurations' gates (``gdn_inputs`` keyword arguments), used by the
long-memory parity tests: ``a_range`` moves the decay parameter (a ~ U(-8, -4) gives
alpha in [0.982, 0.9997]; a ~ U(-14, -10) gives alpha above 0.99995), ``alpha_one`` and
``beta`` ("sigmoid", "zero", "one") fix the gates, and ``keys`` picks the key set:
"random" (the recipe above), "pool" (each key one of ``pool`` fixed random unit
directions, tensor ids 7 and 8: repeated, correlated keys) or "basis" (standard basis
vectors e_i with i uniform, tensor id 7, exact in bf16) or "perm" (the d_k basis vectors
in a random order, repeating only after d_k tokens); ``q_is_k`` makes every query
equal to its token's key.
"""

from __future__ import annotations

import math

import torch

Q, K, V, A, BETA, STATE, WARMUP, KEY_INDEX, KEY_POOL = range(9)


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


def _keys(B, H, T, dk, keys, pool, seed, device):
    if keys == "random":
        return randn((B, H, T, dk), seed, K, device)
    idx_src = rand((B, H, T), seed, KEY_INDEX, device)
    if keys == "basis":
        idx = (idx_src * dk).long().clamp_max(dk - 1)
        return torch.nn.functional.one_hot(idx, dk).to(torch.float32)
    if keys == "perm":  # basis vectors in a random order, none repeated within dk tokens
        order = torch.argsort(rand((B, H, dk), seed, KEY_INDEX, device), dim=-1)
        idx = order[..., torch.arange(T, device=device) % dk]
        return torch.nn.functional.one_hot(idx, dk).to(torch.float32)
    if keys == "pool":
        dirs = randn((B, H, pool, dk), seed, KEY_POOL, device)
        idx = (idx_src * pool).long().clamp_max(pool - 1)
        return torch.gather(dirs, 2, idx[..., None].expand(B, H, T, dk))
    raise ValueError(f"unknown key regime {keys!r}")


def gdn_inputs(B, H, T, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu", normalize=True,
               a_range=(-2.0, 4.0), alpha_one=False, beta="sigmoid", keys="random", pool=16,
               q_is_k=False):
    q = randn((B, H, T, dk), seed, Q, device)
    k = _keys(B, H, T, dk, keys, pool, seed, device)
    if normalize:
        q, k = _l2norm_rows(q), _l2norm_rows(k)
    if q_is_k:
        q = k.clone()
    v = randn((B, H, T, dv), seed, V, device)
    alpha, b = decay_and_strength((B, H, T), seed, device, a_lo=a_range[0], a_hi=a_range[1])
    if alpha_one:
        alpha = torch.ones_like(alpha)
    if beta == "zero":
        b = torch.zeros_like(b)
    elif beta == "one":
        b = torch.ones_like(b)
    elif beta != "sigmoid":
        raise ValueError(f"unknown beta regime {beta!r}")
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), alpha=alpha.to(dtype),
                beta=b.to(dtype))


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
