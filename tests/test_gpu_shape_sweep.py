"""Randomized shape sweep of the prefill against the fp64 oracle (GPU, through the C ABI).

Thirty-six seeded cases over the variants (additive, gated, gated delta, BASED full and compact),
input types (bf16; fp32 for a quarter), key widths (64, 128, 256 for the gated recurrences),
batch and head counts (1-3 x 1-5) and sequence lengths (1 to a few thousand tokens, ragged
tails, chunk multiples and their neighbours), half of them with a start state and half of
the gated ones with slow decay (a ~ U(-8, -4): the carry across chunks and segments
matters).  Small head counts make the segment plan split even short sequences into many
one- and few-chunk segments, so the map, scan and replay passes run at every size.  Each
case is compared element by element on every output (bound 2e-2 for bf16 inputs, 1e-4 for
fp32, per (b, h) slice, max-norm relative)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
BASED_VARIANTS = ("based", "based_compact")


def _cases(n=36, seed=20261202):
    rng = np.random.RandomState(seed)
    out = []
    names = ["additive", "gated", "gated_delta", "based", "based_compact"]
    for i in range(n):
        variant = names[rng.choice(5, p=[0.15, 0.2, 0.35, 0.15, 0.15])]
        dtype = torch.float32 if rng.rand() < 0.25 else torch.bfloat16
        if variant in BASED_VARIANTS:
            dk, dv, tmax = 16, 64, 2600
        elif dtype == torch.bfloat16:
            dk = dv = [128, 128, 256][rng.randint(3)]
            tmax = 1200 if dk == 256 else 2600
        else:
            dk = dv = [64, 128, 256][rng.randint(3)]
            tmax = 700 if dk == 256 else 1500
        B, H = 1 + rng.randint(3), 1 + rng.randint(5)
        kind = rng.randint(4)
        if kind == 0:
            T = 64 * (1 + rng.randint(tmax // 64))      # whole chunks
        elif kind == 1:
            T = 64 * (1 + rng.randint(tmax // 64)) + [-1, 1][rng.randint(2)]
        else:
            T = 1 + rng.randint(tmax)
        start = bool(rng.rand() < 0.5)
        slow = variant in ("gated", "gated_delta") and bool(rng.rand() < 0.5)
        out.append((i, variant, dtype, B, H, T, dk, dv, start, slow))
    return out


def _inputs(variant, B, H, T, dk, dv, dtype, seed, slow):
    if variant in BASED_VARIANTS:
        d = synth.based_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, device=DEV)
        return d["q"], d["k"], d["v"], None, None
    extra = dict(a_range=(-8.0, -4.0)) if slow else {}
    d = synth.gdn_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, device=DEV,
                         normalize=(variant == "gated_delta"), **extra)
    if variant == "additive":
        return d["q"], d["k"], d["v"], None, None
    return d["q"], d["k"], d["v"], d["alpha"], d["beta"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-{'fp32' if c[2] == torch.float32 else 'bf16'}-"
                                                      f"B{c[3]}H{c[4]}T{c[5]}d{c[6]}{'-S0' if c[8] else ''}{'-slow' if c[9] else ''}")
def test_prefill_shape_sweep(la, case):
    i, variant, dtype, B, H, T, dk, dv, start, slow = case
    seed = 7000 + i
    q, k, v, a, b = _inputs(variant, B, H, T, dk, dv, dtype, seed, slow)
    S0 = z0 = None
    if start:
        if variant in BASED_VARIANTS:  # a reachable state: a short prefix's end state
            w = synth.based_inputs(B, H, 37, dk, dv, dtype=dtype, seed=seed + 1, device=DEV)
            _, s0, zz = oracle.prefill(variant, w["q"], w["k"], w["v"])
            S0 = torch.tensor(s0, dtype=torch.float32, device=DEV)
            z0 = torch.tensor(zz, dtype=torch.float32, device=DEV)
        else:
            S0 = synth.gdn_state((B, H, dv, dk), seed=seed + 1, device=DEV) * 0.2
    nseg, sc = la.segments(variant, la.BF16 if dtype == torch.bfloat16 else la.F32, B, H, T, dk, dv)
    print(f"[sweep {i}] {variant} {dtype} B={B} H={H} T={T} d={dk}/{dv} S0={start} slow={slow} "
          f"segments={nseg}x{sc}", flush=True)
    o, S_T, z_T = la.prefill(variant, q, k, v, a, b, S0=S0, z0=z0)
    torch.cuda.synchronize()
    oo, So, zo = oracle.prefill(variant, q, k, v, a, b, S0=S0, z0=z0)
    tol = TOL[dtype]
    assert_close(o, oo, tol, what="o")
    assert_close(S_T, So, tol, what="S_T")
    if variant in BASED_VARIANTS:
        assert_close(z_T, zo, tol, what="z_T")
