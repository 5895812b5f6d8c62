"""Randomized GPU sweep of the map pass's window (through the C ABI), against the fp64
oracle on sampled value rows.

Twelve seeded cases with segments long enough for the window (17 to 40 chunks), over the
gated and gated-delta variants, key widths 128 and 256, 1-16 heads, ragged lengths, start
states, and four gate regimes: the recipe's fast decay (every window's transition zero),
slow decay (none), fast and slow decay alternating in blocks inside the segments, and slow
decay with two state resets (alpha = 1e-30) at random places.  Bound 2e-2 per (b, h)
slice, max-norm relative, on o and S_T."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
MODES = ("fast", "slow", "blocks", "resets")


def _cases(n=12, seed=20261203):
    rng = np.random.RandomState(seed)
    out = []
    for i in range(n):
        variant = ["gated", "gated_delta"][rng.randint(2)]
        D = [128, 128, 256][rng.randint(3)]
        H = int(rng.choice([1, 2, 4, 8, 16]))
        mode = MODES[i % 4]
        out.append((i, variant, D, H, mode, int(rng.randint(17, 41)), int(rng.randint(0, 64)), bool(rng.rand() < 0.5)))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-d{c[2]}-H{c[3]}-{c[4]}")
def test_window_sweep(la, case):
    i, variant, D, H, mode, want_sc, tail, start = case
    # a length whose plan gives several segments of more than 16 chunks (the window's bar)
    n = la.segments(variant, la.BF16, 1, H, 64 * 100000, D, D)[0]
    while True:
        T = 64 * want_sc * n - tail
        nseg, sc = la.segments(variant, la.BF16, 1, H, T, D, D)
        if sc > 16 or n <= 2:
            break
        n //= 2
    assert nseg > 1 and sc > 16
    seed = 9000 + i
    fast = synth.gdn_inputs(1, H, T, D, D, dtype=torch.bfloat16, seed=seed, device=DEV,
                            normalize=(variant == "gated_delta"))
    slow = synth.gdn_inputs(1, H, T, D, D, dtype=torch.bfloat16, seed=seed + 1, device=DEV,
                            normalize=(variant == "gated_delta"), a_range=(-8.0, -4.0))
    q, k, v, b = fast["q"], fast["k"], fast["v"], fast["beta"]
    if mode == "fast":
        a = fast["alpha"]
    elif mode == "slow":
        a = slow["alpha"]
    elif mode == "blocks":
        block = (torch.arange(T, device=DEV) // (64 * 5)) % 2 == 0
        a = torch.where(block, fast["alpha"], slow["alpha"]).contiguous()
    else:
        a = slow["alpha"].clone()
        g = torch.Generator().manual_seed(seed)
        for t in torch.randint(0, T, (2,), generator=g).tolist():
            a[:, :, t] = 1e-30
    S0 = synth.gdn_state((1, H, D, D), seed=seed + 2, device=DEV) * 0.2 if start else None
    print(f"[window sweep {i}] {variant} d={D} H={H} T={T} {mode} S0={start} segments={nseg}x{sc}", flush=True)
    rows = [0, D // 3, D - 1]
    o, S_T, _ = la.prefill(variant, q, k, v, a, b, S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill(variant, q, k, v, a, b, S0=S0, rows=rows)
    assert_close(o[..., rows], oo, 2e-2, what="o (sampled rows)")
    assert_close(S_T[:, :, rows, :], So, 2e-2, what="S_T (sampled rows)")
