"""la_prefill_noalloc (include/la.h): the prefill with its workspace in the library's static
device scratch, for callers that cannot allocate.  Checked through the C ABI against
la_prefill's output on the same inputs, on calls in a row with the second smaller than the
first (the scratch keeps the previous call's contents): bit for bit where both use the same
segment plan, within the bf16 bound (2e-2, per slice, tests/parity.py) where the scratch
forces fewer segments, and against the fp64 oracle on sampled rows."""

import pytest
import torch

import oracle
import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gdn(B, H, T, seed, d=128):
    x = synth.gdn_inputs(B, H, T, d, d, dtype=torch.bfloat16, seed=seed, device=DEV)
    return x["q"], x["k"], x["v"], x["alpha"], x["beta"]


def test_noalloc_matches_prefill_two_calls_second_smaller(la):
    # call 1: 8 heads of 256 x 65536 tokens.  la_prefill's workspace (32 segments per head, a
    # stored transform per chunk) exceeds the scratch, so the no-alloc call runs fewer, longer
    # segments
    B, H, T, D = 1, 8, 65536, 256
    x = _gdn(B, H, T, 31, D)
    S0 = synth.gdn_state((B, H, D, D), seed=31, device=DEV) * 0.3
    assert la.workspace_size("gated_delta", la.BF16, B, H, T, D, D) > la.NOALLOC_SCRATCH_BYTES
    print(f"[noalloc] call 1: gated_delta B={B} H={H} T={T} d={D} (capped plan)", flush=True)
    o_ref, S_ref, _ = la.prefill("gated_delta", *x, S0=S0)
    o1, S1 = torch.empty_like(o_ref), torch.empty_like(S_ref)
    la.prefill_noalloc("gated_delta", *x, S0=S0, o=o1, S_T=S1)
    torch.cuda.synchronize()
    assert_close(o1, o_ref.float(), 2e-2, what="noalloc o vs la_prefill (call 1)")
    assert_close(S1, S_ref, 2e-2, what="noalloc S_T vs la_prefill (call 1)")
    rows = [0, 77, 255]
    oo, So, _ = oracle.prefill("gated_delta", *x, S0=S0, rows=rows)
    assert_close(o1[..., rows], oo, 2e-2, what="noalloc o vs oracle (call 1, sampled rows)")
    assert_close(S1[:, :, rows], So, 2e-2, what="noalloc S_T vs oracle (call 1, sampled rows)")
    del x, o_ref, o1

    # call 2: a smaller problem (d = 128) whose la_prefill workspace fits: the same plan, bit
    # for bit
    B, H, T = 1, 4, 64 * 40 + 5
    x = _gdn(B, H, T, 32)
    assert la.workspace_size("gated_delta", la.BF16, B, H, T, 128, 128) <= la.NOALLOC_SCRATCH_BYTES
    print(f"[noalloc] call 2: gated_delta B={B} H={H} T={T} (same plan)", flush=True)
    o_ref, S_ref, _ = la.prefill("gated_delta", *x)
    o2, S2 = torch.empty_like(o_ref), torch.empty_like(S_ref)
    la.prefill_noalloc("gated_delta", *x, o=o2, S_T=S2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(S2, S_ref)

    # call 3: BASED at its full configuration (its workspace fits): bit for bit
    d = synth.based_inputs(4, 16, 8192, 16, 64, dtype=torch.bfloat16, seed=33, device=DEV)
    print("[noalloc] call 3: based B=4 H=16 T=8192 (same plan)", flush=True)
    o_ref, s_ref, z_ref = la.prefill("based", d["q"], d["k"], d["v"])
    o3, s3, z3 = la.prefill_noalloc("based", d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    assert torch.equal(o3, o_ref) and torch.equal(s3, s_ref) and torch.equal(z3, z_ref)


def test_noalloc_rejects_problems_beyond_the_scratch(la):
    # 8 heads of 256 x 1M tokens: the per-chunk transforms alone exceed the scratch
    B, H, T, D = 1, 8, 1 << 20, 256
    e = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((B, H, T), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LAError) as err:
        la.prefill_noalloc("gated_delta", e, e, e, g, g, o=torch.empty_like(e),
                           S_T=torch.empty((B, H, D, D), device=DEV))
    assert err.value.status == -5  # LA_ERR_WORKSPACE


def test_noalloc_runs_the_million_token_prefill(la):
    """At d = 128 the workspace holds the segment maps and start states only (the map and
    replay passes form each chunk's solve where they use it), at most about 96 MiB: the
    1M-token, 16-head prefill runs in the static scratch with la_prefill's own plan, bit for
    bit."""
    B, H, T = 1, 16, 1 << 20
    assert la.workspace_size("gated_delta", la.BF16, B, H, T, 128, 128) <= la.NOALLOC_SCRATCH_BYTES
    x = _gdn(B, H, T, 34)
    print(f"[noalloc] gated_delta B={B} H={H} T={T} (same plan)", flush=True)
    o_ref, S_ref, _ = la.prefill("gated_delta", *x)
    o, S = torch.empty_like(o_ref), torch.empty_like(S_ref)
    la.prefill_noalloc("gated_delta", *x, o=o, S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
