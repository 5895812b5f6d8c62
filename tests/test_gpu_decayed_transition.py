"""GPU parity of the gated-delta prefill when the segment transitions decay to exactly zero
(GPU, through the C ABI).

The map pass first carries the last 8 chunks of a segment; when the transition over them
is exactly zero in fp32 (every product of decays below the smallest fp32 value), the
segment's map is theirs and its earlier chunks are not carried (Eq. (1) of "History
Replays Itself", Sec. 2, with A_t = alpha_t (I - beta_t k_t k_t^T): a map composes as
M = M_first M_last, B = B_first M_last + B_last).  Otherwise it carries the whole segment,
and stops updating a wave of transition rows once every entry is exactly zero.  One call in
the first test holds heads with fast decay (alpha = exp(-softplus(a)), a ~ U(-2, 4): the
transition is zero after a chunk or two) beside heads with slow decay (a ~ U(-8, -4): it
survives every segment), with a start state and a ragged tail; the test checks on the maps
the map pass leaves in the workspace that both regimes occur.  The second alternates fast
and slow decay in blocks of 8 chunks inside every head, so that some segments end in a
zero window and others carry everything.  The third keeps slow decay but resets the state
twice inside every window (alpha = 1e-30 on two tokens).  All compare o and S_T with the
fp64 oracle on sampled value rows (bound 2e-2 per (b, h) slice, max-norm relative)."""

import pytest
import torch

import oracle
import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mixed_inputs(H, T, D, seed):
    fast = synth.gdn_inputs(1, H // 2, T, D, D, dtype=torch.bfloat16, seed=seed, device=DEV)
    slow = synth.gdn_inputs(1, H // 2, T, D, D, dtype=torch.bfloat16, seed=seed + 1, device=DEV,
                            a_range=(-8.0, -4.0))
    return {key: torch.cat([fast[key], slow[key]], dim=1).contiguous()
            for key in ("q", "k", "v", "alpha", "beta")}


@pytest.mark.parametrize("D,H,T", [(128, 32, 64 * 200 + 21), (256, 16, 64 * 16 * 12 + 5)])
def test_decayed_transitions_skip_exactly(la, D, H, T):
    d = _mixed_inputs(H, T, D, seed=500 + D)
    q, k, v, a, b = d["q"], d["k"], d["v"], d["alpha"], d["beta"]
    S0 = synth.gdn_state((1, H, D, D), seed=510 + D, device=DEV) * 0.2
    nseg, sc = la.segments("gated_delta", la.BF16, 1, H, T, D, D)
    print(f"[decayed] d={D} H={H} T={T} segments={nseg}x{sc}", flush=True)
    assert nseg > 1 and sc > 8  # segments long enough for the map pass to check its rows

    # the maps (workspace offset 0: [H][nseg][B rows, then transition rows][D] fp32)
    ws = torch.empty(la.workspace_size("gated_delta", la.BF16, 1, H, T, D, D), dtype=torch.uint8, device=DEV)
    o_, S_ = torch.empty_like(v), torch.empty((1, H, D, D), dtype=torch.float32, device=DEV)
    for p in (la.PASS_TRANSFORM, la.PASS_MAPS):
        la.prefill("gated_delta", q, k, v, a, b, S0=S0, o=o_, S_T=S_, workspace=ws, pass_=p)
    torch.cuda.synchronize()
    maps = ws[: H * nseg * 2 * D * D * 4].view(torch.float32).view(H, nseg, 2 * D, D)
    trans = maps[:, : nseg - 1, D:, :].abs().amax(dim=(-1, -2))  # [H, nseg - 1]
    assert torch.all(trans[: H // 2] == 0), "fast-decay transitions should be exactly zero"
    assert torch.all(trans[H // 2:] > 0), "slow-decay transitions should survive"

    rows = [0, 37, D // 2, D - 1]
    o, S_T, _ = la.prefill("gated_delta", q, k, v, a, b, S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill("gated_delta", q, k, v, a, b, S0=S0, rows=rows)
    assert_close(o[..., rows], oo, 2e-2, what="o (sampled rows)")
    assert_close(S_T[:, :, rows, :], So, 2e-2, what="S_T (sampled rows)")


@pytest.mark.parametrize("D,H,T", [(128, 32, 64 * 200 + 21), (256, 16, 64 * 16 * 12 + 5)])
def test_decay_changing_inside_segments(la, D, H, T):
    fast = synth.gdn_inputs(1, H, T, D, D, dtype=torch.bfloat16, seed=520 + D, device=DEV)
    slow = synth.gdn_inputs(1, H, T, D, D, dtype=torch.bfloat16, seed=530 + D, device=DEV,
                            a_range=(-8.0, -4.0))
    block = (torch.arange(T, device=DEV) // 512) % 2 == 0  # fast decay in even 8-chunk blocks
    alpha = torch.where(block, fast["alpha"], slow["alpha"]).contiguous()
    q, k, v, b = fast["q"], fast["k"], fast["v"], fast["beta"]
    S0 = synth.gdn_state((1, H, D, D), seed=540 + D, device=DEV) * 0.2
    nseg, sc = la.segments("gated_delta", la.BF16, 1, H, T, D, D)
    print(f"[decay blocks] d={D} H={H} T={T} segments={nseg}x{sc}", flush=True)
    rows = [1, 64, D - 2]
    o, S_T, _ = la.prefill("gated_delta", q, k, v, alpha, b, S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill("gated_delta", q, k, v, alpha, b, S0=S0, rows=rows)
    assert_close(o[..., rows], oo, 2e-2, what="o (sampled rows)")
    assert_close(S_T[:, :, rows, :], So, 2e-2, what="S_T (sampled rows)")


@pytest.mark.parametrize("D,H,T", [(128, 16, 64 * 16 * 24), (256, 8, 64 * 32 * 24)])
def test_sparse_resets_inside_windows(la, D, H, T):
    """Slow decay everywhere except two tokens per segment, inside its last 8 chunks, whose
    decay (alpha = 1e-30) takes the transition to exactly zero in fp32: every map is then
    formed from its window alone, though the window itself carries a long slow-decay
    history, and the scan has nothing to chain."""
    nseg, sc = la.segments("gated_delta", la.BF16, 1, H, T, D, D)
    print(f"[sparse resets] d={D} H={H} T={T} segments={nseg}x{sc}", flush=True)
    assert nseg > 1 and sc > 16
    d = synth.gdn_inputs(1, H, T, D, D, dtype=torch.bfloat16, seed=550 + D, device=DEV, a_range=(-8.0, -4.0))
    alpha = d["alpha"].clone()
    for s0 in range(0, T, 64 * sc):
        for off in (100, 300):
            t = s0 + 64 * (sc - 8) + off
            if t < T:
                alpha[:, :, t] = 1e-30
    S0 = synth.gdn_state((1, H, D, D), seed=560 + D, device=DEV) * 0.2
    # the maps (workspace offset 0): every mapped segment's transition is exactly zero
    ws = torch.empty(la.workspace_size("gated_delta", la.BF16, 1, H, T, D, D), dtype=torch.uint8, device=DEV)
    o_, S_ = torch.empty_like(d["v"]), torch.empty((1, H, D, D), dtype=torch.float32, device=DEV)
    for p in (la.PASS_TRANSFORM, la.PASS_MAPS):
        la.prefill("gated_delta", d["q"], d["k"], d["v"], alpha, d["beta"], S0=S0, o=o_, S_T=S_, workspace=ws, pass_=p)
    torch.cuda.synchronize()
    maps = ws[: H * nseg * 2 * D * D * 4].view(torch.float32).view(H, nseg, 2 * D, D)
    assert torch.all(maps[:, : nseg - 1, D:, :] == 0), "the resets should zero every window's transition"
    assert torch.all(maps[:, : nseg - 1, :D, :].abs().amax(dim=(-1, -2)) > 0)
    rows = [3, D // 2 + 1, D - 1]
    o, S_T, _ = la.prefill("gated_delta", d["q"], d["k"], d["v"], alpha, d["beta"], S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill("gated_delta", d["q"], d["k"], d["v"], alpha, d["beta"], S0=S0, rows=rows)
    assert_close(o[..., rows], oo, 2e-2, what="o (sampled rows)")
    assert_close(S_T[:, :, rows, :], So, 2e-2, what="S_T (sampled rows)")
