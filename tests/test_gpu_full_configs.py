"""Parity at the full sizes of the five benchmark configurations, in the launch
configuration bench.py uses.  Where the fp64 oracle cannot cover everything in seconds
it computes sampled outputs exactly: value rows (gated family) and value columns
(BASED) evolve independently, so the oracle runs only those, over the whole sequence.

  cfg0  additive, B=1 H=1 T=1024 d=64, fp32             -- everything, bound 1e-4
  cfg1  BASED, B=4 H=16 T=8192 d'=16 d_v=64, bf16        -- in test_gpu_parity.py
  cfg2  gated delta, B=1 H=16 T=65536 d=128, bf16        -- all heads, 3 rows each
  cfg3  gated delta, B=1 H=16 T=1048576 d=128, bf16      -- 2 heads x 3 rows, whole T
  cfg4  decode, 256 x 16 states, 1024 steps, GDN + BASED -- o at every step and the
        final state, for 24 sampled states of each kind
  gated delta at the NoteBank paper's own head shape, B=1 H=8 T=1048576 d=256, bf16
        -- 2 heads x 4 rows (both halves of the state), whole T
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_cfg0_additive_fp32(la):
    d = synth.additive_inputs(1, 1, 1024, 64, dtype=torch.float32, seed=0, device=DEV)
    o, S, _ = la.prefill("additive", d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill("additive", d["q"], d["k"], d["v"])
    assert_close(o, oo, 1e-4, what="cfg0 o")
    assert_close(S, So, 1e-4, what="cfg0 S_T")


def _gdn_sampled(la, T, heads, rows, seed, H=16, D=128):
    B = 1
    d = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=seed, device=DEV)
    nseg, sc = la.segments("gated_delta", la.BF16, B, H, T, D, D)
    print(f"[gdn T={T} H={H} d={D}] segments={nseg} x {sc} chunks", flush=True)
    o, S, _ = la.prefill("gated_delta", d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    hs = list(heads)
    sub = {n: t[:, hs] for n, t in d.items()}
    oo, So, _ = oracle.prefill("gated_delta", sub["q"], sub["k"], sub["v"], sub["alpha"],
                               sub["beta"], rows=rows)
    assert_close(o[:, hs][..., rows], oo, 2e-2, what=f"T={T} o (heads {hs}, rows {rows})")
    assert_close(S[:, hs][:, :, rows, :], So, 2e-2, what=f"T={T} S_T (heads {hs}, rows {rows})")


def test_cfg2_gdn_64k_all_heads_sampled_rows(la):
    _gdn_sampled(la, 65536, range(16), [0, 77, 127], seed=2)


def test_cfg3_gdn_1m_sampled(la):
    _gdn_sampled(la, 1 << 20, [0, 15], [3, 64, 126], seed=3)


def test_gdn_8x256_1m_sampled(la):
    # the NoteBank paper's own GDN head shape (8 heads of width 256) at 1M tokens, in the
    # launch configuration bench.py times (32 segments per head, one replay workgroup and two
    # map workgroups each); sampled rows from both map workgroups' halves, whole sequence
    _gdn_sampled(la, 1 << 20, [0, 7], [5, 127, 128, 250], seed=6, H=8, D=256)


def test_cfg4_decode_1024_steps_sampled_states(la):
    N, D, steps = 256 * 16, 128, 1024
    idx = torch.linspace(0, N - 1, 24).long().tolist()
    # gated delta: seeded N(0,1) start states
    S = synth.gdn_state((N, D, D), seed=4, device=DEV)
    S_ref0 = S[idx].clone()
    g = synth.gdn_decode_inputs(steps, N, D, D, dtype=torch.bfloat16, seed=4, device=DEV)
    outs = torch.empty((steps, len(idx), D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    for t in range(steps):
        la.decode_step("gated_delta", S, g["q"][t], g["k"][t], g["v"][t], g["alpha"][t],
                       g["beta"][t], S_out=S, o=o)
        outs[t] = o[idx]
    torch.cuda.synchronize()
    # the oracle runs the same 1024 tokens as one recurrence per sampled state
    tq = lambda n: g[n][:, idx].transpose(0, 1).contiguous()[None]  # [1, states, steps, ...]
    oo, So, _ = oracle.prefill("gated_delta", tq("q"), tq("k"), tq("v"), tq("alpha"), tq("beta"),
                               S0=S_ref0[None])
    assert_close(outs.transpose(0, 1)[None], oo, 2e-2, what="cfg4 GDN o, every step")
    assert_close(S[idx][None], So, 2e-2, what="cfg4 GDN final state")

    # BASED: start states from a 64-token warm-up run by each side on the same tokens
    dp, dvb = 16, 64
    w = synth.based_warmup_inputs(N, 64, dp, dvb, dtype=torch.bfloat16, seed=4, device=DEV)
    _, s, z = la.prefill("based", w["q"][None], w["k"][None], w["v"][None])
    s, z = s[0].contiguous(), z[0].contiguous()
    bd = synth.based_decode_inputs(steps, N, dp, dvb, dtype=torch.bfloat16, seed=5, device=DEV)
    outs_b = torch.empty((steps, len(idx), dvb), dtype=torch.bfloat16, device=DEV)
    ob = torch.empty((N, dvb), dtype=torch.bfloat16, device=DEV)
    for t in range(steps):
        la.decode_step("based", s, bd["q"][t], bd["k"][t], bd["v"][t], z=z, S_out=s, z_out=z, o=ob)
        outs_b[t] = ob[idx]
    torch.cuda.synchronize()
    wq = lambda n: torch.cat([w[n][idx], bd[n][:, idx].transpose(0, 1)], dim=1)[None]
    oo_b, so_b, zo_b = oracle.prefill("based", wq("q"), wq("k"), wq("v"))
    assert_close(outs_b.transpose(0, 1)[None], oo_b[:, :, 64:], 2e-2, what="cfg4 BASED o, every step")
    assert_close(s[idx][None], so_b, 2e-2, what="cfg4 BASED final s")
    assert_close(z[idx][None], zo_b, 2e-2, what="cfg4 BASED final z")


@pytest.mark.parametrize("D,N", [(128, 6144), (256, 2048)])
def test_decode_streaming_state_sets(la, D, N):
    """State sets larger than the Infinity Cache (384 and 512 MiB) take the streaming decode
    kernel (non-temporal accesses, four passes in flight): o at every one of 16 steps and
    the final state, for 16 sampled states, against the oracle run over the same tokens."""
    steps = 16
    idx = torch.linspace(0, N - 1, 16).long().tolist()
    S = synth.gdn_state((N, D, D), seed=15, device=DEV)
    S_ref0 = S[idx].clone()
    g = synth.gdn_decode_inputs(steps, N, D, D, dtype=torch.bfloat16, seed=15, device=DEV)
    outs = torch.empty((steps, len(idx), D), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    print(f"[decode streaming] d={D} N={N} ({N * D * D * 4 >> 20} MiB)", flush=True)
    for t in range(steps):
        la.decode_step("gated_delta", S, g["q"][t], g["k"][t], g["v"][t], g["alpha"][t],
                       g["beta"][t], S_out=S, o=o)
        outs[t] = o[idx]
    torch.cuda.synchronize()
    tq = lambda n: g[n][:, idx].transpose(0, 1).contiguous()[None]
    oo, So, _ = oracle.prefill("gated_delta", tq("q"), tq("k"), tq("v"), tq("alpha"), tq("beta"),
                               S0=S_ref0[None])
    assert_close(outs.transpose(0, 1)[None], oo, 2e-2, what="streaming decode o, every step")
    assert_close(S[idx][None], So, 2e-2, what="streaming decode final state")
