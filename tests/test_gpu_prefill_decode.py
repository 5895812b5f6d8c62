"""GPU prefill followed by GPU decode steps from its end state, against the fp64 oracle run
over the whole sequence at once (GPU, through the C ABI).

A caller serves a sequence by prefilling the prompt and then stepping token by token from
the state the prefill returned (the per-chunk state hand-over of the NoteBank paper's
Algorithm 1, Sec. 3.2).  The prefill's end state [B][H][d_v][d_k] (BASED: s [B][H][D][d_v],
z [B][H][D]) is the decode's state array of B x H entries without a copy or a transpose,
so the n decode outputs must be the oracle's outputs for tokens T .. T + n - 1 of one
prefill over T + n tokens, and the final state its end state.  Bounds as for every bf16
parity check: 2e-2 per (b, h) slice, max-norm relative."""

import pytest
import torch

import oracle
import synth
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
BASED_VARIANTS = ("based", "based_compact")


def _inputs(variant, B, H, T, dk, dv, seed, slow):
    if variant in BASED_VARIANTS:
        d = synth.based_inputs(B, H, T, dk, dv, dtype=torch.bfloat16, seed=seed, device=DEV)
        return d["q"], d["k"], d["v"], None, None
    extra = dict(a_range=(-8.0, -4.0)) if slow else {}
    d = synth.gdn_inputs(B, H, T, dk, dv, dtype=torch.bfloat16, seed=seed, device=DEV,
                         normalize=(variant == "gated_delta"), **extra)
    if variant == "additive":
        return d["q"], d["k"], d["v"], None, None
    return d["q"], d["k"], d["v"], d["alpha"], d["beta"]


CASES = [("additive", 128, False), ("gated", 128, True), ("gated_delta", 128, False),
         ("gated_delta", 128, True), ("gated_delta", 256, True), ("based", 16, False),
         ("based_compact", 16, False)]


@pytest.mark.parametrize("variant,dk,slow", CASES, ids=lambda c: str(c))
def test_prefill_then_decode_matches_one_prefill(la, variant, dk, slow):
    B, H, T, n = 2, 3, 64 * 7 + 19, 6
    dv = 64 if variant in BASED_VARIANTS else dk
    q, k, v, a, b = _inputs(variant, B, H, T + n, dk, dv, seed=300 + dk, slow=slow)
    head = lambda x: None if x is None else x[:, :, :T].contiguous()
    nseg, _ = la.segments(variant, la.BF16, B, H, T, dk, dv)
    print(f"[prefill+decode] {variant} d={dk}/{dv} slow={slow} B={B} H={H} T={T} n={n} "
          f"segments={nseg}", flush=True)
    _, S, z = la.prefill(variant, head(q), head(k), head(v), head(a), head(b))
    N = B * H
    S = S.view(N, *S.shape[2:])  # the same memory: [B][H] -> N states
    if z is not None:
        z = z.view(N, -1)
    outs = []
    for t in range(T, T + n):
        tok = lambda x: None if x is None else x[:, :, t].reshape(N, *x.shape[3:]).contiguous()
        o, S, z = la.decode_step(variant, S, tok(q), tok(k), tok(v), tok(a), tok(b), z=z, S_out=S, z_out=z)
        outs.append(o.view(B, H, dv))
    torch.cuda.synchronize()
    oo, So, zo = oracle.prefill(variant, q, k, v, a, b)
    tol = TOL[torch.bfloat16]
    assert_close(torch.stack(outs, dim=2), oo[:, :, T:], tol, what="decode o")
    assert_close(S.view(B, H, *S.shape[1:]), So, tol, what="S after decode")
    if variant in BASED_VARIANTS:
        assert_close(z.view(B, H, -1), zo, tol, what="z after decode")
