"""GPU parity of the chunkwise bf16 prefill at the gated-delta shape of the NoteBank paper's
own backbone (8 heads of width 256 per layer, "History Replays Itself", App. C on the GDN
configuration): d_k = d_v = 256, fp32 state 256 x 256 per head.  At this width a replay
workgroup carries a whole state (eight waves of 32 value rows), and the segment maps are
512 rows (256 B rows, 256 transition rows) split over two map workgroups, each with half
of the B rows and the transition rows of the same indices.  Every call goes through the C
ABI and is compared with the fp64 oracle on the same seeded inputs (bound 2e-2, per (b, h)
slice, max-norm relative)."""

import pytest
import torch

import oracle
import synth
from tests.parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 256
VARIANTS = ["additive", "gated", "gated_delta"]


def _inputs(variant, B, H, T, seed):
    d = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=seed, device=DEV,
                         normalize=(variant == "gated_delta"))
    if variant == "additive":
        return d["q"], d["k"], d["v"], None, None
    return d["q"], d["k"], d["v"], d["alpha"], d["beta"]


def _check(la, variant, B, H, T, seed, S0=None, rows=None):
    q, k, v, a, b = _inputs(variant, B, H, T, seed)
    nseg, sc = la.segments(variant, la.BF16, B, H, T, D, D)
    print(f"[d256] {variant} B={B} H={H} T={T} segments={nseg}x{sc} rows={rows}", flush=True)
    o, S_T, _ = la.prefill(variant, q, k, v, a, b, S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill(variant, q, k, v, a, b, S0=S0, rows=rows)
    if rows is None:
        assert_close(o, oo, 2e-2, what="o")
        assert_close(S_T, So, 2e-2, what="S_T")
    else:
        assert_close(o[..., rows], oo, 2e-2, what="o (sampled rows)")
        assert_close(S_T[:, :, rows, :], So, 2e-2, what="S_T (sampled rows)")
    return nseg, sc


@pytest.mark.parametrize("variant", VARIANTS)
def test_d256_small_ragged(la, variant):
    # 2 heads: four one-chunk segments (one per chunk), the last one partial
    nseg, _ = _check(la, variant, 1, 2, 203, seed=81)
    assert nseg == 4


@pytest.mark.parametrize("variant", VARIANTS)
def test_d256_multi_chunk_segments(la, variant):
    # 4 heads: 60 segments of 5 chunks; value rows sampled from both map workgroups' halves
    nseg, sc = _check(la, variant, 1, 4, 64 * 300 - 17, seed=82, rows=[0, 101, 127, 128, 200, 255])
    assert nseg > 8 and sc > 1


@pytest.mark.parametrize("variant", VARIANTS)
def test_d256_with_start_state(la, variant):
    S0 = synth.gdn_state((1, 2, D, D), seed=83, device=DEV) * 0.2
    _check(la, variant, 1, 2, 64 * 9 + 5, seed=84, S0=S0)


@pytest.mark.parametrize("variant", VARIANTS)
def test_d256_batched_segments(la, variant):
    # B = 3 x H = 2: several segments per (b, h), start states, a ragged tail
    S0 = synth.gdn_state((3, 2, D, D), seed=93, device=DEV) * 0.2
    nseg, _ = _check(la, variant, 3, 2, 64 * 11 + 33, seed=94, S0=S0, rows=[0, 64, 127, 128, 191, 255])
    assert nseg > 1


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("T", [1, 63, 64, 65])
def test_d256_short_sequences(la, variant, T):
    _check(la, variant, 1, 2, T, seed=90 + T)


@pytest.mark.parametrize("variant", VARIANTS)
def test_d256_single_segment_many_heads(la, variant):
    # 128 heads (one workgroup of all 256 state rows each): one segment, the replay alone from S0
    S0 = synth.gdn_state((8, 16, D, D), seed=85, device=DEV) * 0.1
    nseg, _ = _check(la, variant, 8, 16, 64 * 2 + 7, seed=86, S0=S0, rows=[2, 127, 128, 254])
    assert nseg == 1


@pytest.mark.parametrize("variant", VARIANTS)
def test_d256_passes_compose_to_prefill(la, variant):
    """la_prefill == la_prefill_pass(TRANSFORM); (MAPS); (SCAN); (REPLAY), bit for bit."""
    B, H, T = 1, 3, 64 * 40 + 9
    q, k, v, a, b = _inputs(variant, B, H, T, 87)
    nseg, _ = la.segments(variant, la.BF16, B, H, T, D, D)
    assert nseg > 1
    S0 = synth.gdn_state((B, H, D, D), seed=88, device=DEV) * 0.1
    o1, S1, _ = la.prefill(variant, q, k, v, a, b, S0=S0)
    ws = torch.empty(la.workspace_size(variant, la.BF16, B, H, T, D, D), dtype=torch.uint8, device=DEV)
    o2, S2 = torch.empty_like(o1), torch.empty_like(S1)
    for p in (la.PASS_TRANSFORM, la.PASS_MAPS, la.PASS_SCAN, la.PASS_REPLAY):
        la.prefill(variant, q, k, v, a, b, S0=S0, o=o2, S_T=S2, workspace=ws, pass_=p)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_d256_deterministic(la):
    q, k, v, a, b = _inputs("gated_delta", 1, 2, 64 * 30 + 3, 89)
    o1, S1, _ = la.prefill("gated_delta", q, k, v, a, b)
    o2, S2, _ = la.prefill("gated_delta", q, k, v, a, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_d256_split_resume(la):
    """prefill(x[:a]) then prefill(x[a:], S0=S_a) matches one prefill(x)."""
    q, k, v, a, b = _inputs("gated_delta", 1, 2, 1500, 90)
    o, S, _ = la.prefill("gated_delta", q, k, v, a, b)
    cut = 640
    c = lambda t, sl: t[:, :, sl].contiguous()
    o1, S1, _ = la.prefill("gated_delta", c(q, slice(0, cut)), c(k, slice(0, cut)), c(v, slice(0, cut)),
                           c(a, slice(0, cut)), c(b, slice(0, cut)))
    o2, S2, _ = la.prefill("gated_delta", c(q, slice(cut, None)), c(k, slice(cut, None)),
                           c(v, slice(cut, None)), c(a, slice(cut, None)), c(b, slice(cut, None)), S0=S1)
    torch.cuda.synchronize()
    assert_close(torch.cat([o1, o2], dim=2), o, 2e-2, what="o split")
    assert_close(S2, S, 2e-2, what="S split")
