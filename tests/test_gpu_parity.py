"""GPU parity at sizes the oracle finishes in seconds: every call goes through the C ABI
(libla.so) and is compared element by element with the fp64 oracle on the same seeded
inputs.  Error metric and tolerances: tests/parity.py (2e-2 for bf16 inputs, 1e-4 for
fp32 inputs, per (b, h) slice, max-norm relative)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"

ROWS_VARIANTS = ["additive", "gated", "gated_delta"]
BASED_VARIANTS = ["based", "based_compact"]


def _inputs(variant, B, H, T, dk, dv, dtype, seed):
    if variant in BASED_VARIANTS:
        d = synth.based_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, device=DEV)
        return d["q"], d["k"], d["v"], None, None
    d = synth.gdn_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, device=DEV,
                         normalize=(variant == "gated_delta"))
    if variant == "additive":
        return d["q"], d["k"], d["v"], None, None
    return d["q"], d["k"], d["v"], d["alpha"], d["beta"]


def _check_prefill(la, variant, B, H, T, dk, dv, dtype, seed, S0=None, z0=None):
    q, k, v, a, b = _inputs(variant, B, H, T, dk, dv, dtype, seed)
    print(f"[prefill] {variant} B={B} H={H} T={T} dk={dk} dv={dv} {dtype} seed={seed}", flush=True)
    o, S_T, z_T = la.prefill(variant, q, k, v, a, b, S0=S0, z0=z0)
    torch.cuda.synchronize()
    oo, So, zo = oracle.prefill(variant, q, k, v, a, b, S0=S0, z0=z0)
    tol = TOL[dtype]
    assert_close(o, oo, tol, what="o")
    assert_close(S_T, So, tol, what="S_T")
    if variant in BASED_VARIANTS:
        assert_close(z_T, zo, tol, what="z_T")
    return o, S_T, z_T


@pytest.mark.parametrize("variant", ROWS_VARIANTS + BASED_VARIANTS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_small(la, variant, dtype):
    if variant in BASED_VARIANTS:
        _check_prefill(la, variant, 2, 3, 203, 16, 64, dtype, seed=11)
    else:
        for dk in (64, 128):
            _check_prefill(la, variant, 2, 3, 203, dk, dk, dtype, seed=12 + dk)


@pytest.mark.parametrize("variant", ROWS_VARIANTS)
def test_prefill_fp32_other_widths(la, variant):
    _check_prefill(la, variant, 1, 2, 77, 256, 40, torch.float32, seed=3)
    _check_prefill(la, variant, 1, 2, 77, 64, 17, torch.float32, seed=4)


@pytest.mark.parametrize("variant", ["additive", "gated"])
@pytest.mark.parametrize("T", [2048, 2049])
def test_prefill_fp32_attention_form_limit(la, variant, T):
    # fp32 additive/gated prefills of at most 2048 tokens use the masked attention form
    # (parallel over tokens), longer ones the token-recurrent walk: both sides of the limit,
    # with a start state and beta given
    S0 = synth.gdn_state((1, 2, 64, 64), seed=17, device=DEV) * 0.3
    _check_prefill(la, variant, 1, 2, T, 64, 64, torch.float32, seed=18, S0=S0)


@pytest.mark.parametrize("variant", ROWS_VARIANTS + BASED_VARIANTS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_with_start_state(la, variant, dtype):
    B, H, T = 1, 2, 130
    if variant in BASED_VARIANTS:
        dk, dv = 16, 64
        w = synth.based_inputs(B, H, 40, dk, dv, dtype=dtype, seed=99, device=DEV)
        _, s0, z0 = oracle.prefill(variant, w["q"], w["k"], w["v"])
        S0 = torch.tensor(s0, dtype=torch.float32, device=DEV)
        z0 = torch.tensor(z0, dtype=torch.float32, device=DEV)
    else:
        dk = dv = 128
        S0 = synth.gdn_state((B, H, dv, dk), seed=5, device=DEV) * 0.3
        z0 = None
    _check_prefill(la, variant, B, H, T, dk, dv, dtype, seed=21, S0=S0, z0=z0)


@pytest.mark.parametrize("variant", ROWS_VARIANTS + BASED_VARIANTS)
def test_prefill_empty_sequence_returns_start_state(la, variant):
    dk, dv = (16, 64) if variant in BASED_VARIANTS else (128, 128)
    q, k, v, a, b = _inputs(variant, 1, 2, 0, dk, dv, torch.bfloat16, 1)
    if variant in BASED_VARIANTS:
        D = oracle.feature_dim(dk, compact=(variant == "based_compact"))
        S0 = torch.randn(1, 2, D, dv, device=DEV)
        z0 = torch.rand(1, 2, D, device=DEV)
    else:
        S0, z0 = torch.randn(1, 2, dv, dk, device=DEV), None
    o, S_T, z_T = la.prefill(variant, q, k, v, a, b, S0=S0, z0=z0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S_T, S0)
    if z0 is not None:
        assert torch.equal(z_T, z0)
    _, S_T, _ = la.prefill(variant, q, k, v, a, b)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S_T) == 0


@pytest.mark.parametrize("variant", ROWS_VARIANTS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 50), (256, 32), (256, 256), (256, 200)])
def test_decode_steps(la, variant, dtype, dk, dv):
    N, steps = 37, 6
    print(f"[decode] {variant} N={N} dk={dk} dv={dv} {dtype}", flush=True)
    d = synth.gdn_decode_inputs(steps, N, dk, dv, dtype=dtype, seed=7, device=DEV)
    S = synth.gdn_state((N, dv, dk), seed=8, device=DEV)
    S_ref = to64(S)
    tol = TOL[dtype]
    for t in range(steps):
        a = None if variant == "additive" else d["alpha"][t]
        b = None if variant == "additive" else d["beta"][t]
        o, S, _ = la.decode_step(variant, S, d["q"][t], d["k"][t], d["v"][t], a, b, S_out=S)
        torch.cuda.synchronize()
        oo, S_ref, _ = oracle.decode_step(variant, S_ref, d["q"][t], d["k"][t], d["v"][t], a, b)
        assert_close(o, oo, tol, lead=1, what=f"o step {t}")
    assert_close(S, S_ref, tol, lead=1, what="S")


@pytest.mark.parametrize("variant", BASED_VARIANTS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_based_steps(la, variant, dtype):
    N, steps, dp, dv = 29, 5, 16, 64
    w = synth.based_warmup_inputs(N, 24, dp, dv, dtype=dtype, seed=3, device=DEV)
    # both sides build the start state from the same warm-up tokens: the GPU through its
    # own prefill, the oracle through its own recurrence
    _, s, z = la.prefill(variant, w["q"][None], w["k"][None], w["v"][None])
    s, z = s[0].contiguous(), z[0].contiguous()
    _, s_ref, z_ref = oracle.prefill(variant, w["q"][None], w["k"][None], w["v"][None])
    s_ref, z_ref = s_ref[0], z_ref[0]
    d = synth.based_decode_inputs(steps, N, dp, dv, dtype=dtype, seed=4, device=DEV)
    tol = TOL[dtype]
    for t in range(steps):
        o, s, z = la.decode_step(variant, s, d["q"][t], d["k"][t], d["v"][t], z=z, S_out=s, z_out=z)
        torch.cuda.synchronize()
        oo, s_ref, z_ref = oracle.decode_step(variant, s_ref, d["q"][t], d["k"][t], d["v"][t],
                                              z=z_ref)
        assert_close(o, oo, tol, lead=1, what=f"o step {t}")
    assert_close(s, s_ref, tol, lead=1, what="s")
    assert_close(z, z_ref, tol, lead=1, what="z")


@pytest.mark.parametrize("variant", ROWS_VARIANTS + BASED_VARIANTS)
def test_prefill_deterministic(la, variant):
    dk, dv = (16, 64) if variant in BASED_VARIANTS else (128, 128)
    q, k, v, a, b = _inputs(variant, 1, 4, 333, dk, dv, torch.bfloat16, 5)
    o1, S1, _ = la.prefill(variant, q, k, v, a, b)
    o2, S2, _ = la.prefill(variant, q, k, v, a, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def _check_prefill_sampled(la, variant, B, H, T, dk, dv, dtype, seed, rows, S0=None):
    """Parity on a sample of value rows (rows evolve independently, so the oracle can
    compute just those) for shapes where the full fp64 oracle would be slow."""
    q, k, v, a, b = _inputs(variant, B, H, T, dk, dv, dtype, seed)
    print(f"[prefill-sampled] {variant} B={B} H={H} T={T} rows={rows} {dtype}", flush=True)
    o, S_T, _ = la.prefill(variant, q, k, v, a, b, S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill(variant, q, k, v, a, b, S0=S0, rows=rows)
    tol = TOL[dtype]
    assert_close(o[..., rows], oo, tol, what="o (sampled rows)")
    assert_close(S_T[:, :, rows, :], So, tol, what="S_T (sampled rows)")


@pytest.mark.parametrize("variant", ROWS_VARIANTS)
def test_chunk_multi_chunk_segments(la, variant):
    # 64 heads -> 16 segments of several chunks each, ragged tail
    _check_prefill_sampled(la, variant, 4, 16, 64 * 37 + 29, 128, 128, torch.bfloat16, 31,
                           rows=[0, 17, 63, 127])


@pytest.mark.parametrize("variant", ROWS_VARIANTS)
def test_chunk_single_segment_many_heads(la, variant):
    # 128 heads fill the chip: one segment, no map/scan passes
    S0 = synth.gdn_state((8, 16, 128, 128), seed=9, device=DEV) * 0.1
    _check_prefill_sampled(la, variant, 8, 16, 64 * 3 + 10, 128, 128, torch.bfloat16, 32,
                           rows=[1, 64, 126], S0=S0)


@pytest.mark.parametrize("variant", ROWS_VARIANTS)
@pytest.mark.parametrize("T", [1, 63, 64, 65])
def test_chunk_short_sequences(la, variant, T):
    _check_prefill(la, variant, 1, 2, T, 128, 128, torch.bfloat16, seed=40 + T)


def test_chunk_split_resume_on_gpu(la):
    """prefill(x[:a]) then prefill(x[a:], S0=S_a) matches one prefill(x) (within bf16 parity)."""
    q, k, v, a, b = _inputs("gated_delta", 1, 4, 1000, 128, 128, torch.bfloat16, 50)
    o, S, _ = la.prefill("gated_delta", q, k, v, a, b)
    cut = 448
    o1, S1, _ = la.prefill("gated_delta", q[:, :, :cut].contiguous(), k[:, :, :cut].contiguous(),
                           v[:, :, :cut].contiguous(), a[:, :, :cut].contiguous(),
                           b[:, :, :cut].contiguous())
    o2, S2, _ = la.prefill("gated_delta", q[:, :, cut:].contiguous(), k[:, :, cut:].contiguous(),
                           v[:, :, cut:].contiguous(), a[:, :, cut:].contiguous(),
                           b[:, :, cut:].contiguous(), S0=S1)
    torch.cuda.synchronize()
    assert_close(torch.cat([o1, o2], dim=2), o, 2e-2, what="o split")
    assert_close(S2, S, 2e-2, what="S split")


@pytest.mark.parametrize("variant", ROWS_VARIANTS)
def test_prefill_passes_compose_to_prefill(la, variant):
    """la_prefill == la_prefill_pass(TRANSFORM); (MAPS); (SCAN); (REPLAY), bit for bit."""
    q, k, v, a, b = _inputs(variant, 1, 4, 64 * 20 + 7, 128, 128, torch.bfloat16, 60)
    nseg, _ = la.segments(variant, la.BF16, 1, 4, q.shape[2], 128, 128)
    assert nseg > 1
    o1, S1, _ = la.prefill(variant, q, k, v, a, b)
    ws = torch.empty(la.workspace_size(variant, la.BF16, 1, 4, q.shape[2], 128, 128),
                     dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    for p in (la.PASS_TRANSFORM, la.PASS_MAPS, la.PASS_SCAN, la.PASS_REPLAY):
        la.prefill(variant, q, k, v, a, b, o=o2, S_T=S2, workspace=ws, pass_=p)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_based_chunk_full_config_sampled_columns(la):
    """BASED prefill at its full configuration (B=4, H=16, T=8192, d'=16, d_v=64, bf16):
    every output element of a sample of value columns against the oracle; z_T in full."""
    B, H, T, dp, dv = 4, 16, 8192, 16, 64
    q, k, v, _, _ = _inputs("based", B, H, T, dp, dv, torch.bfloat16, seed=1)
    nseg, _ = la.segments("based", la.BF16, B, H, T, dp, dv)
    assert nseg > 1
    print(f"[based full] segments={nseg}", flush=True)
    o, s_T, z_T = la.prefill("based", q, k, v)
    torch.cuda.synchronize()
    cols = [0, 21, 42, 63]
    oo, so, zo = oracle.prefill("based", q, k, v, rows=cols)
    assert_close(o[..., cols], oo, 2e-2, what="o (sampled columns)")
    assert_close(s_T[..., cols], so, 2e-2, what="s_T (sampled columns)")
    assert_close(z_T, zo, 2e-2, what="z_T")


@pytest.mark.parametrize("variant", BASED_VARIANTS)
@pytest.mark.parametrize("T", [1, 63, 64, 65, 1000])
def test_based_chunk_short_and_ragged(la, variant, T):
    _check_prefill(la, variant, 1, 3, T, 16, 64, torch.bfloat16, seed=70 + T)


@pytest.mark.parametrize("variant", BASED_VARIANTS)
def test_based_passes_compose_to_prefill(la, variant):
    """BASED: la_prefill == la_prefill_pass(MAPS); (SCAN); (REPLAY), bit for bit, with a
    start state (segment 0 starts from it, the last segment writes the end state)."""
    B, H, T, dp, dv = 1, 4, 64 * 20 + 7, 16, 64
    q, k, v, _, _ = _inputs(variant, B, H, T, dp, dv, torch.bfloat16, 61)
    nseg, _ = la.segments(variant, la.BF16, B, H, T, dp, dv)
    assert nseg > 1
    w = synth.based_inputs(B, H, 50, dp, dv, dtype=torch.bfloat16, seed=62, device=DEV)
    _, s0, z0 = la.prefill(variant, w["q"], w["k"], w["v"])
    o1, s1, z1 = la.prefill(variant, q, k, v, S0=s0, z0=z0)
    ws = torch.empty(la.workspace_size(variant, la.BF16, B, H, T, dp, dv), dtype=torch.uint8, device=DEV)
    o2, s2, z2 = torch.empty_like(o1), torch.empty_like(s1), torch.empty_like(z1)
    for p in (la.PASS_TRANSFORM, la.PASS_MAPS, la.PASS_SCAN, la.PASS_REPLAY):
        la.prefill(variant, q, k, v, S0=s0, z0=z0, o=o2, S_T=s2, z_T=z2, workspace=ws, pass_=p)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and torch.equal(z1, z2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_based_compact_matches_full(la, dtype):
    """Both feature layouts give the same outputs (the kernel value is the same), and the
    compact end state is the full one with each unordered pair folded."""
    B, H, T, dp, dv = 2, 2, 300, 16, 64
    q, k, v, _, _ = _inputs("based", B, H, T, dp, dv, dtype, 63)
    of, sf, zf = la.prefill("based", q, k, v)
    oc, sc, zc = la.prefill("based_compact", q, k, v)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert_close(oc, to64(of), tol, what="o compact vs full")
    sf, zf = to64(sf), to64(zf)
    idx = [(a, b) for a in range(dp) for b in range(a, dp)]
    fold_s = np.stack([sf[:, :, 1 + dp + a * dp + a] if a == b else
                       (sf[:, :, 1 + dp + a * dp + b] + sf[:, :, 1 + dp + b * dp + a]) / np.sqrt(2)
                       for a, b in idx], axis=2)
    assert_close(sc[:, :, 1 + dp:], fold_s, tol, what="s compact vs folded full")
    assert_close(sc[:, :, :1 + dp], sf[:, :, :1 + dp], tol, what="s [1, x] rows")


@pytest.mark.parametrize("variant", ROWS_VARIANTS + BASED_VARIANTS)
def test_prefill_in_place_state_across_segments(la, variant):
    """S_T may be S0's own buffer (include/la.h) also when the sequence is split into
    segments, whose replays run concurrently: the in-place result equals the out-of-place
    one bit for bit."""
    B, H, T = 1, 4, 64 * 20 + 7
    dk, dv = (16, 64) if variant in BASED_VARIANTS else (128, 128)
    q, k, v, a, b = _inputs(variant, B, H, T, dk, dv, torch.bfloat16, 64)
    nseg, _ = la.segments(variant, la.BF16, B, H, T, dk, dv)
    assert nseg > 1
    if variant in BASED_VARIANTS:
        w = synth.based_inputs(B, H, 50, dk, dv, dtype=torch.bfloat16, seed=65, device=DEV)
        _, S0, z0 = la.prefill(variant, w["q"], w["k"], w["v"])
    else:
        S0, z0 = synth.gdn_state((B, H, dv, dk), seed=65, device=DEV) * 0.3, None
    o1, S1, z1 = la.prefill(variant, q, k, v, a, b, S0=S0, z0=z0)
    S_io = S0.clone()
    z_io = None if z0 is None else z0.clone()
    o2, S2, z2 = la.prefill(variant, q, k, v, a, b, S0=S_io, z0=z_io, S_T=S_io, z_T=z_io)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_io.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S_io)
    if z0 is not None:
        assert torch.equal(z1, z_io)


@pytest.mark.parametrize("variant", ["gated", "gated_delta"])
@pytest.mark.parametrize("D", [128, 256])
def test_prefill_in_place_state_windowed_segments(la, variant, D):
    """The same with segments long enough (20 chunks) for the map pass to form each map from
    its last 8 chunks, whose transition the recipe's gates take to exactly zero: the scan
    then only copies S0 for the first segment and the replay starts every other segment
    from the previous map's B rows, while the last segment writes S_T over S0."""
    B, H = 1, 8
    T = 64 * 32 * 20 - 5
    q, k, v, a, b = _inputs(variant, B, H, T, D, D, torch.bfloat16, 68)
    nseg, sc = la.segments(variant, la.BF16, B, H, T, D, D)
    print(f"[in-place windowed] {variant} d={D} segments={nseg}x{sc}", flush=True)
    assert nseg > 1 and sc > 16
    S0 = synth.gdn_state((B, H, D, D), seed=69, device=DEV) * 0.3
    o1, S1, _ = la.prefill(variant, q, k, v, a, b, S0=S0)
    S_io = S0.clone()
    o2, S2, _ = la.prefill(variant, q, k, v, a, b, S0=S_io, S_T=S_io)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_io.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S_io)


@pytest.mark.parametrize("variant", ["additive", "gated"])
@pytest.mark.parametrize("T", [130, 1024])
def test_prefill_fp32_chunk_form_in_place(la, variant, T):
    """fp32 additive/gated prefills of 2..32 chunks run in the fp32 chunk form, whose chunks'
    workgroups all start from S0 while the last writes S_T: in place (S_T is S0's buffer)
    equals out of place bit for bit, and both match the oracle at the fp32 bound."""
    B, H, dk = 1, 2, 64
    q, k, v, a, b = _inputs(variant, B, H, T, dk, dk, torch.float32, 66)
    S0 = synth.gdn_state((B, H, dk, dk), seed=67, device=DEV) * 0.3
    o1, S1, _ = la.prefill(variant, q, k, v, a, b, S0=S0)
    S_io = S0.clone()
    o2, _, _ = la.prefill(variant, q, k, v, a, b, S0=S_io, S_T=S_io)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S_io)
    oo, So, _ = oracle.prefill(variant, q, k, v, a, b, S0=S0)
    assert_close(o1, oo, 1e-4, what="o")
    assert_close(S1, So, 1e-4, what="S_T")
