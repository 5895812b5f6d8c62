"""GPU parity in the long-memory regime and on the delta rule's defining cases.

Under the configurations' gates (alpha = exp(-softplus(a)), a ~ U(-2, 4)) a 64-token chunk
decays the carried state by about e^-100, so the state that crosses chunk and segment
boundaries contributes nothing measurable to the outputs, and a wrong segment transition
M_seg (or scalar segment decay) would pass every parity test.  The cases here keep the
carry alive, from Eq. (1) of "History Replays Itself" (Sec. 2) with the gated and
delta-rule transitions A_t = alpha_t I and A_t = alpha_t (I - beta_t k_t k_t^T):

  slow    a ~ U(-8, -4): alpha in [0.98, 1] (bf16 rounds 44% of them to exactly 1)
  pool    slow gates, every key one of 16 fixed directions (repeated, correlated keys:
          the delta rule never erases the part of S outside their span)
  alpha1  alpha = 1 (no decay), pool keys
  beta0   slow gates, beta = 0: the delta rule degenerates to pure decay S_t = alpha_t S_{t-1}
  basis   standard-basis keys with repeats, beta = 1, q_t = k_t: exact overwrite, o_t = v_t
  perm    alpha = 1, basis keys never repeated, S0 = 0: the delta rule equals the gated one

Before it compares anything, each test asserts on the oracle alone that its inputs make
the carry matter: replacing the true start state of a segment by the end state of the
previous segment run from zero (that is, dropping the previous segment's transition)
moves the oracle's outputs on the segment by more than ten times the parity bound.  So
each of these tests fails if the GPU path zeroes or garbles M_seg or the scan.

Every call goes through the C ABI; bound 2e-2 (bf16 inputs), per (b, h) slice,
max-norm relative (tests/parity.py).  The printed errors are the recorded margins.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_close, slice_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2

REGIMES = {
    "slow": dict(a_range=(-8.0, -4.0)),
    "pool": dict(a_range=(-8.0, -4.0), keys="pool"),
    "alpha1": dict(alpha_one=True, keys="pool"),
    "beta0": dict(a_range=(-8.0, -4.0), beta="zero"),
}
# (B, H, T) per key width: several multi-chunk segments per (b, h), ragged last chunk
SHAPES = {128: (1, 8, 64 * 63 + 37), 256: (1, 8, 64 * 40 + 5)}


def _inputs(variant, B, H, T, D, seed, **regime):
    return synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=seed, device=DEV,
                            normalize=(variant == "gated_delta"), **regime)


def _args(d):
    return d["q"], d["k"], d["v"], d["alpha"], d["beta"]


def _sub(d, heads, lo, hi):
    return {n: t[:, heads, lo:hi] for n, t in d.items()}


def _full_rows(S_rows, rows, dv):
    """Sampled rows of a state embedded in a full-size one (other rows zero): the oracle
    reads only the rows it is asked for."""
    B, H, _, dk = S_rows.shape
    F = np.zeros((B, H, dv, dk))
    F[:, :, rows] = S_rows
    return F


def assert_carry_matters(variant, d, S0, seg_tokens, heads=None, rows=None, factor=10.0):
    """Oracle only: the start state of segment 2 (S_2 = S_1 M_1 + B_1) against B_1 alone
    (segment 1 from a zero start), and the outputs of segment 2 from each of them."""
    B, H, T, dk = d["q"].shape
    dv = d["v"].shape[-1]
    heads = list(range(H)) if heads is None else list(heads)
    rows = list(range(dv)) if rows is None else list(rows)
    s1, s2, s3 = seg_tokens, 2 * seg_tokens, min(3 * seg_tokens, T)
    assert s3 > s2, "needs at least three segments"
    S0h = None if S0 is None else S0[:, heads]
    _, S_true, _ = oracle.prefill(variant, *_args(_sub(d, heads, 0, s2)), S0=S0h, rows=rows)
    _, B_1, _ = oracle.prefill(variant, *_args(_sub(d, heads, s1, s2)), rows=rows)
    seg2 = _args(_sub(d, heads, s2, s3))
    o_true, _, _ = oracle.prefill(variant, *seg2, S0=_full_rows(S_true, rows, dv), rows=rows)
    o_wrong, _, _ = oracle.prefill(variant, *seg2, S0=_full_rows(B_1, rows, dv), rows=rows)
    ds, _ = slice_rel(B_1, S_true)
    do, _ = slice_rel(o_wrong, o_true)
    print(f"    carry sensitivity: start state without M_seg off by {ds:.2e}, "
          f"segment outputs off by {do:.2e} (need > {factor * TOL:.0e})", flush=True)
    assert do > factor * TOL, "inputs do not exercise the segment transition"


def _run_full(la, variant, D, regime, seed):
    B, H, T = SHAPES[D]
    d = _inputs(variant, B, H, T, D, seed, **REGIMES[regime])
    S0 = synth.gdn_state((B, H, D, D), seed=seed, device=DEV) * 0.3
    nseg, sc = la.segments(variant, la.BF16, B, H, T, D, D)
    print(f"[long-memory] {variant} d={D} regime={regime} B={B} H={H} T={T} segments={nseg}x{sc}",
          flush=True)
    assert nseg >= 3 and sc >= 2, "multi-chunk segments expected"
    assert_carry_matters(variant, d, S0.cpu().numpy().astype(np.float64), sc * 64)
    o, S_T, _ = la.prefill(variant, *_args(d), S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill(variant, *_args(d), S0=S0)
    e_o = assert_close(o, oo, TOL, what=f"o [{regime}, d={D}]")
    e_s = assert_close(S_T, So, TOL, what=f"S_T [{regime}, d={D}]")
    return e_o, e_s


@pytest.mark.parametrize("regime", list(REGIMES))
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("variant", ["gated", "gated_delta"])
def test_long_memory_multichunk_segments_full(la, variant, D, regime):
    """Every element of o and S_T, multi-chunk segments, a start state, a ragged tail."""
    _run_full(la, variant, D, regime, seed=100 + D + len(regime))


@pytest.mark.parametrize("D", [128, 256])
def test_delta_basis_keys_exact_overwrite(la, D):
    """beta = 1 on standard-basis keys: S_t k_t = v_t whatever S_{t-1} and alpha_t, so with
    q_t = k_t every output equals its own value vector (exact in the recurrence; the bf16
    chunk path rounds its operands).  S_T against the oracle: each slot holds its last
    write, decayed since."""
    B, H, T = SHAPES[D]
    d = _inputs("gated_delta", B, H, T, D, seed=7 + D, a_range=(-8.0, -4.0), keys="basis",
                beta="one", q_is_k=True)
    S0 = synth.gdn_state((B, H, D, D), seed=8, device=DEV) * 0.3
    print(f"[basis overwrite] d={D} B={B} H={H} T={T}", flush=True)
    o, S_T, _ = la.prefill("gated_delta", *_args(d), S0=S0)
    torch.cuda.synchronize()
    assert_close(o, d["v"], TOL, what=f"o against v [d={D}]")
    oo, So, _ = oracle.prefill("gated_delta", *_args(d), S0=S0)
    assert_close(o, oo, TOL, what=f"o [basis, d={D}]")
    assert_close(S_T, So, TOL, what=f"S_T [basis, d={D}]")


@pytest.mark.parametrize("D", [128, 256])
def test_delta_alpha1_unrepeated_keys_equals_gated(la, D):
    """alpha = 1, S0 = 0 and keys that never repeat (basis vectors in a random order, d_k
    tokens): S_{t-1} k_t = 0 at every step, so the delta rule's correction vanishes and it
    equals the gated recurrence with the same beta."""
    B, H, T = 1, 8, D
    d = _inputs("gated_delta", B, H, T, D, seed=9, alpha_one=True, keys="perm")
    print(f"[alpha=1 unrepeated] d={D} H={H} T={T}", flush=True)
    od, Sd, _ = la.prefill("gated_delta", *_args(d))
    og, Sg, _ = la.prefill("gated", *_args(d))
    torch.cuda.synchronize()
    assert_close(od, og.float(), TOL, what=f"o delta vs gated [d={D}]")
    assert_close(Sd, Sg, TOL, what=f"S_T delta vs gated [d={D}]")
    oo, So, _ = oracle.prefill("gated_delta", *_args(d))
    assert_close(od, oo, TOL, what=f"o [perm, d={D}]")
    assert_close(Sd, So, TOL, what=f"S_T [perm, d={D}]")


@pytest.mark.parametrize("variant", ["gated", "gated_delta"])
def test_beta0_pure_decay_across_segments(la, variant):
    """beta = 0: S_t = alpha_t S_{t-1} for both variants, so S_T = gamma_T S0 and
    o_t = gamma_t S0 q_t; the scan carries nothing but the decayed start state."""
    (B, H, T), D = SHAPES[128], 128
    d = _inputs(variant, B, H, T, D, seed=11, a_range=(-8.0, -4.0), beta="zero")
    S0 = synth.gdn_state((B, H, D, D), seed=12, device=DEV)
    nseg, sc = la.segments(variant, la.BF16, B, H, T, D, D)
    print(f"[beta=0] {variant} segments={nseg}x{sc}", flush=True)
    o, S_T, _ = la.prefill(variant, *_args(d), S0=S0)
    torch.cuda.synchronize()
    oo, So, _ = oracle.prefill(variant, *_args(d), S0=S0)
    assert_close(o, oo, TOL, what="o [beta=0]")
    assert_close(S_T, So, TOL, what="S_T [beta=0]")


# ------------------------------------------------------------------ million-token runs
def _million(la, variant, D, H, heads, rows, seed, sensitive, **regime):
    B, T = 1, 1 << 20
    d = _inputs(variant, B, H, T, D, seed, **regime)
    S0 = synth.gdn_state((B, H, D, D), seed=seed, device=DEV) * 0.3
    nseg, sc = la.segments(variant, la.BF16, B, H, T, D, D)
    print(f"[1M long-memory] {variant} d={D} H={H} {regime} segments={nseg}x{sc}", flush=True)
    o, S_T, _ = la.prefill(variant, *_args(d), S0=S0)
    torch.cuda.synchronize()
    hs = list(heads)
    o_s = o[:, hs][..., rows].cpu()
    S_s = S_T[:, hs][:, :, rows, :].cpu()
    del o, S_T
    host = {n: t[:, hs].cpu() for n, t in d.items()}
    S0h = S0[:, hs].cpu().numpy().astype(np.float64)
    del d
    torch.cuda.empty_cache()
    if sensitive:
        assert_carry_matters(variant, host, S0h, sc * 64, rows=rows)
    oo, So, _ = oracle.prefill(variant, *_args(host), S0=S0h, rows=rows)
    assert_close(o_s, oo, TOL, what=f"1M o (heads {hs}, rows {rows})")
    assert_close(S_s, So, TOL, what=f"1M S_T (heads {hs}, rows {rows})")


def test_1m_delta_alpha1_pool_keys_sampled(la):
    """1M tokens x 16 heads, alpha = 1 and pooled keys: the part of S outside the keys' span
    is carried unchanged through all 32 segments, so every transition matters."""
    _million(la, "gated_delta", 128, 16, [0, 9], [3, 64, 126], seed=21, sensitive=True,
             alpha_one=True, keys="pool")


def test_1m_gated_alpha1_sampled(la):
    """1M tokens, the scalar-gated carry with alpha = 1: each segment's decay is exactly 1."""
    _million(la, "gated", 128, 16, [0, 15], [5, 100], seed=22, sensitive=True, alpha_one=True)


def test_1m_delta_slow_gates_sampled(la):
    """1M tokens under slow gates with the configuration's random keys: the accumulated
    rounding of the bf16 state operands over the whole sequence."""
    _million(la, "gated_delta", 128, 16, [3, 12], [0, 77, 127], seed=23, sensitive=False,
             a_range=(-8.0, -4.0))


def test_1m_delta_d256_alpha1_pool_keys_sampled(la):
    """The 8-head x 256 shape at 1M tokens, alpha = 1 and pooled keys, rows of both row
    blocks of a head."""
    _million(la, "gated_delta", 256, 8, [0, 5], [7, 127, 128, 255], seed=24, sensitive=True,
             alpha_one=True, keys="pool")
