"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: a brute-force evaluation of
a closed form, an invariant, a special case with a known answer, or a number printed
on the pages (tests/golden/printed_values.json).  A plausible mistake in the oracle
(dropped term, wrong sign, off-by-one in the causal mask, transposed operand, wrong
feature layout, gate applied to the write term) fails at least one of them; see also
test_oracle_mutants.py, which plants such mistakes and checks that they are caught.
"""

import json
import math
from pathlib import Path

import numpy as np
import pytest

import oracle
from tests import models

GOLDEN = json.loads((Path(__file__).parent / "golden" / "printed_values.json").read_text())


def rel(x, y):
    return float(np.max(np.abs(np.asarray(x) - np.asarray(y))) / max(np.max(np.abs(y)), 1e-300))


def rng(seed):
    return np.random.default_rng(seed)


def gdn_like(r, B, H, T, dk, dv, normalize=True, a_range=(-2, 4)):
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    if normalize:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, dv))
    a = r.uniform(a_range[0], a_range[1], (B, H, T))
    alpha = np.exp(-np.log1p(np.exp(a)))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, H, T))))
    return q, k, v, alpha, beta


# ----------------------------------------------------------------------------- additive
def test_additive_matches_causal_bruteforce():
    """Additive case: O = (Q K^T . M) V + Q S0^T, S_T = S0 + V^T K (M causal incl. diagonal)."""
    r = rng(1)
    B, H, T, dk, dv = 2, 3, 37, 5, 4
    q, k, v = (r.standard_normal((B, H, T, d)) for d in (dk, dk, dv))
    S0 = r.standard_normal((B, H, dv, dk))
    o, S_T, _ = oracle.prefill("additive", q, k, v, S0=S0)
    M = np.tril(np.ones((T, T)))
    for b in range(B):
        for h in range(H):
            ref = ((q[b, h] @ k[b, h].T) * M) @ v[b, h] + q[b, h] @ S0[b, h].T
            assert rel(o[b, h], ref) < 1e-12
            assert rel(S_T[b, h], S0[b, h] + v[b, h].T @ k[b, h]) < 1e-12


def test_additive_reads_after_write():
    """o_t = S_t q_t reads the state *after* token t's write (diagonal included)."""
    q = np.zeros((1, 1, 1, 3))
    k = np.zeros((1, 1, 1, 3))
    q[..., 0] = 1.0
    k[..., 0] = 2.0
    v = np.array([[[[5.0, -1.0]]]])
    o, _, _ = oracle.prefill("additive", q, k, v)
    assert np.array_equal(o[0, 0, 0], np.array([10.0, -2.0]))


# ----------------------------------------------------------------------------- BASED
def test_golden_feature_dims():
    assert oracle.feature_dim(16) == GOLDEN["based_feature_dim_full_dprime16"]["value"]
    assert 1 + 16 + 16 * 17 // 2 == GOLDEN["based_feature_dim_compact_dprime16"]["value"]
    assert -(-273 // 64) * 64 == GOLDEN["based_feature_dim_padded_dprime16"]["value"]
    assert oracle.based_phi(np.ones(16)).size == 273


def test_taylor_feature_map_closed_form():
    """phi(q).phi(k) = 1 + q.k + (q.k)^2/2 for 10^4 random pairs, d' = 16."""
    r = rng(2)
    worst = 0.0
    for _ in range(10_000):
        x, y = r.standard_normal(16), r.standard_normal(16)
        t = float(x @ y)
        kern = 1.0 + t + t * t / 2.0
        worst = max(worst, abs(oracle.based_phi(x) @ oracle.based_phi(y) - kern) / abs(kern))
    assert worst < 1e-13


def test_taylor_scaled_closed_form():
    """With xbar = x / d'^(1/4): phi(qbar).phi(kbar) = 1 + q.k/sqrt(d') + (q.k)^2/(2 d')."""
    r = rng(3)
    dp = 16
    for _ in range(1000):
        x, y = r.standard_normal(dp), r.standard_normal(dp)
        t = float(x @ y)
        s = dp ** 0.25
        val = oracle.based_phi(x / s) @ oracle.based_phi(y / s)
        assert abs(val - (1 + t / math.sqrt(dp) + t * t / (2 * dp))) < 1e-12 * (1 + t * t)


def _compact_pairs(dp):
    """(a, b) of every compact order-2 feature, in its stored order: row-major upper triangle."""
    return [(a, b) for a in range(dp) for b in range(a, dp)]


def test_compact_feature_map_layout_and_kernel():
    """The compact map keeps x_a^2/sqrt 2 and x_a x_b (a < b) once each, after [1, x], and has
    the kernel value of the full map: phi_c(q).phi_c(k) = 1 + q.k + (q.k)^2/2."""
    r = rng(21)
    dp = 16
    assert oracle.feature_dim(dp, compact=True) == GOLDEN["based_feature_dim_compact_dprime16"]["value"]
    x = r.standard_normal(dp)
    f = oracle.based_phi_compact(x)
    assert f.size == 153 and f[0] == 1.0 and np.array_equal(f[1:1 + dp], x)
    for i, (a, b) in enumerate(_compact_pairs(dp)):
        want = x[a] * x[a] / math.sqrt(2) if a == b else x[a] * x[b]
        assert abs(f[1 + dp + i] - want) <= 1e-15 * max(1.0, abs(want))
    worst = 0.0
    for _ in range(10_000):
        x, y = r.standard_normal(dp), r.standard_normal(dp)
        t = float(x @ y)
        kern = 1.0 + t + t * t / 2.0
        worst = max(worst, abs(oracle.based_phi_compact(x) @ oracle.based_phi_compact(y) - kern) / abs(kern))
    assert worst < 1e-13


def test_compact_scaled_closed_form():
    """The scaled identity holds for the compact map too (inputs pre-scaled by d'^(-1/4))."""
    r = rng(22)
    dp = 16
    for _ in range(1000):
        x, y = r.standard_normal(dp), r.standard_normal(dp)
        t = float(x @ y)
        s = dp ** 0.25
        val = oracle.based_phi_compact(x / s) @ oracle.based_phi_compact(y / s)
        assert abs(val - (1 + t / math.sqrt(dp) + t * t / (2 * dp))) < 1e-12 * (1 + t * t)


def test_taylor_positivity():
    """((t+1)^2+1)/2 >= 1/2: every kernel term is at least 1/2."""
    t = np.linspace(-50, 50, 100001)
    kern = 1 + t + t * t / 2
    assert np.allclose(kern, ((t + 1) ** 2 + 1) / 2, rtol=1e-14, atol=0)
    assert kern.min() >= 0.5 - 1e-15


def _based_bruteforce(q, k, v, eps, prefix=None):
    """y_i = sum_{j<=i} K(q_i,k_j) v_j / (sum_{j<=i} K(q_i,k_j) + eps), K(q,k)=1+q.k+(q.k)^2/2."""
    if prefix is not None:
        kq, vq = prefix
        k = np.concatenate([kq, k])
        v = np.concatenate([vq, v])
    P = 0 if prefix is None else prefix[0].shape[0]
    T = q.shape[0]
    dots = q @ k.T
    Kmat = 1 + dots + dots ** 2 / 2
    mask = np.arange(P + T)[None, :] <= (P + np.arange(T))[:, None]
    Kmat = Kmat * mask
    den = Kmat.sum(1)
    return (Kmat @ v) / (den + eps)[:, None], den


def test_based_matches_bruteforce_and_denominator_bound():
    r = rng(4)
    B, H, T, dp, dv = 1, 2, 64, 4, 3
    q = r.standard_normal((B, H, T, dp)) / 2
    k = r.standard_normal((B, H, T, dp)) / 2
    v = r.standard_normal((B, H, T, dv))
    eps = 1e-6
    o, s_T, z_T = oracle.prefill("based", q, k, v, eps=eps)
    for h in range(H):
        ref, den = _based_bruteforce(q[0, h], k[0, h], v[0, h], eps)
        assert rel(o[0, h], ref) < 1e-12
        assert np.all(den >= (np.arange(T) + 1) / 2 - 1e-12)
        # the final state reproduces the sum over all keys for a fresh query
        x = r.standard_normal(dp)
        f = oracle.based_phi(x)
        Kx = 1 + k[0, h] @ x + (k[0, h] @ x) ** 2 / 2
        assert rel(s_T[0, h].T @ f, Kx @ v[0, h]) < 1e-12
        assert abs(z_T[0, h] @ f - Kx.sum()) < 1e-10 * Kx.sum()


def test_based_start_state_equals_prefix():
    """Start (s0, z0) from a prefix == brute force over prefix + tokens."""
    r = rng(5)
    dp, dv, P, T = 3, 2, 20, 30
    kp = r.standard_normal((1, 1, P, dp))
    qp = r.standard_normal((1, 1, P, dp))
    vp = r.standard_normal((1, 1, P, dv))
    _, s0, z0 = oracle.prefill("based", qp, kp, vp)
    q = r.standard_normal((1, 1, T, dp))
    k = r.standard_normal((1, 1, T, dp))
    v = r.standard_normal((1, 1, T, dv))
    o, _, _ = oracle.prefill("based", q, k, v, S0=s0, z0=z0, eps=1e-6)
    ref, _ = _based_bruteforce(q[0, 0], k[0, 0], v[0, 0], 1e-6, prefix=(kp[0, 0], vp[0, 0]))
    assert rel(o[0, 0], ref) < 1e-12


def test_compact_matches_bruteforce_and_full_state():
    """Compact BASED: outputs equal brute force; its end state is the full one with each
    unordered pair folded, (s(a,b) + s(b,a)) / sqrt 2, and the squares kept."""
    r = rng(23)
    B, H, T, dp, dv = 1, 2, 48, 4, 3
    q = r.standard_normal((B, H, T, dp)) / 2
    k = r.standard_normal((B, H, T, dp)) / 2
    v = r.standard_normal((B, H, T, dv))
    eps = 1e-6
    oc, sc, zc = oracle.prefill("based_compact", q, k, v, eps=eps)
    of, sf, zf = oracle.prefill("based", q, k, v, eps=eps)
    for h in range(H):
        ref, _ = _based_bruteforce(q[0, h], k[0, h], v[0, h], eps)
        assert rel(oc[0, h], ref) < 1e-12
    assert rel(oc, of) < 1e-12
    for i, (a, b) in enumerate(_compact_pairs(dp)):
        fa, fb = 1 + dp + a * dp + b, 1 + dp + b * dp + a
        want_s = sf[:, :, fa] if a == b else (sf[:, :, fa] + sf[:, :, fb]) / math.sqrt(2)
        want_z = zf[:, :, fa] if a == b else (zf[:, :, fa] + zf[:, :, fb]) / math.sqrt(2)
        assert rel(sc[:, :, 1 + dp + i], want_s) < 1e-12 and rel(zc[:, :, 1 + dp + i], want_z) < 1e-12
    assert rel(sc[:, :, :1 + dp], sf[:, :, :1 + dp]) < 1e-12 and rel(zc[:, :, :1 + dp], zf[:, :, :1 + dp]) < 1e-12


def test_compact_start_state_equals_prefix():
    r = rng(24)
    dp, dv, P, T = 3, 2, 20, 30
    kp, qp, vp = r.standard_normal((1, 1, P, dp)), r.standard_normal((1, 1, P, dp)), r.standard_normal((1, 1, P, dv))
    _, s0, z0 = oracle.prefill("based_compact", qp, kp, vp)
    q, k, v = r.standard_normal((1, 1, T, dp)), r.standard_normal((1, 1, T, dp)), r.standard_normal((1, 1, T, dv))
    o, _, _ = oracle.prefill("based_compact", q, k, v, S0=s0, z0=z0, eps=1e-6)
    ref, _ = _based_bruteforce(q[0, 0], k[0, 0], v[0, 0], 1e-6, prefix=(kp[0, 0], vp[0, 0]))
    assert rel(o[0, 0], ref) < 1e-12


# ----------------------------------------------------------------------------- gated
def test_gated_alpha_one_is_additive_bitwise():
    r = rng(6)
    B, H, T, dk, dv = 1, 2, 50, 6, 5
    q, k, v = (r.standard_normal((B, H, T, d)) for d in (dk, dk, dv))
    S0 = r.standard_normal((B, H, dv, dk))
    ones = np.ones((B, H, T))
    o1, S1, _ = oracle.prefill("gated", q, k, v, alpha=ones, beta=ones, S0=S0)
    o2, S2, _ = oracle.prefill("additive", q, k, v, S0=S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    o3, S3, _ = oracle.prefill("gated", q, k, v, alpha=ones, beta=None, S0=S0)
    assert np.array_equal(o3, o2) and np.array_equal(S3, S2)


def test_gated_closed_form():
    """o_t = gamma_t S0 q_t + sum_{j<=t} (prod_{i=j+1..t} alpha_i) beta_j (k_j.q_t) v_j."""
    r = rng(7)
    T, dk, dv = 40, 5, 4
    q, k, v, alpha, beta = gdn_like(r, 1, 1, T, dk, dv, normalize=False)
    S0 = r.standard_normal((1, 1, dv, dk))
    o, S_T, _ = oracle.prefill("gated", q, k, v, alpha=alpha, beta=beta, S0=S0)
    a, b = alpha[0, 0], beta[0, 0]
    ref = np.zeros((T, dv))
    for t in range(T):
        acc = np.prod(a[: t + 1]) * (S0[0, 0] @ q[0, 0, t])
        for j in range(t + 1):
            acc = acc + np.prod(a[j + 1: t + 1]) * b[j] * (k[0, 0, j] @ q[0, 0, t]) * v[0, 0, j]
        ref[t] = acc
    assert rel(o[0, 0], ref) < 1e-12
    ST = np.prod(a) * S0[0, 0] + sum(np.prod(a[j + 1:]) * b[j] * np.outer(v[0, 0, j], k[0, 0, j])
                                      for j in range(T))
    assert rel(S_T[0, 0], ST) < 1e-12


# ----------------------------------------------------------------------------- delta rule
def test_delta_exact_overwrite():
    """beta_t = 1 and k_t a standard basis vector e_i: S_t e_i = v_t exactly, for any
    alpha and any previous state (read back with q_t = k_t)."""
    r = rng(8)
    T, dk, dv = 64, 8, 6
    idx = r.integers(0, dk, T)
    k = np.zeros((1, 1, T, dk))
    k[0, 0, np.arange(T), idx] = 1.0
    v = r.standard_normal((1, 1, T, dv))
    alpha = r.uniform(0.05, 1.0, (1, 1, T))
    beta = np.ones((1, 1, T))
    S0 = r.standard_normal((1, 1, dv, dk)) * 3
    o, _, _ = oracle.prefill("gated_delta", k, k, v, alpha=alpha, beta=beta, S0=S0)
    assert np.array_equal(o, v)


def test_delta_slot_memory():
    """Keys from {e_i} with repeats, beta = 1: S_T e_i = (prod_{s > t_i} alpha_s) v_{t_i}
    for the last write t_i to slot i, else (prod alpha) S0 e_i."""
    r = rng(9)
    T, dk, dv = 48, 10, 3
    idx = r.integers(0, dk - 2, T)  # the last two slots are never written
    k = np.zeros((1, 1, T, dk))
    k[0, 0, np.arange(T), idx] = 1.0
    q = r.standard_normal((1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    alpha = r.uniform(0.5, 1.0, (1, 1, T))
    S0 = r.standard_normal((1, 1, dv, dk))
    _, S_T, _ = oracle.prefill("gated_delta", q, k, v, alpha=alpha, beta=np.ones((1, 1, T)), S0=S0)
    a = alpha[0, 0]
    for i in range(dk):
        writes = np.nonzero(idx == i)[0]
        if writes.size:
            ti = writes[-1]
            expect = np.prod(a[ti + 1:]) * v[0, 0, ti]
        else:
            expect = np.prod(a) * S0[0, 0, :, i]
        assert np.allclose(S_T[0, 0, :, i], expect, rtol=1e-14, atol=1e-15)


def test_delta_beta_zero_is_pure_decay():
    r = rng(10)
    T, dk, dv = 30, 6, 4
    q, k, v, alpha, _ = gdn_like(r, 1, 1, T, dk, dv)
    S0 = r.standard_normal((1, 1, dv, dk))
    o, S_T, _ = oracle.prefill("gated_delta", q, k, v, alpha=alpha, beta=np.zeros((1, 1, T)), S0=S0)
    g = np.cumprod(alpha[0, 0])
    assert rel(S_T[0, 0], g[-1] * S0[0, 0]) < 1e-14
    assert rel(o[0, 0], g[:, None] * (q[0, 0] @ S0[0, 0].T)) < 1e-13


def test_delta_orthonormal_unrepeated_keys_equal_gated():
    """alpha = 1, keys orthonormal and never repeated, S0 = 0: S_{t-1} k_t = 0, so the delta
    rule reduces to the (beta-weighted) gated/additive write."""
    r = rng(11)
    dk = dv = 12
    T = dk
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm.T[None, None]  # rows orthonormal
    q = r.standard_normal((1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    beta = r.uniform(0.1, 1.0, (1, 1, T))
    ones = np.ones((1, 1, T))
    o1, S1, _ = oracle.prefill("gated_delta", q, k, v, alpha=ones, beta=beta)
    o2, S2, _ = oracle.prefill("gated", q, k, v, alpha=ones, beta=beta)
    assert rel(o1, o2) < 1e-13 and rel(S1, S2) < 1e-13


@pytest.mark.parametrize("variant", ["additive", "gated", "gated_delta"])
def test_rank1_form_matches_explicit_transition(variant):
    """Row-wise rank-1 update == S_{t-1} A_t + beta_t v_t k_t^T with A_t built explicitly."""
    r = rng(12)
    T, dk, dv = 9, 4, 3
    q, k, v, alpha, beta = gdn_like(r, 1, 1, T, dk, dv, normalize=False)
    S0 = r.standard_normal((1, 1, dv, dk))
    o, S_T, _ = oracle.prefill(variant, q, k, v, alpha=alpha, beta=beta, S0=S0)
    ol, SL = oracle.literal(variant, q[0, 0], k[0, 0], v[0, 0], alpha[0, 0], beta[0, 0], S0[0, 0])
    assert rel(o[0, 0], ol) < 1e-13 and rel(S_T[0, 0], SL) < 1e-13


# ----------------------------------------------------------------------------- structure
@pytest.mark.parametrize("variant", ["additive", "gated", "gated_delta"])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_derivation_matches_sequential(variant, C):
    """The block algebra the kernels use (tests/models.py) equals the token recurrence."""
    r = rng(13)
    T, dk, dv = 203, 16, 12
    q, k, v, alpha, beta = gdn_like(r, 1, 1, T, dk, dv)
    S0 = r.standard_normal((1, 1, dv, dk)) * 0.5
    o, S_T, _ = oracle.prefill(variant, q, k, v, alpha=alpha, beta=beta, S0=S0)
    oc, Sc = models.chunked(variant, q[0, 0], k[0, 0], v[0, 0],
                            None if variant == "additive" else alpha[0, 0],
                            None if variant == "additive" else beta[0, 0], S0[0, 0], C)
    assert rel(oc, o[0, 0]) < 1e-10 and rel(Sc, S_T[0, 0]) < 1e-10


def _segment_case(variant):
    # slow gates (a ~ U(-8, -4), alpha in [0.98, 0.9997]): the state carried across a
    # 48-token segment keeps most of its size, so the segment transitions matter
    r = rng(14)
    T, dk, dv, C = 64 * 7 + 13, 16, 8, 16
    q, k, v, alpha, beta = gdn_like(r, 1, 1, T, dk, dv, a_range=(-8, -4))
    S0 = r.standard_normal((1, 1, dv, dk))
    o, S_T, _ = oracle.prefill(variant, q, k, v, alpha=alpha, beta=beta, S0=S0)
    os_, Ss = models.segmented(variant, q[0, 0], k[0, 0], v[0, 0],
                               None if variant == "additive" else alpha[0, 0],
                               None if variant == "additive" else beta[0, 0], S0[0, 0], C, 3)
    return max(rel(os_, o[0, 0]), rel(Ss, S_T[0, 0]))


@pytest.mark.parametrize("variant", ["additive", "gated", "gated_delta"])
def test_segment_scan_matches_sequential(variant):
    """Per-segment affine maps + scan + rerun (the three-pass prefill) == recurrence."""
    assert _segment_case(variant) < 1e-10


@pytest.mark.parametrize("mistake", ["zero_transition", "transposed_transition", "dropped_decay"])
@pytest.mark.parametrize("variant", ["gated", "gated_delta"])
def test_segment_pin_catches_planted_transition_mistakes(monkeypatch, variant, mistake):
    """The segment pin above is sensitive to the transition M_c that the map pass composes:
    a zeroed, transposed or undecayed transition, planted in a copy of the chunk-map model,
    moves the result far past the pin's bound."""
    good = models.chunk_map

    def planted(variant_, K, V, a, b):
        M, Bc = good(variant_, K, V, a, b)
        if mistake == "zero_transition":
            M = np.zeros_like(M)
        elif mistake == "transposed_transition":
            M = M.T.copy()
        else:  # the chunk's decay left out of the transition
            M = M / np.exp(np.sum(np.log(a)))
        return M, Bc

    monkeypatch.setattr(models, "chunk_map", planted)
    err = _segment_case(variant)
    if variant == "gated" and mistake == "transposed_transition":
        assert err < 1e-10  # gamma I is symmetric: nothing to catch
    else:
        assert err > 1e-2, f"planted {mistake} gives only {err:.2e}"


def _window_case(variant, kill, force=False):
    # segments of 8 chunks of 8 tokens, windows of 3 chunks; kill=True sets alpha = 1e-200 on
    # two tokens inside every segment's window, whose decay product (1e-400) is exactly zero
    # in fp64, so the window's transition is zero; otherwise slow gates keep it alive
    r = rng(16)
    C, seg_chunks, window = 8, 8, 3
    T, dk, dv = C * seg_chunks * 4 - 3, 6, 5
    q, k, v, alpha, beta = gdn_like(r, 1, 1, T, dk, dv, a_range=(-8, -4))
    if kill:
        for s0 in range(0, T, C * seg_chunks):
            for t in (s0 + C * (seg_chunks - window) + 2, s0 + C * (seg_chunks - window) + 5):
                if t < T:
                    alpha[0, 0, t] = 1e-200
    S0 = r.standard_normal((1, 1, dv, dk))
    o, S_T, _ = oracle.prefill(variant, q, k, v, alpha=alpha, beta=beta, S0=S0)
    ow, Sw, used = models.windowed_segmented(variant, q[0, 0], k[0, 0], v[0, 0], alpha[0, 0],
                                             beta[0, 0], S0[0, 0], C, seg_chunks, window, force)
    return max(rel(ow, o[0, 0]), rel(Sw, S_T[0, 0])), used


@pytest.mark.parametrize("variant", ["gated", "gated_delta"])
def test_window_maps_match_sequential(variant):
    """The map pass's window: a segment whose last chunks compose to an exactly zero
    transition is mapped from those chunks alone, (0, B_last); with the window's
    transition zero (decay underflowing fp64) every full segment takes the window and the
    result still equals the token recurrence; with slow decay no segment takes it."""
    err, used = _window_case(variant, kill=True)
    assert err < 1e-10 and used[:-1] == [True] * (len(used) - 1)
    err, used = _window_case(variant, kill=False)
    assert err < 1e-10 and not any(used)


@pytest.mark.parametrize("variant", ["gated", "gated_delta"])
def test_window_pin_catches_a_window_taken_without_a_zero_transition(variant):
    """Taking the window's map while its transition is not zero drops the earlier chunks'
    contribution B_first M_last and the start state's S M_first M_last: far past the bound."""
    err, used = _window_case(variant, kill=False, force=True)
    assert any(used) and err > 1e-2, f"forced window gives only {err:.2e}"


@pytest.mark.parametrize("variant", ["additive", "gated", "gated_delta", "based", "based_compact"])
def test_split_resume(variant):
    """prefill(x[:a]) -> S_a; prefill(x[a:], S0=S_a) == prefill(x)."""
    r = rng(15)
    T, dk, dv, a = 90, 6, 5, 37
    q, k, v, alpha, beta = gdn_like(r, 2, 2, T, dk, dv)
    kw = dict(eps=1e-6)
    o, S, z = oracle.prefill(variant, q, k, v, alpha, beta, **kw)
    o1, S1, z1 = oracle.prefill(variant, q[:, :, :a], k[:, :, :a], v[:, :, :a], alpha[:, :, :a],
                                beta[:, :, :a], **kw)
    o2, S2, z2 = oracle.prefill(variant, q[:, :, a:], k[:, :, a:], v[:, :, a:], alpha[:, :, a:],
                                beta[:, :, a:], S0=S1, z0=z1, **kw)
    assert rel(np.concatenate([o1, o2], axis=2), o) < 1e-12
    assert rel(S2, S) < 1e-12
    if z is not None:
        assert rel(z2, z) < 1e-12


@pytest.mark.parametrize("variant", ["additive", "gated", "gated_delta", "based", "based_compact"])
def test_prefill_then_decode_equals_longer_prefill(variant):
    r = rng(16)
    T, n, dk, dv = 20, 5, 4, 3
    q, k, v, alpha, beta = gdn_like(r, 1, 3, T + n, dk, dv)
    o, S, z = oracle.prefill(variant, q, k, v, alpha, beta)
    _, St, zt = oracle.prefill(variant, q[:, :, :T], k[:, :, :T], v[:, :, :T], alpha[:, :, :T],
                               beta[:, :, :T])
    St, zt = St[0], None if zt is None else zt[0]
    for i in range(n):
        t = T + i
        od, St, zt = oracle.decode_step(variant, St, q[0, :, t], k[0, :, t], v[0, :, t],
                                        alpha[0, :, t], beta[0, :, t], z=zt)
        assert rel(od, o[0, :, t]) < 1e-12
    assert rel(St, S[0]) < 1e-12


@pytest.mark.parametrize("variant", ["additive", "gated", "gated_delta"])
def test_linear_in_values_and_start_state(variant):
    r = rng(17)
    T, dk, dv = 33, 5, 4
    q, k, v1, alpha, beta = gdn_like(r, 1, 1, T, dk, dv)
    v2 = r.standard_normal(v1.shape)
    S1, S2 = r.standard_normal((2, 1, 1, dv, dk))
    c1, c2 = 0.7, -1.3
    oa, Sa, _ = oracle.prefill(variant, q, k, v1, alpha, beta, S0=S1)
    ob, Sb, _ = oracle.prefill(variant, q, k, v2, alpha, beta, S0=S2)
    oc, Sc, _ = oracle.prefill(variant, q, k, c1 * v1 + c2 * v2, alpha, beta, S0=c1 * S1 + c2 * S2)
    assert rel(oc, c1 * oa + c2 * ob) < 1e-12 and rel(Sc, c1 * Sa + c2 * Sb) < 1e-12


@pytest.mark.parametrize("variant", ["gated_delta", "based", "based_compact"])
def test_row_subset_matches_full(variant):
    """The sampled-rows path (used for long-sequence parity) returns the same numbers."""
    r = rng(18)
    T, dk, dv = 25, 4, 6
    q, k, v, alpha, beta = gdn_like(r, 2, 2, T, dk, dv)
    rows = [5, 0, 3]
    o, S, z = oracle.prefill(variant, q, k, v, alpha, beta)
    os_, Ss, zs = oracle.prefill(variant, q, k, v, alpha, beta, rows=rows)
    assert np.array_equal(os_, o[..., rows])
    if variant.startswith("based"):
        assert np.array_equal(Ss, S[..., rows]) and np.array_equal(zs, z)
    else:
        assert np.array_equal(Ss, S[:, :, rows, :])


def test_state_bytes_match_printed_accounting():
    J = GOLDEN["notebank_gdn_channels_J"]["value"]
    d = GOLDEN["notebank_gdn_dk_dv"]["value"]
    assert J == GOLDEN["notebank_gdn_layers"]["value"] * GOLDEN["notebank_gdn_heads_per_layer"]["value"]
    assert 4 * J * d * d == GOLDEN["notebank_fp32_state_MiB"]["value"] * 2 ** 20
    _, S, _ = oracle.prefill("gated_delta", *gdn_like(rng(19), 1, 1, 2, d, d))
    assert S[0, 0].size * 4 * J == 48 * 2 ** 20
    _, s, z = oracle.prefill("based", *gdn_like(rng(20), 1, 1, 2, 16, 64)[:3])
    assert s[0, 0].size + z[0, 0].size == 273 * (64 + 1)


def test_state_scale_pins():
    """S <- lambda S at the readout boundary ([NoteBank] App. C.3): lambda = 1 leaves the state
    unchanged and lambda = 0 resets it (the two values the pages fix), and rescaling the start
    state of a recurrence with zero values rescales its end state by the same factor (the
    decays act linearly on S, Eq. (1))."""
    rng = np.random.default_rng(5)
    S = rng.standard_normal((3, 4, 5))
    assert np.array_equal(oracle.state_scale(S, 1.0), S)
    Sbad = S.copy()
    Sbad[0, 0, 0] = np.inf
    assert np.array_equal(oracle.state_scale(Sbad, 0.0), np.zeros_like(S))
    B, H, T, d = 1, 2, 37, 8
    q, k = rng.standard_normal((B, H, T, d)), rng.standard_normal((B, H, T, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = np.zeros((B, H, T, d))
    al = rng.uniform(0.5, 1.0, (B, H, T))
    be = rng.uniform(0.0, 1.0, (B, H, T))
    S0 = rng.standard_normal((B, H, d, d))
    lam = 0.375
    _, S1, _ = oracle.prefill("gated_delta", q, k, v, al, be, S0=oracle.state_scale(S0, lam))
    _, S2, _ = oracle.prefill("gated_delta", q, k, v, al, be, S0=S0)
    assert np.allclose(S1, lam * S2, rtol=1e-13, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.state_scale(S, 1.25)

