"""Pins of the oracle's NoteBank write and address steps ("History Replays Itself", Sec. 3
Eqs. (3)-(5), App. B.2 Eq. (8), App. B.3 Eq. (9)) against closed forms, invariants, brute
force and the pages' own vote example.  CPU only."""

import math

import numpy as np

import oracle


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- write scores


def test_write_scores_two_direction_closed_form():
    """A chunk of n1 keys along e1 and n2 along e2 (any positive lengths): the normalised
    mean is (n1, n2)/sqrt(n1^2 + n2^2), so d = 1 - n1/sqrt(n1^2 + n2^2) for the e1 keys."""
    r = rng(1)
    dk, C, n1, n2 = 8, 40, 31, 9
    k = np.zeros((1, 1, C, dk))
    which = r.permutation(np.r_[np.zeros(n1, int), np.ones(n2, int)])
    k[0, 0, np.arange(C), which] = r.uniform(0.1, 5.0, C)
    d, dm = oracle.write_scores(k, chunk=C)
    h = math.hypot(n1, n2)
    want = np.where(which == 0, 1 - n1 / h, 1 - n2 / h)
    assert np.max(np.abs(d[0, 0] - want)) < 1e-14
    assert np.array_equal(dm[0], d[0, 0])


def test_write_scores_invariants():
    r = rng(2)
    B, H, T, dk, C = 2, 3, 700, 16, 256
    k = r.standard_normal((B, H, T, dk))
    d, dm = oracle.write_scores(k, chunk=C)
    assert d.min() >= 0 and d.max() <= 2
    assert np.max(np.abs(dm - d.mean(axis=1))) < 1e-15
    # positive rescaling of any key changes nothing (keys are normalised first)
    k2 = k * r.uniform(0.01, 100.0, (B, H, T, 1))
    assert np.max(np.abs(oracle.write_scores(k2, chunk=C)[0] - d)) < 1e-13
    # permuting tokens inside a chunk permutes their scores
    perm = np.r_[r.permutation(C), C + np.arange(T - C)]
    assert np.max(np.abs(oracle.write_scores(k[:, :, perm], chunk=C)[0] - d[:, :, perm])) < 1e-13
    # chunks are independent: changing chunk 1 leaves chunks 0 and 2 unchanged
    k3 = k.copy()
    k3[:, :, C:2 * C] = r.standard_normal((B, H, C, dk))
    d3 = oracle.write_scores(k3, chunk=C)[0]
    assert np.array_equal(d3[:, :, :C], d[:, :, :C]) and np.array_equal(d3[:, :, 2 * C:], d[:, :, 2 * C:])
    # the partial tail chunk uses its own tokens only
    dt = oracle.write_scores(k[:, :, 2 * C:], chunk=C)[0]
    assert np.max(np.abs(dt - d[:, :, 2 * C:])) < 1e-15
    # identical keys: zero distinctiveness; a zero key scores 1
    k4 = np.tile(r.standard_normal(dk), (1, 1, 10, 1))
    k4[0, 0, 3] = 0
    d4 = oracle.write_scores(k4, chunk=10)[0][0, 0]
    assert abs(d4[3] - 1) < 1e-15 and np.max(np.abs(np.delete(d4, 3))) < 1e-14


# ----------------------------------------------------------------------------- windows


def _windows_brute(d, C, W, tail):
    B, T = d.shape
    out = np.zeros((B, T // C), dtype=np.int64)
    for b in range(B):
        for c in range(T // C):
            lo, hi = max(0, c * C - tail), (c + 1) * C
            w = min(W, hi - lo)
            sums = [d[b, s:s + w].sum() for s in range(lo, hi - w + 1)]
            out[b, c] = lo + int(np.argmax(sums))
    return out


def test_write_windows_examples_and_brute_force():
    r = rng(3)
    C, W, tail, T = 512, 48, 32, 512 * 4 + 100
    d = np.zeros((1, T))
    d[0, 700] = 1.0                      # chunk 1: every window covering 700 ties -> earliest
    d[0, 2 * C - 10] = 2.0               # chunk 1's last tokens, seen again by chunk 2 (tail)
    s, v = oracle.write_windows(d, C, W, tail)
    assert s.shape == (1, 4)             # the 100-token incomplete tail makes no note
    assert s[0, 0] == 0 and v[0, 0] == 0  # all zero: the first window
    assert s[0, 1] == 2 * C - 10 - W + 1 and v[0, 1] == 2.0
    assert s[0, 2] == 2 * C - tail and v[0, 2] == 2.0
    # a region shorter than the window is scored as a whole
    s2, v2 = oracle.write_windows(d[:, :60], 20, 48, 0)
    assert list(s2[0]) == [0, 20, 40]
    dr = r.uniform(0, 2, (3, 512 * 3 + 7))
    assert np.array_equal(oracle.write_windows(dr, 512, 48, 32)[0], _windows_brute(dr, 512, 48, 32))


# ----------------------------------------------------------------------------- addresses


def test_note_addresses_argmax_and_gather():
    r = rng(4)
    B, H, T, dk, N, drho = 2, 3, 300, 32, 5, 16
    d = r.uniform(0, 2, (B, H, T))
    d[0, 1, 50:60] = 5.0                 # a tie inside note 0's span: the earliest wins
    q = r.standard_normal((B, H, T, dk))
    spans = np.stack([np.stack([r.integers(0, T - 64, N), r.integers(1, 65, N)], -1) for _ in range(B)])
    spans[0, 0] = (45, 20)
    coords = np.stack([r.permutation(dk)[:drho] for _ in range(H)])
    t_star, rho = oracle.note_addresses(d, q, spans, coords)
    assert t_star[0, 0, 1] == 50
    for b in range(B):
        for i in range(N):
            s0, ln = spans[b, i]
            for h in range(H):
                assert t_star[b, i, h] == s0 + int(np.argmax(d[b, h, s0:s0 + ln]))
                assert np.array_equal(rho[b, i, h], q[b, h, t_star[b, i, h], coords[h]])


def test_address_votes_pages_example():
    """Three channels vote A, B, A: A has two votes, B one; with R = 2 both come back, in
    document order (B sits before A in the text), with R = 1 only A."""
    e = np.eye(2)
    # notes A (index 0, later in the text) and B (index 1, earlier), channels j = 0, 1, 2
    rho = np.stack([np.stack([e[0], e[0], e[0]]), np.stack([e[1], e[1], e[1]])])  # [N=2, J=3, 2]
    u = np.stack([np.stack([e[0], 3 * e[1], 0.5 * e[0]])])                          # [nQ=1, J, 2]
    pos = [900, 100]
    score, choice, votes, sel = oracle.address_votes(rho, u, 2, pos)
    assert list(choice) == [0, 1, 0] and list(votes) == [2, 1]
    assert list(sel) == [1, 0]
    assert list(oracle.address_votes(rho, u, 1, pos)[3]) == [0]
    assert np.allclose(score, [[1, 0], [0, 1], [1, 0]])


def test_address_votes_max_over_question_and_ties():
    r = rng(5)
    N, J, nQ, drho = 6, 4, 3, 16
    rho = r.standard_normal((N, J, drho))
    u = r.standard_normal((nQ, J, drho))
    # channel 0: the second question token is exactly note 4's direction -> cosine 1
    u[1, 0] = 2.5 * rho[4, 0]
    # channel 1: notes 2 and 5 identical and the best -> the earlier one (2) gets the vote
    rho[5, 1] = rho[2, 1]
    u[0, 1] = rho[2, 1]
    score, choice, votes, sel = oracle.address_votes(rho, u, 3, np.arange(N) * 10)
    assert choice[0] == 4 and abs(score[0, 4] - 1) < 1e-14
    assert choice[1] == 2
    # brute force of the cosine maximum
    for j in range(J):
        for i in range(N):
            c = [u[t, j] @ rho[i, j] / np.linalg.norm(u[t, j]) / np.linalg.norm(rho[i, j]) for t in range(nQ)]
            assert abs(score[j, i] - max(c)) < 1e-14
    assert votes.sum() == J and sorted(v for v in sel if v >= 0) == sorted(set(choice))[:3]
    # equal votes: the earlier-inserted note is ranked first, then document order applies
    e = np.eye(2)
    rho2 = np.stack([np.stack([e[1], e[1]]), np.stack([e[1], e[0]]), np.stack([e[0], e[1]])])  # [N=3, J=2, 2]
    u2 = np.stack([e[0], e[0]])[None]                  # the question along e0 in both channels
    _, ch2, v2, s2 = oracle.address_votes(rho2, u2, 1, [5, 9, 3])
    assert list(ch2) == [2, 1] and list(v2) == [0, 1, 1] and list(s2) == [1]
    assert list(oracle.address_votes(rho2, u2, 3, [5, 9, 3])[3]) == [2, 1, -1]
