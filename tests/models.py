"""fp64 numpy models of the chunked decomposition the kernels implement.

These are test helpers, not the oracle: they are checked *against* the oracle (which
walks the recurrence token by token) so that the block algebra the HIP kernels rely on
is pinned independently of GPU precision.  Nothing here is imported by the library.

Derivation (from Eq. (1) of "History Replays Itself", Sec. 2; the BASED notes' Sec. 2.5
block decomposition U_b = (M_b . Phi_Q Phi_K^T) V_b + Phi_Q S_{<b} is the additive
special case).  Inside a chunk of n tokens with entering state S (d_v x d_k):
    g_t = sum_{i<=t} log alpha_i,   gamma_t = exp(g_t),   P_tj = exp(g_t - g_j) [j <= t]
    gated delta:  u_t = beta_t (v_t - alpha_t S_{t-1} k_t)
                  (I + L) U = diag(beta) V - diag(beta gamma) K S^T,
                  L_tj = beta_t exp(g_t - g_j) k_t.k_j  (j < t)
                  T = (I + L)^{-1},  W = T diag(beta gamma) K,  U~ = T diag(beta) V,
                  U = U~ - W S^T
    gated / additive: U = diag(beta) V (no solve)
    O  = diag(gamma) Q S^T + (P . Q K^T) U
    S' = gamma_n S + U^T diag(exp(g_n - g)) K  =  S M_c + B_c,
         M_c = gamma_n I - W^T diag(exp(g_n - g)) K,   B_c = U~^T diag(exp(g_n - g)) K
"""

from __future__ import annotations

import numpy as np


def chunk_step(variant, Q, K, V, a, b, S):
    """One chunk; returns (O, S_next).  variant in {'additive','gated','gated_delta'}."""
    n = Q.shape[0]
    if variant == "additive":
        a = np.ones(n)
        b = np.ones(n)
    elif b is None:
        b = np.ones(n)
    g = np.cumsum(np.log(a))
    gamma = np.exp(g)
    E = np.exp(np.minimum(g[:, None] - g[None, :], 0.0))  # only j <= t is used
    P = np.tril(E)
    if variant == "gated_delta":
        L = np.tril(b[:, None] * E * (K @ K.T), -1)
        T = np.linalg.inv(np.eye(n) + L)
        W = T @ ((b * gamma)[:, None] * K)
        Ut = T @ (b[:, None] * V)
        U = Ut - W @ S.T
    else:
        U = b[:, None] * V
    O = gamma[:, None] * (Q @ S.T) + (P * (Q @ K.T)) @ U
    S_next = gamma[-1] * S + U.T @ (np.exp(g[-1] - g)[:, None] * K)
    return O, S_next


def chunked(variant, q, k, v, alpha, beta, S0, C):
    """Chunked evaluation of one (b,h) slice: q,k [T,dk], v [T,dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        a = None if alpha is None else alpha[sl]
        bb = None if beta is None else beta[sl]
        o[sl], S = chunk_step(variant, q[sl], k[sl], v[sl], a, bb, S)
    return o, S


def chunk_map(variant, K, V, a, b):
    """The chunk's affine map S -> S M_c + B_c (M_c d_k x d_k, B_c d_v x d_k)."""
    n, dk = K.shape
    if variant == "additive":
        a = np.ones(n)
        b = np.ones(n)
    elif b is None:
        b = np.ones(n)
    g = np.cumsum(np.log(a))
    gamma = np.exp(g)
    dec = np.exp(g[-1] - g)
    if variant == "gated_delta":
        E = np.exp(np.minimum(g[:, None] - g[None, :], 0.0))
        L = np.tril(b[:, None] * E * (K @ K.T), -1)
        T = np.linalg.inv(np.eye(n) + L)
        W = T @ ((b * gamma)[:, None] * K)
        Ut = T @ (b[:, None] * V)
        M = gamma[-1] * np.eye(dk) - W.T @ (dec[:, None] * K)
    else:
        Ut = b[:, None] * V
        M = gamma[-1] * np.eye(dk)
    Bc = Ut.T @ (dec[:, None] * K)
    return M, Bc


def segmented(variant, q, k, v, alpha, beta, S0, C, seg_chunks):
    """Three-pass segment scan: per-segment maps from a zero/identity start, a
    sequential scan of segment start states, then a rerun of every segment."""
    T, dk = q.shape
    dv = v.shape[1]
    seg = C * seg_chunks
    starts = list(range(0, T, seg))
    maps = []
    for s0 in starts:
        M = np.eye(dk)
        Bm = np.zeros((dv, dk))
        for c0 in range(s0, min(s0 + seg, T), C):
            sl = slice(c0, min(c0 + C, T))
            a = None if alpha is None else alpha[sl]
            bb = None if beta is None else beta[sl]
            Mc, Bc = chunk_map(variant, k[sl], v[sl], a, bb)
            M, Bm = M @ Mc, Bm @ Mc + Bc
        maps.append((M, Bm))
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    seg_start = []
    for M, Bm in maps:
        seg_start.append(S)
        S = S @ M + Bm
    o = np.zeros((T, dv))
    for s0, Sst in zip(starts, seg_start):
        sl = slice(s0, min(s0 + seg, T))
        a = None if alpha is None else alpha[sl]
        bb = None if beta is None else beta[sl]
        o[sl], _ = chunked(variant, q[sl], k[sl], v[sl], a, bb, Sst, C)
    return o, S


def windowed_segmented(variant, q, k, v, alpha, beta, S0, C, seg_chunks, window, force=False):
    """segmented(), with each segment's map formed as the map pass forms it: first from its
    last `window` chunks alone; when their composed transition is exactly zero the
    segment's map is (0, B_last), since the whole map composes as M = M_first M_last,
    B = B_first M_last + B_last; otherwise from all its chunks.  force=True takes the
    window's map even when its transition is not zero (a planted mistake)."""
    T, dk = q.shape
    dv = v.shape[1]
    seg = C * seg_chunks
    starts = list(range(0, T, seg))

    def compose(c_from, c_to):
        M = np.eye(dk)
        Bm = np.zeros((dv, dk))
        for c0 in range(c_from, c_to, C):
            sl = slice(c0, min(c0 + C, T))
            a = None if alpha is None else alpha[sl]
            bb = None if beta is None else beta[sl]
            Mc, Bc = chunk_map(variant, k[sl], v[sl], a, bb)
            M, Bm = M @ Mc, Bm @ Mc + Bc
        return M, Bm

    maps, used_window = [], []
    for s0 in starts:
        s1 = min(s0 + seg, T)
        nch = (s1 - s0 + C - 1) // C
        if nch > 2 * window:
            Mw, Bw = compose(s1 - window * C, s1)
            if force or not np.any(Mw):
                maps.append((np.zeros((dk, dk)) if not force else Mw, Bw))
                used_window.append(True)
                continue
        maps.append(compose(s0, s1))
        used_window.append(False)
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    seg_start = []
    for M, Bm in maps:
        seg_start.append(S)
        S = S @ M + Bm
    o = np.zeros((T, dv))
    for s0, Sst in zip(starts, seg_start):
        sl = slice(s0, min(s0 + seg, T))
        a = None if alpha is None else alpha[sl]
        bb = None if beta is None else beta[sl]
        o[sl], _ = chunked(variant, q[sl], k[sl], v[sl], a, bb, Sst, C)
    return o, S, used_window
