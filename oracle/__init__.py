"""fp64 CPU oracle for the generalized linear-attention recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  It shares no code with the HIP
library (``gated_delta_rule_chunkwise_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, per-token loops, OpenMP over
independent slices); this module only builds it with gcc, marshals numpy arrays and
promotes inputs exactly to float64.  What is computed, with citations:

* [NoteBank] "History Replays Itself: Unleashing Long-Context Capability in Linear
  Attention", Sec. 2 Preliminary, Eq. (1):  S_t = S_{t-1} A_t + beta_t v_t k_t^T,
  o_t = S_t q_t, with A_t = I (additive), alpha_t I (gated) or
  alpha_t (I - beta_t k_t k_t^T) (gated delta rule).
* [BASED] "Simple linear attention language models balance the recall-throughput
  tradeoff", Sec. 2.2 (paper Eqs. (1)-(3)) and Sec. 2.3 (paper Eq. (4)): Taylor feature
  map phi(x) = [1, x, vec(x x^T)/sqrt 2], s_t = s_{t-1} + phi(k_t) v_t^T,
  z_t = z_{t-1} + phi(k_t), o_t = s_t^T phi(q_t) / (z_t^T phi(q_t) + eps).
  ``based_compact``: the same recurrence with the compact map of the notes' feature-width
  table (Sec. 2.3), [1, x, x_a^2/sqrt 2 (a = b), x_a x_b (a < b)], pairs in row-major
  upper-triangle order (D = 1 + d' + d'(d'+1)/2 = 153 for d' = 16).

* [NoteBank] App. B Algorithm 1 and App. C.3: the retained state is copied for each
  branch and rescaled at the readout boundary, S <- lambda S, lambda in [0, 1]
  (``state_scale``; lambda = 0 is read as the reset to the zero state).
* [NoteBank] Sec. 3 Eqs. (3)-(5), App. B.2 Eq. (8), App. B.3 Eq. (9): the write step's key
  distinctiveness per write chunk (``write_scores``), the best scoring window of each
  complete chunk (``write_windows``), the per-channel note addresses (``note_addresses``)
  and the addressing votes (``address_votes``).  Argmax ties go to the earliest index.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, brute force and invariants.  The eps convention and the absence of
input scaling for BASED are chosen conventions that no page value fixes
("parity unpinned" for those two choices only).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

ADDITIVE, BASED, GATED, GATED_DELTA, BASED_COMPACT = 0, 1, 2, 3, 4
VARIANTS = {"additive": ADDITIVE, "based": BASED, "gated": GATED, "gated_delta": GATED_DELTA,
            "based_compact": BASED_COMPACT}

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile oracle.c with gcc into liboracle.so (fp64, no fast-math, no FMA contraction)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("ORACLE_LIB")  # test hook: load a deliberately broken build
    if override:
        lib = ctypes.CDLL(override)
    else:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB))
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_prefill.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long,
                                   ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp,
                                   ctypes.c_double, ip, ctypes.c_int, dp, dp, dp, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_decode_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       dp, dp, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, dp,
                                       ctypes.c_int]
    lib.oracle_decode_step.restype = ctypes.c_int
    lib.oracle_literal.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                   dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_literal.restype = ctypes.c_int
    lib.oracle_based_phi.argtypes = [dp, ctypes.c_int, dp]
    lib.oracle_based_phi.restype = None
    lib.oracle_based_phi_compact.argtypes = [dp, ctypes.c_int, dp]
    lib.oracle_based_phi_compact.restype = None
    lib.oracle_max_threads.restype = ctypes.c_int
    lp = ctypes.POINTER(ctypes.c_long)
    lib.oracle_write_scores.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_int,
                                        ctypes.c_long, dp, dp, dp]
    lib.oracle_write_scores.restype = ctypes.c_int
    lib.oracle_write_windows.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                         ctypes.c_long, dp, lp, dp]
    lib.oracle_write_windows.restype = ctypes.c_int
    lib.oracle_note_addresses.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_long, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, dp, dp, lp, ip, lp, dp]
    lib.oracle_note_addresses.restype = ctypes.c_int
    lib.oracle_address_votes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp,
                                         ctypes.c_int, lp, dp, ip, ip, ip]
    lib.oracle_address_votes.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a):
    """Exact promotion to contiguous float64 (bf16 and fp32 values are exact in fp64)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: exact float32 view of bf16/fp32 values
        a = a.detach().float().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _variant(v) -> int:
    return VARIANTS[v] if isinstance(v, str) else int(v)


def feature_dim(dp: int, compact: bool = False) -> int:
    return 1 + dp + dp * (dp + 1) // 2 if compact else 1 + dp + dp * dp


def max_threads() -> int:
    return _load().oracle_max_threads()


def prefill(variant, q, k, v, alpha=None, beta=None, S0=None, z0=None, eps=1e-6, rows=None,
            want_state=True, nthreads=0):
    """Run the recurrence over T tokens.

    q, k: [B, H, T, d_k]; v: [B, H, T, d_v]; alpha, beta: [B, H, T]; S0: [B, H, d_v, d_k]
    (BASED: s0 [B, H, D, d_v], z0 [B, H, D]).  ``rows`` selects value rows (GDN family) or
    value columns (BASED).  Returns (o, S_T, z_T) in float64; z_T is None unless BASED.
    """
    var = _variant(variant)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    alpha = _f64(alpha) if var in (GATED, GATED_DELTA) else None
    beta = _f64(beta) if var in (GATED, GATED_DELTA) else None
    S0, z0 = _f64(S0), _f64(z0)
    if rows is None:
        nr, rows_arr = dv, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nr = int(rows_arr.size)
    o = np.zeros((B, H, T, nr), dtype=np.float64)
    if var in (BASED, BASED_COMPACT):
        D = feature_dim(dk, var == BASED_COMPACT)
        S_T = np.zeros((B, H, D, nr)) if want_state else None
        z_T = np.zeros((B, H, D)) if want_state else None
    else:
        S_T = np.zeros((B, H, nr, dk)) if want_state else None
        z_T = None
    rc = _load().oracle_prefill(
        var, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0),
        _ptr(z0), float(eps),
        None if rows_arr is None else rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
        nr, _ptr(o), _ptr(S_T), _ptr(z_T), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return o, S_T, z_T


def decode_step(variant, S, q, k, v, alpha=None, beta=None, z=None, eps=1e-6, nthreads=0):
    """One recurrence step for N independent states.  S: [N, d_v, d_k] (BASED: s [N, D, d_v]
    and z [N, D]); q, k: [N, d_k]; v: [N, d_v]; alpha, beta: [N].  Returns (o, S', z')."""
    var = _variant(variant)
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, dk = q.shape
    dv = v.shape[-1]
    S = _f64(S)
    z = _f64(z)
    alpha = _f64(alpha) if var in (GATED, GATED_DELTA) else None
    beta = _f64(beta) if var in (GATED, GATED_DELTA) else None
    o = np.zeros((N, dv))
    if var in (BASED, BASED_COMPACT):
        D = feature_dim(dk, var == BASED_COMPACT)
        S_out, z_out = np.zeros((N, D, dv)), np.zeros((N, D))
    else:
        S_out, z_out = np.zeros((N, dv, dk)), None
    rc = _load().oracle_decode_step(var, N, dk, dv, _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(alpha), _ptr(beta), float(eps), _ptr(S_out), _ptr(z_out),
                                    _ptr(o), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    return o, S_out, z_out


def literal(variant, q, k, v, alpha=None, beta=None, S0=None):
    """Explicit-A_t form for one (b,h) slice (tiny inputs only): q,k [T,d_k], v [T,d_v]."""
    var = _variant(variant)
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, dk = q.shape
    dv = v.shape[-1]
    alpha = _f64(alpha) if var in (GATED, GATED_DELTA) else None
    beta = _f64(beta) if var in (GATED, GATED_DELTA) else None
    S0 = _f64(S0)
    o = np.zeros((T, dv))
    S_T = np.zeros((dv, dk))
    rc = _load().oracle_literal(var, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T))
    if rc != 0:
        raise ValueError("oracle_literal rejected its arguments")
    return o, S_T


def based_phi(x):
    """phi(x) for a 1-D vector x (fp64)."""
    x = _f64(x)
    f = np.zeros(feature_dim(x.size))
    _load().oracle_based_phi(_ptr(x), int(x.size), _ptr(f))
    return f


def based_phi_compact(x):
    """The compact map phi_c(x) for a 1-D vector x (fp64)."""
    x = _f64(x)
    f = np.zeros(feature_dim(x.size, compact=True))
    _load().oracle_based_phi_compact(_ptr(x), int(x.size), _ptr(f))
    return f


def _lptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_long))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def write_scores(k, chunk=512):
    """Key distinctiveness d_t = 1 - <khat_t, mubar> per write chunk and head (Eqs. (3), (8)).
    k [B, H, T, d_k].  Returns (d_head [B, H, T], d_mean [B, T]) in float64."""
    k = _f64(k)
    B, H, T, dk = k.shape
    d_head, d_mean = np.zeros((B, H, T)), np.zeros((B, T))
    if _load().oracle_write_scores(B, H, T, dk, int(chunk), _ptr(k), _ptr(d_head), _ptr(d_mean)) != 0:
        raise ValueError("oracle_write_scores rejected its arguments")
    return d_head, d_mean


def write_windows(d_mean, chunk=512, window=48, tail=32):
    """Best window (start, sum) per complete write chunk of d_mean [B, T] (App. B.2)."""
    d = _f64(d_mean)
    B, T = d.shape
    nc = T // chunk
    start, val = np.zeros((B, nc), dtype=np.int64), np.zeros((B, nc))
    if _load().oracle_write_windows(B, T, int(chunk), int(window), int(tail), _ptr(d), _lptr(start),
                                    _ptr(val)) != 0:
        raise ValueError("oracle_write_windows rejected its arguments")
    return start, val


def note_addresses(d_head, q, spans, coords):
    """Eqs. (4), (9): t* [B, N, H] = argmax of d_head over each note's span, rho [B, N, H, d_rho]
    = q at t* on the head's coordinates.  spans [B, N, 2] (start, length); coords [H, d_rho]."""
    d, q = _f64(d_head), _f64(q)
    B, H, T, dk = q.shape
    spans = np.ascontiguousarray(np.asarray(spans, dtype=np.int64))
    coords = np.ascontiguousarray(np.asarray(coords, dtype=np.int32))
    N, drho = spans.shape[1], coords.shape[1]
    t_star, rho = np.zeros((B, N, H), dtype=np.int64), np.zeros((B, N, H, drho))
    if _load().oracle_note_addresses(B, H, T, dk, N, drho, _ptr(d), _ptr(q), _lptr(spans), _iptr(coords),
                                     _lptr(t_star), _ptr(rho)) != 0:
        raise ValueError("oracle_note_addresses rejected its arguments")
    return t_star, rho


def address_votes(rho, u, R, positions):
    """Eq. (5): rho [N, J, d_rho] note addresses, u [n_Q, J, d_rho] question features.
    Returns (score [J, N], choice [J], votes [N], selected [R], -1 padded, in document order)."""
    rho, u = _f64(rho), _f64(u)
    N, J, drho = rho.shape
    nQ = u.shape[0]
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    score = np.zeros((J, N))
    choice, votes = np.zeros(J, dtype=np.int32), np.zeros(N, dtype=np.int32)
    sel = np.zeros(R, dtype=np.int32)
    if _load().oracle_address_votes(N, J, nQ, drho, _ptr(rho), _ptr(u), int(R), _lptr(pos), _ptr(score),
                                    _iptr(choice), _iptr(votes), _iptr(sel)) != 0:
        raise ValueError("oracle_address_votes rejected its arguments")
    return score, choice, votes, sel


def state_scale(S, lam):
    """S <- lambda S ([NoteBank] App. C.3: lambda in [0, 1], 1 leaves the state unchanged,
    0 resets it).  fp64; lambda = 0 gives the zero state whatever S holds (the reset)."""
    lam = float(lam)
    if not 0.0 <= lam <= 1.0:
        raise ValueError("lambda must lie in [0, 1]")
    x = _f64(S)
    return np.zeros_like(x) if lam == 0.0 else lam * x

