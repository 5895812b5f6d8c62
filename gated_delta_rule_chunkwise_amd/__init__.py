"""Python binding of libla (MI355X / gfx950 linear-attention recurrence).

Thin argument marshalling only: torch tensors provide device memory and the stream;
every step of the computation runs in the HIP kernels behind the C ABI of
``include/la.h``.  There is no CPU fallback -- if ``libla.so`` is missing or cannot be
loaded, every call raises.

    o, S_T, z_T = prefill("gated_delta", q, k, v, alpha, beta, S0=None)
    o, S, z     = decode_step("gated_delta", S, q, k, v, alpha, beta, S_out=S)  # in place
"""

from __future__ import annotations

import ctypes
from pathlib import Path

import torch

ADDITIVE, BASED, GATED, GATED_DELTA, BASED_COMPACT = 0, 1, 2, 3, 4
VARIANTS = {"additive": ADDITIVE, "based": BASED, "gated": GATED, "gated_delta": GATED_DELTA,
            "based_compact": BASED_COMPACT}
F32, BF16 = 0, 1
STATUS = {0: "LA_OK", -1: "LA_ERR_NULL", -2: "LA_ERR_INVALID", -3: "LA_ERR_UNSUPPORTED",
          -4: "LA_ERR_ALIGN", -5: "LA_ERR_WORKSPACE", -6: "LA_ERR_ALIAS", -7: "LA_ERR_HIP"}
EXPORTS = ("la_abi_version", "la_status_string", "la_prefill_workspace_size", "la_prefill",
           "la_prefill_pass", "la_prefill_segments", "la_decode_step",
           "la_write_scores", "la_write_windows", "la_note_addresses", "la_address_votes",
           "la_state_scale", "la_prefill_noalloc")
NOALLOC_SCRATCH_BYTES = 128 << 20  # LA_NOALLOC_SCRATCH_BYTES
PASS_MAPS, PASS_SCAN, PASS_REPLAY, PASS_TRANSFORM = 1, 2, 3, 4

LIB_PATH = Path(__file__).resolve().parent / "libla.so"
_lib = None


class LAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def load(path: str | None = None):
    """Load libla.so (raises OSError if it is missing or broken)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise OSError(f"{p} not found: build it with `python -m gated_delta_rule_chunkwise_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.la_abi_version.restype = i32
    lib.la_status_string.argtypes = [i32]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i64, i32, i32,
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.la_prefill_workspace_size.restype = i32
    lib.la_prefill.argtypes = [i32, i32, i32, i32, i64, i32, i32, f32] + [vp] * 11 + \
        [ctypes.c_size_t, vp]
    lib.la_prefill.restype = i32
    lib.la_prefill_pass.argtypes = [i32] + lib.la_prefill.argtypes
    lib.la_prefill_pass.restype = i32
    lib.la_prefill_noalloc.argtypes = [i32, i32, i32, i32, i64, i32, i32, f32] + [vp] * 11
    lib.la_prefill_noalloc.restype = i32
    lib.la_prefill_segments.argtypes = [i32, i32, i32, i32, i64, i32, i32,
                                        ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.la_prefill_segments.restype = i32
    lib.la_decode_step.argtypes = [i32, i32, i32, i32, i32, f32] + [vp] * 10 + [vp]
    lib.la_decode_step.restype = i32
    lib.la_write_scores.argtypes = [i32, i32, i32, i64, i32, i32, vp, vp, vp, vp]
    lib.la_write_scores.restype = i32
    lib.la_write_windows.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.la_write_windows.restype = i32
    lib.la_note_addresses.argtypes = [i32, i32, i32, i64, i32, i32, i32] + [vp] * 7
    lib.la_note_addresses.restype = i32
    lib.la_address_votes.argtypes = [i32, i32, i32, i32, i32, vp, vp, i32] + [vp] * 6
    lib.la_address_votes.restype = i32
    lib.la_state_scale.argtypes = [i64, f32, vp, vp, vp]
    lib.la_state_scale.restype = i32
    if path is None:
        _lib = lib
    return lib


def _var(v) -> int:
    return VARIANTS[v] if isinstance(v, str) else int(v)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def feature_dim(dp: int, compact: bool = False) -> int:
    """State rows of the BASED variants: 1 + d' + d'^2, or 1 + d' + d'(d'+1)/2 (compact)."""
    return 1 + dp + dp * (dp + 1) // 2 if compact else 1 + dp + dp * dp


def workspace_size(variant, dtype, B, H, T, d_k, d_v) -> int:
    n = ctypes.c_size_t(0)
    st = load().la_prefill_workspace_size(_var(variant), dtype, B, H, T, d_k, d_v, ctypes.byref(n))
    if st != 0:
        raise LAError(st, "la_prefill_workspace_size")
    return int(n.value)


def segments(variant, dtype, B, H, T, d_k, d_v):
    """(n_segments, chunks_per_segment) that la_prefill uses for this problem."""
    n, c = ctypes.c_int(0), ctypes.c_int(0)
    st = load().la_prefill_segments(_var(variant), dtype, B, H, T, d_k, d_v, ctypes.byref(n),
                                    ctypes.byref(c))
    if st != 0:
        raise LAError(st, "la_prefill_segments")
    return n.value, c.value


def prefill_passes(variant, dtype, B, H, T, d_k, d_v):
    """The passes la_prefill runs for this problem, in order: calling la_prefill_pass with
    each in turn (same buffers, one workspace) is la_prefill."""
    nseg, _ = segments(variant, dtype, B, H, T, d_k, d_v)
    # the stored transforms exist at d = 256 only (at 128 the passes form each chunk's solve)
    ps = [PASS_TRANSFORM] if (_var(variant) == GATED_DELTA and dtype == BF16 and d_k == d_v == 256) else []
    if nseg > 1:
        ps += [PASS_MAPS, PASS_SCAN]
    return ps + [PASS_REPLAY]


def prefill(variant, q, k, v, alpha=None, beta=None, S0=None, z0=None, eps=1e-6, want_state=True,
            o=None, S_T=None, z_T=None, workspace=None, stream=None, pass_=None):
    """Run la_prefill (or one pass of it, ``pass_`` in PASS_TRANSFORM/MAPS/SCAN/REPLAY, see la.h).
    q, k [B,H,T,d_k]; v [B,H,T,d_v]; alpha, beta [B,H,T] (same dtype as q); S0 [B,H,d_v,d_k]
    fp32 (BASED: s0 [B,H,D,d_v], z0 [B,H,D]).  Returns (o, S_T, z_T)."""
    var = _var(variant)
    lib = load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype(q)
    dev = q.device
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    if want_state and S_T is None:
        if var in (BASED, BASED_COMPACT):
            D = feature_dim(dk, var == BASED_COMPACT)
            S_T = torch.empty((B, H, D, dv), dtype=torch.float32, device=dev)
            z_T = torch.empty((B, H, D), dtype=torch.float32, device=dev) if z_T is None else z_T
        else:
            S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    ws_n = workspace_size(var, dt, B, H, T, dk, dv)
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    args = (var, dt, B, H, T, dk, dv, float(eps), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(S0),
            _p(z0), _p(o), _p(S_T), _p(z_T), _p(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream))
    st = lib.la_prefill(*args) if pass_ is None else lib.la_prefill_pass(int(pass_), *args)
    if st != 0:
        raise LAError(st, "la_prefill" if pass_ is None else "la_prefill_pass")
    return o, S_T, z_T


def prefill_noalloc(variant, q, k, v, alpha=None, beta=None, S0=None, z0=None, eps=1e-6, o=None,
                    S_T=None, z_T=None, stream=None):
    """Run la_prefill_noalloc: la_prefill with its workspace in the library's static device
    scratch (the call itself allocates nothing; pass o and S_T (z_T) to allocate nothing
    here either).  Same layouts as prefill().  Returns (o, S_T, z_T)."""
    var = _var(variant)
    lib = load()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_T is None:
        if var in (BASED, BASED_COMPACT):
            D = feature_dim(dk, var == BASED_COMPACT)
            S_T = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
            z_T = torch.empty((B, H, D), dtype=torch.float32, device=q.device) if z_T is None else z_T
        else:
            S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
    st = lib.la_prefill_noalloc(var, _dtype(q), B, H, T, dk, dv, float(eps), _p(q), _p(k), _p(v), _p(alpha),
                                _p(beta), _p(S0), _p(z0), _p(o), _p(S_T), _p(z_T), _stream(stream))
    if st != 0:
        raise LAError(st, "la_prefill_noalloc")
    return o, S_T, z_T


def decode_step(variant, S, q, k, v, alpha=None, beta=None, z=None, eps=1e-6, S_out=None,
                z_out=None, o=None, stream=None):
    """Run la_decode_step on N states.  S [N,d_v,d_k] (BASED: s [N,D,d_v], z [N,D]); q,k [N,d_k];
    v [N,d_v]; alpha, beta [N].  S_out=S (and z_out=z) updates in place.  Returns (o, S_out, z_out)."""
    var = _var(variant)
    lib = load()
    N, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype(q)
    if o is None:
        o = torch.empty((N, dv), dtype=q.dtype, device=q.device)
    if S_out is None:
        S_out = torch.empty_like(S)
    if var in (BASED, BASED_COMPACT) and z_out is None:
        z_out = torch.empty_like(z)
    st = lib.la_decode_step(var, dt, N, dk, dv, float(eps), _p(S), _p(z), _p(S_out), _p(z_out),
                            _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(o), _stream(stream))
    if st != 0:
        raise LAError(st, "la_decode_step")
    return o, S_out, z_out


# ------------------------------------------------------------------ NoteBank write / address steps


def write_scores(k, chunk=512, d_head=None, d_mean=None, stream=None):
    """la_write_scores: key distinctiveness per write chunk.  k [B,H,T,d_k] (fp32 or bf16).
    Returns (d_head [B,H,T], d_mean [B,T]) fp32."""
    B, H, T, dk = k.shape
    if d_head is None:
        d_head = torch.empty((B, H, T), dtype=torch.float32, device=k.device)
    if d_mean is None:
        d_mean = torch.empty((B, T), dtype=torch.float32, device=k.device)
    st = load().la_write_scores(_dtype(k), B, H, T, dk, int(chunk), _p(k), _p(d_head), _p(d_mean),
                                _stream(stream))
    if st != 0:
        raise LAError(st, "la_write_scores")
    return d_head, d_mean


def write_windows(d_mean, chunk=512, window=48, tail=32, stream=None):
    """la_write_windows: (best_start [B, T//chunk] int64, best_sum fp32) per complete chunk."""
    B, T = d_mean.shape
    nc = T // chunk
    start = torch.empty((B, nc), dtype=torch.int64, device=d_mean.device)
    val = torch.empty((B, nc), dtype=torch.float32, device=d_mean.device)
    st = load().la_write_windows(B, T, int(chunk), int(window), int(tail), _p(d_mean), _p(start), _p(val),
                                 _stream(stream))
    if st != 0:
        raise LAError(st, "la_write_windows")
    return start, val


def note_addresses(d_head, q, spans, coords, stream=None):
    """la_note_addresses: (t_star [B,N,H] int64, rho [B,N,H,d_rho] in q's dtype) for spans
    [B,N,2] int64 (start, length) and coords [H,d_rho] int32."""
    B, H, T, dk = q.shape
    N, drho = spans.shape[1], coords.shape[1]
    t_star = torch.empty((B, N, H), dtype=torch.int64, device=q.device)
    rho = torch.empty((B, N, H, drho), dtype=q.dtype, device=q.device)
    st = load().la_note_addresses(_dtype(q), B, H, T, dk, N, drho, _p(d_head), _p(q), _p(spans), _p(coords),
                                  _p(t_star), _p(rho), _stream(stream))
    if st != 0:
        raise LAError(st, "la_note_addresses")
    return t_star, rho


def address_votes(rho, u, R, positions, want_score=True, stream=None):
    """la_address_votes: rho [N,J,d_rho], u [n_Q,J,d_rho] (same dtype), positions [N] int64.
    Returns (score [J,N] fp32 or None, choice [J], votes [N], selected [R]) int32."""
    N, J, drho = rho.shape
    nQ = u.shape[0]
    dev = rho.device
    score = torch.empty((J, N), dtype=torch.float32, device=dev) if want_score else None
    choice = torch.empty(J, dtype=torch.int32, device=dev)
    votes = torch.empty(N, dtype=torch.int32, device=dev)
    sel = torch.empty(R, dtype=torch.int32, device=dev)
    st = load().la_address_votes(_dtype(rho), N, J, nQ, drho, _p(rho), _p(u), int(R), _p(positions), _p(score),
                                 _p(choice), _p(votes), _p(sel), _stream(stream))
    if st != 0:
        raise LAError(st, "la_address_votes")
    return score, choice, votes, sel


def state_scale(S, lam, out=None, stream=None):
    """la_state_scale: out = lam * S for an fp32 state of any shape (lam in [0, 1]; lam = 0
    writes zeros).  out=S rescales in place; out=None returns a new tensor (with lam = 1,
    the copy a replay branch starts from)."""
    if S.dtype != torch.float32:
        raise TypeError("states are float32")
    if out is None:
        out = torch.empty_like(S)
    elif out.dtype != torch.float32 or out.numel() != S.numel():
        raise ValueError("out must be a float32 tensor with as many elements as S")
    st = load().la_state_scale(S.numel(), float(lam), _p(S), _p(out), _stream(stream))
    if st != 0:
        raise LAError(st, "la_state_scale")
    return out

