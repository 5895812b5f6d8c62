"""C-ABI checks that need no GPU: the library loads, exports every symbol declared in
include/la.h, and rejects bad arguments before launching anything.  Every call here
fails validation (fake device addresses are never dereferenced)."""

import ctypes
import re
from pathlib import Path

import pytest

import gated_delta_rule_chunkwise_amd as la

ROOT = Path(__file__).resolve().parent.parent
HEADER = (ROOT / "include" / "la.h").read_text()

A = 1 << 20  # a fake, 16-byte aligned "device" address: validation never dereferences it


def declared_functions():
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s*(la_\w+)\s*\(", HEADER, re.M)))


@pytest.fixture(scope="module")
def lib():
    return la.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"la_prefill", "la_decode_step", "la_prefill_workspace_size",
                          "la_status_string", "la_abi_version"}
    raw = ctypes.CDLL(str(la.LIB_PATH))
    for n in names:
        assert hasattr(raw, n), f"libla.so does not export {n}"
    assert set(la.EXPORTS) <= set(names)


def test_version_and_status_strings(lib):
    assert lib.la_abi_version() == 1
    for code, name in la.STATUS.items():
        assert lib.la_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.la_status_string(12345)


def P(addr):
    return ctypes.c_void_p(addr)


def prefill(lib, variant=la.GATED_DELTA, dtype=la.BF16, B=1, H=2, T=100, dk=128, dv=128,
            q=A, k=2 * A, v=3 * A, alpha=4 * A, beta=5 * A, S0=None, z0=None, o=6 * A, S_T=8 * A,
            z_T=None, ws=None, ws_bytes=0):
    if ws is None:
        n = ctypes.c_size_t(0)
        st = lib.la_prefill_workspace_size(variant, dtype, B, H, T, dk, dv, ctypes.byref(n))
        if st == 0 and n.value:
            ws, ws_bytes = 64 * A, n.value
    return lib.la_prefill(variant, dtype, B, H, T, dk, dv, 1e-6, P(q), P(k), P(v),
                          None if alpha is None else P(alpha), None if beta is None else P(beta),
                          None if S0 is None else P(S0), None if z0 is None else P(z0), P(o),
                          None if S_T is None else P(S_T), None if z_T is None else P(z_T),
                          None if ws is None else P(ws), ws_bytes, None)


def test_prefill_rejects_bad_variant_and_dtype(lib):
    assert prefill(lib, variant=7) == -2
    assert prefill(lib, variant=5) == -2
    assert prefill(lib, variant=-1) == -2
    assert prefill(lib, dtype=5) == -2


def test_prefill_rejects_bad_sizes(lib):
    assert prefill(lib, B=0) == -2
    assert prefill(lib, H=-3) == -2
    assert prefill(lib, T=-1) == -2
    assert prefill(lib, dk=0) == -2


def test_prefill_unsupported_shapes(lib):
    assert prefill(lib, dk=96, dv=96) == -3
    assert prefill(lib, dk=128, dv=64) == -3
    assert prefill(lib, variant=la.BASED, alpha=None, beta=None, dk=8, dv=64) == -3


def test_prefill_variant_pointer_rules(lib):
    assert prefill(lib, variant=la.ADDITIVE) == -2             # alpha/beta must be NULL
    assert prefill(lib, variant=la.GATED, alpha=None) == -1    # alpha required
    assert prefill(lib, variant=la.GATED_DELTA, beta=None) == -1
    assert prefill(lib, q=0) == -1
    assert prefill(lib, variant=la.BASED, alpha=None, beta=None, dk=16, dv=64, S_T=8 * A,
                   z_T=None) == -2                              # s without z
    assert prefill(lib, z0=9 * A) == -2                         # z only for BASED


def test_prefill_alignment(lib):
    assert prefill(lib, q=A + 2) == -4
    assert prefill(lib, S_T=8 * A + 4) == -4


def test_prefill_aliasing(lib):
    # o overlapping q
    assert prefill(lib, o=A + 16) == -6
    # S_T overlapping o
    assert prefill(lib, S_T=6 * A + 64) == -6
    # S_T overlapping S0 without being the same buffer
    assert prefill(lib, S0=8 * A, S_T=8 * A + 256) == -6


def test_prefill_workspace_rules(lib):
    n = ctypes.c_size_t(0)
    assert lib.la_prefill_workspace_size(la.GATED_DELTA, la.BF16, 1, 16, 1 << 20, 128, 128,
                                         ctypes.byref(n)) == 0
    if n.value == 0:
        pytest.skip("this configuration needs no workspace")
    assert prefill(lib, T=1 << 20, H=16, ws=64 * A, ws_bytes=n.value - 1, q=A, k=A + (1 << 32),
                   v=A + (2 << 32), alpha=A + (3 << 32), beta=A + (4 << 32), o=A + (5 << 32),
                   S_T=A + (6 << 32)) == -5
    assert lib.la_prefill_workspace_size(la.GATED_DELTA, la.BF16, 1, 16, 100, 128, 128, None) == -1


def test_workspace_size_validates(lib):
    n = ctypes.c_size_t(0)
    assert lib.la_prefill_workspace_size(9, la.BF16, 1, 1, 10, 128, 128, ctypes.byref(n)) == -2
    assert lib.la_prefill_workspace_size(la.GATED_DELTA, la.BF16, 1, 1, 10, 96, 96,
                                         ctypes.byref(n)) == -3
    assert lib.la_prefill_workspace_size(la.GATED_DELTA, la.F32, 1, 1, 10, 128, 128,
                                         ctypes.byref(n)) == 0 and n.value == 0


def test_workspace_holds_one_transform_per_chunk(lib):
    """One segment per head (128 heads): at d = 256 the gated delta rule needs exactly one
    stored transform per chunk and head (the lower-triangular 64 x 64 bf16 T diag(beta)
    without the blocks right of the diagonal in its first 32 rows: 32 x 32 + 32 x 64
    values); at d = 128, where the passes form each chunk's solve from the keys they load,
    and for the gated variant, nothing."""
    n = ctypes.c_size_t(0)
    T = 64 * 100 + 5  # 101 chunks, the last partial
    assert lib.la_prefill_workspace_size(la.GATED_DELTA, la.BF16, 2, 64, T, 256, 256,
                                         ctypes.byref(n)) == 0
    assert n.value == 2 * 64 * 101 * (32 * 32 + 32 * 64) * 2
    for variant in (la.GATED_DELTA, la.GATED):
        assert lib.la_prefill_workspace_size(variant, la.BF16, 2, 64, T, 128, 128,
                                             ctypes.byref(n)) == 0
        assert n.value == 0


def test_width_256_plan_and_workspace(lib):
    """d_k = d_v = 256 (bf16) takes the chunk path: a replay workgroup carries a whole state
    (eight waves of 32 value rows), and when the sequence is split into segments one round of
    workgroups fills the chip (256 at d = 256, one per CU; 512 at d = 128, two per CU): 1M
    tokens over 8 heads of 256 make 32 segments of 512 chunks, over 16 heads of 128 32
    segments of 512; the workspace holds per segment a 512 x 256 fp32 map (B rows, then
    transition rows) and a 256 x 256 start state, and one stored transform per chunk."""
    n, c = ctypes.c_int(0), ctypes.c_int(0)
    for (H, d, plan) in ((8, 256, (32, 512)), (16, 128, (32, 512))):
        assert lib.la_prefill_segments(la.GATED_DELTA, la.BF16, 1, H, 1 << 20, d, d, ctypes.byref(n),
                                       ctypes.byref(c)) == 0
        assert (n.value, c.value) == plan
    up = lambda x: (x + 255) // 256 * 256
    ws = ctypes.c_size_t(0)
    assert lib.la_prefill_workspace_size(la.GATED_DELTA, la.BF16, 1, 8, 1 << 20, 256, 256,
                                         ctypes.byref(ws)) == 0
    bhs = 8 * 32
    assert ws.value == up(bhs * 512 * 256 * 4) + up(bhs * 4) + up(bhs * 256 * 256 * 4) + \
        8 * 16384 * (32 * 32 + 32 * 64) * 2
    # one segment once the heads alone reach half a round (128 workgroups)
    assert lib.la_prefill_segments(la.GATED, la.BF16, 8, 16, 1000, 256, 256, ctypes.byref(n),
                                   ctypes.byref(c)) == 0 and n.value == 1
    assert lib.la_prefill_segments(la.GATED, la.BF16, 4, 16, 1000, 256, 256, ctypes.byref(n),
                                   ctypes.byref(c)) == 0 and n.value == 4
    assert prefill(lib, dk=256, dv=128) == -3


def test_prefill_pass_rejects_unknown_pass(lib):
    for bad in (0, 5, -1):
        assert lib.la_prefill_pass(bad, la.GATED_DELTA, la.BF16, 1, 2, 100, 128, 128, 1e-6,
                                   P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), None, None,
                                   P(6 * A), P(8 * A), None, None, 0, None) == -2


def decode(lib, variant=la.GATED_DELTA, dtype=la.BF16, n=16, dk=128, dv=128, S_in=A, z_in=None,
           S_out=2 * A, z_out=None, q=4 * A, k=5 * A, v=6 * A, alpha=7 * A, beta=8 * A, o=9 * A):
    f = lambda x: None if x is None else P(x)
    return lib.la_decode_step(variant, dtype, n, dk, dv, 1e-6, f(S_in), f(z_in), f(S_out), f(z_out),
                              f(q), f(k), f(v), f(alpha), f(beta), f(o), None)


def test_decode_validation(lib):
    assert decode(lib, variant=5) == -2
    assert decode(lib, variant=la.BASED_COMPACT, alpha=None, beta=None, dk=16, dv=64) == -1  # z missing
    assert decode(lib, variant=la.BASED_COMPACT, alpha=None, beta=None, dk=16, dv=32) == -3
    assert decode(lib, n=0) == -2
    assert decode(lib, dk=100) == -3
    assert decode(lib, variant=la.BASED, alpha=None, beta=None, dk=16, dv=32) == -3
    assert decode(lib, S_in=None) == -1
    assert decode(lib, beta=None) == -1
    assert decode(lib, variant=la.ADDITIVE) == -2
    assert decode(lib, variant=la.BASED, alpha=None, beta=None, dk=16, dv=64) == -1  # z missing
    assert decode(lib, q=4 * A + 1) == -4             # q must be element aligned
    assert decode(lib, S_in=A + 8) == -4              # states 16-byte aligned
    assert decode(lib, o=6 * A + 32) == -6            # o overlaps v
    assert decode(lib, S_out=A + 1024) == -6          # partial overlap of the states


def test_state_scale_validation(lib):
    """la_state_scale validates before launching; n = 0 is a no-op (no device needed)."""
    f = lambda n=1024, lam=0.5, src=A, dst=2 * A: lib.la_state_scale(
        n, ctypes.c_float(lam), None if src is None else P(src), None if dst is None else P(dst), None)
    assert f(n=-1) == -2
    assert f(lam=1.5) == -2 and f(lam=-0.25) == -2 and f(lam=float("nan")) == -2
    assert f(n=0) == 0
    assert f(dst=None) == -1
    assert f(src=None) == -1           # lambda != 0 reads S_in
    assert f(src=A + 4) == -4 and f(dst=2 * A + 8) == -4
    assert f(dst=A + 16) == -6         # partial overlap (n = 1024 floats = 4 KiB)


def test_notebank_validation(lib):
    """The NoteBank entry points validate before launching (no device memory is touched)."""
    f = lambda x: None if x is None else P(x)
    ws = lambda dtype=la.BF16, B=1, H=4, T=1000, dk=128, C=512, k=A, dh=2 * A, dm=3 * A: \
        lib.la_write_scores(dtype, B, H, T, dk, C, f(k), f(dh), f(dm), None)
    assert ws(dtype=3) == -2 and ws(C=0) == -2 and ws(B=0) == -2
    assert ws(dk=96) == -3
    assert ws(k=None) == -1 and ws(dh=None) == -1
    assert ws(k=A + 8) == -4
    assert ws(dh=A) == -6  # output overlaps the keys
    assert ws(T=0, k=None) == 0
    ww = lambda B=1, T=1024, C=512, W=48, tail=32, dm=A, bs=2 * A, bv=3 * A: \
        lib.la_write_windows(B, T, C, W, tail, f(dm), f(bs), f(bv), None)
    assert ww(tail=600) == -2 and ww(W=0) == -2 and ww(tail=-1) == -2
    assert ww(bs=None) == -1 and ww(bs=A + 4) == -4
    assert ww(T=100, dm=None, bs=None) == 0  # no complete chunk: nothing to do
    na = lambda dtype=la.BF16, B=1, H=8, T=1000, dk=128, N=4, dr=16, dh=A, q=2 * A, sp=3 * A, co=4 * A, \
        ts=5 * A, rho=6 * A: lib.la_note_addresses(dtype, B, H, T, dk, N, dr, f(dh), f(q), f(sp), f(co),
                                                   f(ts), f(rho), None)
    assert na(H=17) == -3 and na(dr=200) == -3 and na(N=-1) == -2
    assert na(sp=None) == -1 and na(ts=A) == -6
    assert na(N=0, dh=None) == 0
    av = lambda dtype=la.BF16, N=100, J=8, nQ=20, dr=16, R=4, rho=A, u=2 * A, pos=3 * A, sc=4 * A, ch=5 * A, \
        vo=6 * A, se=7 * A: lib.la_address_votes(dtype, N, J, nQ, dr, f(rho), f(u), R, f(pos), f(sc), f(ch),
                                                 f(vo), f(se), None)
    assert av(dr=12) == -3 and av(nQ=2000) == -3 and av(R=65) == -3 and av(R=0) == -2 and av(N=20000) == -3
    assert av(ch=None) == -1 and av(se=A) == -6


def test_noalloc_rejects_before_any_hip_call(lib):
    """la_prefill_noalloc validates the shape and checks that the workspace fits its static
    scratch (even with one segment) before it touches the device."""
    args = [P(A), P(2 * A), P(3 * A), P(4 * A), P(5 * A), None, None, P(6 * A), P(8 * A), None, None]
    # 8 heads of 256 x 1M tokens of gated delta rule: the per-chunk transforms alone exceed it
    assert lib.la_prefill_noalloc(la.GATED_DELTA, la.BF16, 1, 8, 1 << 20, 256, 256, 1e-6, *args) == -5
    assert lib.la_prefill_noalloc(9, la.BF16, 1, 2, 100, 128, 128, 1e-6, *args) == -2
    assert lib.la_prefill_noalloc(la.GATED_DELTA, la.BF16, 1, 2, 100, 96, 96, 1e-6, *args) == -3
