"""GPU parity of the NoteBank write and address steps (la_write_scores, la_write_windows,
la_note_addresses, la_address_votes) against the fp64 oracle on the same seeded inputs.

Where a floating-point value decides an index (an argmax), both sides decide on the same
fp32 numbers when the step's input is fp32 (note addresses: the d_head values), so the
indices must match exactly; where the deciding value is itself computed (window sums,
cosines), the GPU's choice must match the oracle's whenever the oracle's best beats the
runner-up by more than the arithmetic's error bound, and otherwise be one of the tied
candidates.  Integer bookkeeping downstream (votes, selection, document order) is exact."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def assert_abs(x, y, tol, what):
    """Max absolute error (the scores live in [0, 2], so an absolute bound is the natural one)."""
    err = float(np.max(np.abs(to64(x) - to64(y)))) if np.size(to64(y)) else 0.0
    print(f"    parity {what}: max abs err {err:.3e} (bound {tol:.0e})", flush=True)
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _keys(B, H, T, dk, dtype, seed):
    d = synth.gdn_inputs(B, H, T, dk, dk, dtype=dtype, seed=seed, device=DEV, normalize=False)
    return d["k"], d["q"]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk", [64, 128, 256])
def test_write_scores(la, dtype, dk):
    B, H, T, C = 2, 3, 512 * 3 + 77, 512
    k, _ = _keys(B, H, T, dk, dtype, seed=dk)
    print(f"[write_scores] B={B} H={H} T={T} dk={dk} {dtype}", flush=True)
    dh, dm = la.write_scores(k, chunk=C)
    torch.cuda.synchronize()
    odh, odm = oracle.write_scores(k, chunk=C)
    assert_abs(dh, odh, 1e-5, "d_head")
    assert_abs(dm, odm, 1e-5, "d_mean")


@pytest.mark.parametrize("C", [511, 777])
def test_write_scores_bf16_chunk_lengths(la, C):
    # bf16 keys: chunks of at most 512 tokens are scored from registers, longer ones by the
    # two-pass kernel; both against the oracle, with a partial last chunk
    k, _ = _keys(1, 2, 3 * C + 100, 128, torch.bfloat16, seed=C)
    dh, dm = la.write_scores(k, chunk=C)
    torch.cuda.synchronize()
    odh, odm = oracle.write_scores(k, chunk=C)
    assert_abs(dh, odh, 1e-5, f"d_head, chunk {C}")
    assert_abs(dm, odm, 1e-5, f"d_mean, chunk {C}")


def test_write_scores_edge_cases(la):
    # one partial chunk; a zero key (scores 1); identical keys (score 0); chunk of 1 token
    k = torch.zeros((1, 2, 37, 128), dtype=torch.bfloat16, device=DEV)
    k[0, 0] = torch.randn(128, device=DEV).to(torch.bfloat16)       # all identical
    k[0, 1] = torch.randn(37, 128, device=DEV).to(torch.bfloat16)
    k[0, 1, 5] = 0
    dh, dm = la.write_scores(k, chunk=512)
    torch.cuda.synchronize()
    odh, odm = oracle.write_scores(k, chunk=512)
    assert float(dh[0, 0].abs().max()) < 1e-6 and float(dh[0, 1, 5]) == 1.0
    assert_abs(dh, odh, 1e-5, "d_head")
    dh1, _ = la.write_scores(k, chunk=1)
    torch.cuda.synchronize()
    assert_abs(dh1, oracle.write_scores(k, chunk=1)[0], 1e-5, "d_head, chunk 1")


def _check_windows(gs, gv, d, C, W, tail):
    """GPU choice vs the oracle's window sums (fp64 of the same fp32 d_mean values)."""
    B, T = d.shape
    os_, ov = oracle.write_windows(d, C, W, tail)
    for b in range(B):
        for c in range(T // C):
            lo, hi = max(0, c * C - tail), (c + 1) * C
            w = min(W, hi - lo)
            sums = np.array([d[b, s:s + w].sum() for s in range(lo, hi - w + 1)])
            tol = 1e-5 * max(1.0, np.abs(sums).max())
            g = int(gs[b, c])
            assert lo <= g <= hi - w
            assert sums[g - lo] >= sums.max() - tol, (b, c, g, int(os_[b, c]))
            srt = np.sort(sums)
            if len(srt) < 2 or srt[-1] - srt[-2] > tol:
                assert g == os_[b, c]
            assert abs(float(gv[b, c]) - sums[g - lo]) <= tol


@pytest.mark.parametrize("C,W,tail", [(512, 48, 32), (100, 48, 0), (20, 48, 5), (64, 1, 64)])
def test_write_windows(la, C, W, tail):
    r = np.random.default_rng(C + W + tail)
    B, T = 3, 5 * C + C // 2
    d = r.uniform(0, 2, (B, T)).astype(np.float32)
    d[0, C + 7] = 9.0                    # a spike: every covering window ties but the earliest wins
    gs, gv = la.write_windows(torch.tensor(d, device=DEV), chunk=C, window=W, tail=tail)
    torch.cuda.synchronize()
    assert gs.shape == (B, T // C)
    _check_windows(gs.cpu().numpy(), gv.cpu().numpy(), d.astype(np.float64), C, W, tail)


def test_write_pipeline_on_keys(la):
    """Keys -> scores -> windows, each side on its own scores."""
    B, H, T = 1, 8, 512 * 6 + 100
    k, _ = _keys(B, H, T, 128, torch.bfloat16, seed=5)
    _, dm = la.write_scores(k)
    gs, gv = la.write_windows(dm)
    torch.cuda.synchronize()
    _, odm = oracle.write_scores(k)
    # the GPU's window, scored on the oracle's d_mean, is within the fp32 error of the best
    for c in range(T // 512):
        lo, hi = max(0, 512 * c - 32), 512 * (c + 1)
        sums = np.array([odm[0, s:s + 48].sum() for s in range(lo, hi - 47)])
        assert sums[int(gs[0, c]) - lo] >= sums.max() - 1e-3


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_note_addresses(la, dtype):
    r = np.random.default_rng(7)
    B, H, T, dk, N, drho = 2, 8, 900, 128, 37, 16
    _, q = _keys(B, H, T, dk, dtype, seed=9)
    k, _ = _keys(B, H, T, dk, torch.float32, seed=10)
    d32 = oracle.write_scores(k, chunk=300)[0].astype(np.float32)    # an oracle-made fp32 input
    d32[0, 2, 100:110] = 3.0                                            # a tie inside note 0's span
    spans = np.stack([np.stack([r.integers(0, T - 64, N), r.integers(1, 65, N)], -1) for _ in range(B)])
    spans[0, 0] = (95, 30)
    spans[1, 3] = (T - 1, 1)
    coords = np.stack([r.permutation(dk)[:drho] for _ in range(H)]).astype(np.int32)
    ts, rho = la.note_addresses(torch.tensor(d32, device=DEV), q, torch.tensor(spans, device=DEV),
                                torch.tensor(coords, device=DEV))
    torch.cuda.synchronize()
    ots, orho = oracle.note_addresses(d32.astype(np.float64), q, spans, coords)
    assert np.array_equal(ts.cpu().numpy(), ots)          # the same fp32 numbers decide
    assert int(ts[0, 0, 2]) == 100
    assert np.array_equal(to64(rho), orho)                # a gather: bit-exact


def test_note_addresses_invalid_span_and_coord(la):
    B, H, T, dk = 1, 2, 50, 64
    q = torch.randn(B, H, T, dk, device=DEV).to(torch.bfloat16)
    d = torch.rand(B, H, T, device=DEV)
    spans = torch.tensor([[[10, 5], [48, 5], [-1, 3], [0, 0]]], dtype=torch.int64, device=DEV)
    coords = torch.tensor([[0, 1, 2, 99], [3, 4, 5, 6]], dtype=torch.int32, device=DEV)
    ts, rho = la.note_addresses(d, q, spans, coords)
    torch.cuda.synchronize()
    assert ts[0, 1:].eq(-1).all() and rho[0, 1:].eq(0).all()
    assert int(ts[0, 0, 0]) == 10 + int(torch.argmax(d[0, 0, 10:15]))
    assert float(rho[0, 0, 0, 3]) == 0.0                  # out-of-range coordinate
    t0 = int(ts[0, 0, 1])
    assert torch.equal(rho[0, 0, 1], q[0, 1, t0, 3:7])


def _check_votes(gscore, gchoice, gvotes, gsel, rho, u, R, pos, tol=1e-5):
    osc, och, ovo, osel = oracle.address_votes(rho, u, R, pos)
    assert_abs(gscore, osc, tol, "score")
    J, N = osc.shape
    for j in range(J):
        g = int(gchoice[j])
        assert osc[j, g] >= osc[j].max() - tol
        srt = np.sort(osc[j])
        if srt[-1] - srt[-2] > 2 * tol:
            assert g == och[j]
    assert np.array_equal(gvotes, np.bincount(gchoice, minlength=N))
    # the selection rule applied to the GPU's votes
    order = sorted((i for i in range(N) if gvotes[i] > 0), key=lambda i: (-gvotes[i], i))[:R]
    order = sorted(order, key=lambda i: (pos[i], i))
    assert list(gsel) == order + [-1] * (R - len(order))
    if np.array_equal(gchoice, och):
        assert np.array_equal(gsel, osel)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("drho", [8, 16, 32])
def test_address_votes(la, dtype, drho):
    r = np.random.default_rng(drho)
    N, J, nQ, R = 600, 24, 40, 8
    rho = torch.tensor(r.standard_normal((N, J, drho)), dtype=dtype, device=DEV)
    u = torch.tensor(r.standard_normal((nQ, J, drho)), dtype=dtype, device=DEV)
    u[3, 5] = rho[77, 5] * 2                               # channel 5: an exact match with note 77
    pos = torch.tensor(r.permutation(N) * 10, dtype=torch.int64, device=DEV)
    sc, ch, vo, sel = la.address_votes(rho, u, R, pos)
    torch.cuda.synchronize()
    assert int(ch[5]) == 77
    _check_votes(sc.cpu().numpy(), ch.cpu().numpy(), vo.cpu().numpy(), sel.cpu().numpy(),
                 to64(rho), to64(u), R, pos.cpu().numpy())


def test_address_votes_pages_example(la):
    """The notes' example: channels vote A, B, A -> A two votes, B one; R = 2 returns both in
    document order (B first: it sits earlier in the text)."""
    e = torch.eye(16, device=DEV)
    rho = torch.stack([torch.stack([e[0], e[0], e[0]]), torch.stack([e[1], e[1], e[1]])]).to(torch.bfloat16)
    u = torch.stack([torch.stack([e[0], 3 * e[1], 0.5 * e[0]])]).to(torch.bfloat16)
    pos = torch.tensor([900, 100], dtype=torch.int64, device=DEV)
    _, ch, vo, sel = la.address_votes(rho, u, 2, pos)
    _, _, _, sel1 = la.address_votes(rho, u, 1, pos)
    _, _, _, sel4 = la.address_votes(rho, u, 4, pos)
    torch.cuda.synchronize()
    assert ch.tolist() == [0, 1, 0] and vo.tolist() == [2, 1]
    assert sel.tolist() == [1, 0] and sel1.tolist() == [0] and sel4.tolist() == [1, 0, -1, -1]


def test_write_scores_full_size_sampled_chunks(la):
    """The 1M-token, 16-head keys of the gated-delta prefill: every score of a sample of write
    chunks (chunks are independent, so the oracle scores just those) and the windows of the
    sampled chunks from the GPU's own d_mean."""
    B, H, T, D, C = 1, 16, 1 << 20, 128, 512
    k = synth.gdn_inputs(B, H, T, D, D, dtype=torch.bfloat16, seed=3, device=DEV)["k"]
    dh, dm = la.write_scores(k, chunk=C)
    torch.cuda.synchronize()
    for c in (0, 1, 777, T // C - 1):
        kc = k[:, :, c * C:(c + 1) * C]
        odh, odm = oracle.write_scores(kc, chunk=C)
        assert_abs(dh[:, :, c * C:(c + 1) * C], odh, 1e-5, f"d_head chunk {c}")
        assert_abs(dm[:, c * C:(c + 1) * C], odm, 1e-5, f"d_mean chunk {c}")


def test_address_votes_pages_archive_size(la):
    """Addressing at the pages' archive size: 4092 notes, 192 channels (24 layers x 8 heads),
    d_rho = 16, a 128-token question, R = 8."""
    r = np.random.default_rng(12)
    N, J, nQ, R = 4092, 192, 128, 8
    rho = torch.tensor(r.standard_normal((N, J, 16)), dtype=torch.bfloat16, device=DEV)
    u = torch.tensor(r.standard_normal((nQ, J, 16)), dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor(np.arange(N) * 256, dtype=torch.int64, device=DEV)
    sc, ch, vo, sel = la.address_votes(rho, u, R, pos)
    torch.cuda.synchronize()
    _check_votes(sc.cpu().numpy(), ch.cpu().numpy(), vo.cpu().numpy(), sel.cpu().numpy(),
                 to64(rho), to64(u), R, pos.cpu().numpy())
