"""GPU parity of la_state_scale, the state handling around a NoteBank replay ("History
Replays Itself", App. B Algorithm 1: each branch starts from a copy of the retained state;
App. C.3: S <- lambda S at the readout boundary, lambda = 0 resetting it).  The products
are single fp32 multiplications, so the result must equal the fp64 oracle rounded to fp32
bit for bit."""

import numpy as np
import pytest
import torch

import gated_delta_rule_chunkwise_amd as la_mod
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _expect(S, lam):
    return torch.from_numpy(oracle.state_scale(S, lam).astype(np.float32))


@pytest.mark.parametrize("lam", [0.0, 0.37, 1.0])
@pytest.mark.parametrize("shape", [(8, 256, 256), (3, 128, 127), (5,)])
def test_state_scale_bit_exact(la, lam, shape):
    lam = float(np.float32(lam))  # the ABI takes lambda as fp32: both sides use that value
    S = synth.gdn_state(shape, seed=11, device=DEV)
    out = la.state_scale(S, lam)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), _expect(S, lam))


def test_state_scale_in_place_and_reset(la):
    S = synth.gdn_state((2, 256, 256), seed=12, device=DEV)
    ref = _expect(S, 0.5)
    la.state_scale(S, 0.5, out=S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), ref)
    S[0, 0, :3] = torch.tensor([float("inf"), float("nan"), -float("inf")], device=DEV)
    la.state_scale(S, 0.0, out=S)  # the reset clears non-finite values too
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_branch_copy_leaves_retained_state(la):
    """A read branch: copy the retained state (lambda = 1), continue the copy with a replay,
    and the retained state is untouched; the branch equals a prefill from the state itself."""
    d = synth.gdn_inputs(1, 2, 300, 256, 256, dtype=torch.bfloat16, seed=13, device=DEV)
    _, S, _ = la.prefill("gated_delta", d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    keep = S.clone()
    Sr = la.state_scale(S, 1.0)
    r = synth.gdn_inputs(1, 2, 70, 256, 256, dtype=torch.bfloat16, seed=14, device=DEV)
    o1, S1, _ = la.prefill("gated_delta", r["q"], r["k"], r["v"], r["alpha"], r["beta"], S0=Sr, S_T=Sr)
    o2, S2, _ = la.prefill("gated_delta", r["q"], r["k"], r["v"], r["alpha"], r["beta"], S0=S)
    torch.cuda.synchronize()
    assert torch.equal(S, keep)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_state_scale_reset_without_input_through_abi(la):
    """lambda = 0 with a NULL S_in through the C ABI: the reset reads nothing and writes zeros."""
    import ctypes
    S = torch.full((1000,), 7.0, device=DEV)
    st = la.load().la_state_scale(S.numel(), ctypes.c_float(0.0), None, ctypes.c_void_p(S.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and torch.count_nonzero(S) == 0

