"""Output hygiene of the HIP path: every output element is written, results
repeat bit for bit, the in-place state update equals the out-of-place one, the
autograd op matches the raw calls, and bad arguments on real device buffers
are rejected before launch."""
import pytest
import torch

import linear_rnn_lm_amd as L
from linear_rnn_lm_amd.inputs import make_inputs
from tests.gpu_util import note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(B=2, T=75, H=3, dtype=torch.bfloat16, seed=5):
    x = make_inputs(B, T, H, dtype, seed=seed, with_h0=True)
    return [t.to(DEV) for t in x.tensors()], x.h0.to(DEV), x.dy.to(DEV)


def test_nan_prefilled_outputs_are_overwritten():
    ins, h0, dy = _inputs()
    B, T, H, D = ins[0].shape
    nan = lambda *s: torch.full(s, float("nan"), device=DEV)
    y, ck, hT = nan(B, T, H, D), nan(B, H, L.num_chunks(T), D, D), nan(B, H, D, D)
    note("nan prefill fwd")
    L.fwd(*ins, h0, y=y, ckpt=ck, hT=hT)
    out = [nan(B, T, H, D) for _ in range(6)]
    ws = nan(L.workspace_bytes(B, T, H) // 4)
    note("nan prefill bwd")
    g = L.bwd(dy, *ins, ck, None, out=out, workspace=ws)
    torch.cuda.synchronize()
    for t in (y, ck, hT, *g):
        assert torch.isfinite(t).all()


def test_results_repeat_bitwise():
    ins, h0, dy = _inputs(seed=6)
    note("repeatability")
    runs = []
    for _ in range(2):
        y, ck, hT = L.fwd(*ins, h0)
        g = L.bwd(dy, *ins, ck, hT * 0.5)
        runs.append([y, ck, hT, *g])
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_in_place_state_update():
    ins, h0, _ = _inputs(T=1, seed=7)
    note("in-place step")
    y_ref, _, hT_ref = L.fwd(*ins, h0, want_ckpt=False)
    state = h0.clone()
    y = L.step(*ins, state)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(state, hT_ref)
    ins, h0, _ = _inputs(T=40, seed=8)
    y_ref, _, hT_ref = L.fwd(*ins, h0, want_ckpt=False)
    state = h0.clone()
    L.fwd(*ins, state, want_ckpt=False, hT=state)
    torch.cuda.synchronize()
    assert torch.equal(state, hT_ref)


def test_autograd_op_matches_raw_calls():
    ins, h0, dy = _inputs(dtype=torch.float32, seed=9)
    dhT = torch.randn(h0.shape, device=DEV)
    leaves = [t.clone().requires_grad_(True) for t in ins] + [h0.clone().requires_grad_(True)]
    note("autograd op")
    y, hT = L.WKV7.apply(*leaves)
    ((y * dy).sum() + (hT * dhT).sum()).backward()
    _, ck, _ = L.fwd(*ins, h0)
    g = L.bwd(dy, *ins, ck, dhT)
    torch.cuda.synchronize()
    for leaf, ref in zip(leaves, g):
        assert torch.allclose(leaf.grad, ref, rtol=0, atol=0)


def test_device_buffers_rejected_before_launch():
    ins, h0, dy = _inputs(seed=10)
    B, T, H, D = ins[0].shape
    lib = L.lib()
    y = torch.empty(B, T, H, D, device=DEV)
    ck = torch.empty(B, H, L.num_chunks(T), D, D, device=DEV)
    p = [t.data_ptr() for t in ins]
    s = torch.cuda.current_stream().cuda_stream
    wsb = L.fwd_workspace_bytes(B, T, H)
    fws = torch.empty(wsb // 4, device=DEV)
    w_ = (fws.data_ptr(), wsb)
    # y aliasing r, hT inside the checkpoints, misaligned y, workspace too small
    assert lib.wkv7_fwd(B, T, H, D, 1, *p, None, p[0], ck.data_ptr(), None, *w_, s) == 5
    assert lib.wkv7_fwd(B, T, H, D, 1, *p, None, y.data_ptr(), ck.data_ptr(), ck.data_ptr() + 64, *w_, s) == 5
    assert lib.wkv7_fwd(B, T, H, D, 1, *p, None, y.data_ptr() + 4, ck.data_ptr(), None, *w_, s) == 4
    assert lib.wkv7_fwd(B, T, H, D, 1, *p, None, y.data_ptr(), ck.data_ptr(), None, fws.data_ptr(), wsb - 4,
                        s) == 7
    ws = torch.empty(16, device=DEV)
    with pytest.raises(ValueError, match="workspace"):
        L.bwd(dy, *ins, ck, None, workspace=ws)
    # the library's own check, reached through the C ABI with the same buffer
    out = [torch.empty(B, T, H, D, device=DEV) for _ in range(6)]
    assert lib.wkv7_bwd(B, T, H, D, 1, dy.data_ptr(), None, *p, ck.data_ptr(), *[o.data_ptr() for o in out], None,
                        ws.data_ptr(), 64, s) == 7


def test_autograd_op_without_kept_operands():
    """keep_ops=False (the forward keeps only the checkpoints; the backward prepares
    the chunk operands again) gives the same outputs and gradients, bit for bit."""
    ins, h0, dy = _inputs(T=100, seed=11)
    dhT = torch.randn(h0.shape, device=DEV)
    res = []
    for keep in (True, False):
        leaves = [t.clone().requires_grad_(True) for t in ins] + [h0.clone().requires_grad_(True)]
        note(f"autograd op keep_ops={keep}")
        y, hT = L.WKV7.apply(*leaves, keep)
        ((y * dy).sum() + (hT * dhT).sum()).backward()
        res.append([y.detach(), hT.detach()] + [leaf.grad for leaf in leaves])
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)
