"""The layer with its time-mix prologue (w, a, b formed inside the kernels
from w_raw, kappa, alpha) through the C ABI, against the oracle's prologue
followed by its recurrence, and the recurrence's backward followed by the
prologue's backward."""
import numpy as np
import pytest
import torch

import linear_rnn_lm_amd as L
import oracle
from linear_rnn_lm_amd.inputs import ProjInputs, make_proj_inputs
from tests.gpu_util import TOL, note, rel_heads

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16
FWD = ("y", "ckpt", "hT")
BWD = ("dr", "dw_raw", "dk", "dv", "dkappa", "dalpha", "dh0")


def _np(t):
    return None if t is None else t.detach().double().cpu().numpy()


def run_gpu_proj(x, dhT=None):
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in x.tensors()]
    h0 = None if x.h0 is None else x.h0.to(dev)
    y, ck, hT = L.fwd_proj(*ins, h0)
    g = L.bwd_proj(x.dy.to(dev), *ins, ck, None if dhT is None else dhT.to(dev))
    torch.cuda.synchronize()
    out = {"y": y, "ckpt": ck, "hT": hT}
    out.update(dict(zip(BWD, g)))
    return {k: _np(v) for k, v in out.items()}


def run_oracle_proj(x, dhT=None):
    r, w_raw, k, v, kappa, alpha = x.tensors()
    w, a, b = oracle.proj_fwd(w_raw, kappa, alpha)
    y, ck, hT = oracle.fwd(r, w, k, v, a, b, x.h0)
    dr, dw, dk, dv, da, db, dh0 = oracle.bwd(r, w, k, v, a, b, x.dy, x.h0, dhT)
    dw_raw, dkappa, dalpha = oracle.proj_bwd(w_raw, kappa, alpha, dw, da, db)
    return {"y": y, "ckpt": ck, "hT": hT, "dr": dr, "dw_raw": dw_raw, "dk": dk, "dv": dv,
            "dkappa": dkappa, "dalpha": dalpha, "dh0": dh0}


def check(gpu, ref, dtype, names=FWD + BWD):
    """Every output, every (b, h) head within tolerance (worst head reported)."""
    errs = {n: rel_heads(n, gpu[n], ref[n]) for n in names}
    bad = [n for n in names if not errs[n] <= TOL[dtype]["fwd" if n in FWD else "bwd"]]
    note(f"rel-L2 {errs}")
    assert not bad, (bad, errs)


SMALL = [
    (1, 64, 1, F32, False, False),
    (2, 1, 3, F32, True, True),
    (3, 1, 5, BF16, True, True),
    (1, 31, 2, BF16, True, True),
    (2, 70, 3, F32, True, True),
    (3, 33, 1, F32, False, False),
    (1, 5, 2, BF16, True, False),
    (2, 100, 2, BF16, False, True),
]


@pytest.mark.parametrize("B,T,H,dtype,with_h0,with_dhT", SMALL,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}-{str(c[3])[6:]}-h0{int(c[4])}-dhT{int(c[5])}" for c in SMALL])
def test_proj_small_shapes(B, T, H, dtype, with_h0, with_dhT):
    x = make_proj_inputs(B, T, H, dtype, seed=700 + T, with_h0=with_h0)
    dhT = torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(701)) * 0.1 if with_dhT else None
    note(f"proj B{B} T{T} H{H} {dtype} h0={with_h0} dhT={with_dhT}")
    check(run_gpu_proj(x, dhT), run_oracle_proj(x, dhT), dtype)


def test_proj_zero_kappa_tokens():
    """Tokens whose kappa is zero get a = b = 0 and a zero kappa gradient; the
    rest of the sequence is unaffected."""
    x = make_proj_inputs(2, 45, 2, F32, seed=702, with_h0=True)
    kappa = x.kappa.clone()
    kappa[0, 3] = 0.0
    kappa[1, 40, 1] = 0.0
    x = ProjInputs(x.r, x.w_raw, x.k, x.v, kappa, x.alpha, x.h0, x.dy)
    note("proj zero kappa tokens")
    gpu, ref = run_gpu_proj(x), run_oracle_proj(x)
    assert np.all(gpu["dkappa"][0, 3] == 0.0) and np.all(gpu["dkappa"][1, 40, 1] == 0.0)
    check(gpu, ref, F32)


def test_proj_debug_shape_all_heads():
    """B12 T1024 H6 bf16 (the training-shape layer) in one call, every output
    of all 72 heads against the oracle's prologue and recurrence, head by head."""
    B, T, H = 12, 1024, 6
    x = make_proj_inputs(B, T, H, BF16, seed=703)
    note("proj B12 T1024 H6 bf16, all heads")
    check(run_gpu_proj(x), run_oracle_proj(x), BF16)


def test_proj_autograd_op_matches_raw_calls():
    """The autograd op over the prologue path gives the raw calls' gradients, bitwise."""
    dev = torch.device("cuda:0")
    x = make_proj_inputs(2, 70, 3, F32, seed=704, with_h0=True)
    ins = [t.to(dev) for t in x.tensors()]
    h0, dy = x.h0.to(dev), x.dy.to(dev)
    dhT = (torch.randn(2, 3, 64, 64, generator=torch.Generator().manual_seed(705)) * 0.1).to(dev)
    leaves = [t.clone().requires_grad_(True) for t in ins] + [h0.clone().requires_grad_(True)]
    note("proj autograd op")
    y, hT = L.WKV7Proj.apply(*leaves)
    ((y * dy).sum() + (hT * dhT).sum()).backward()
    _, ck, _ = L.fwd_proj(*ins, h0)
    g = L.bwd_proj(dy, *ins, ck, dhT)
    torch.cuda.synchronize()
    for leaf, ref in zip(leaves, g):
        assert torch.equal(leaf.grad, ref)


def test_proj_recurrent_step_7b_layer():
    """The one-token step with the prologue in its loads (B256 H64, one layer of the 7B
    step shape, state in place): y and the new state against the oracle on every head."""
    dev = torch.device("cuda:0")
    x = make_proj_inputs(256, 1, 64, BF16, seed=706, with_h0=True)
    ins = [t.to(dev) for t in x.tensors()]
    state = x.h0.to(dev).clone()
    note("proj step B256 T1 H64 bf16, in place")
    y, _, _ = L.fwd_proj(*ins, state, want_ckpt=False, hT=state)
    torch.cuda.synchronize()
    r, w_raw, k, v, kappa, alpha = x.tensors()
    w, a, b = oracle.proj_fwd(w_raw, kappa, alpha)
    yo, _, hTo = oracle.fwd(r, w, k, v, a, b, x.h0, want_ckpt=False)
    errs = {"y": rel_heads("y", _np(y), yo), "hT": rel_heads("hT", _np(state), hTo)}
    note(f"rel-L2 {errs}")
    assert max(errs.values()) <= TOL[BF16]["fwd"], errs
