"""The division-walk backward (the rwkv-mlx page's design, kept as a
diagnostic) through the C ABI: where undoing the update is well conditioned
it gives the oracle's gradients; at the workloads' decays its error grows
with the number of tokens walked between exact states, as the page says,
while the recompute backward stays at rounding level."""
import numpy as np
import pytest
import torch

import linear_rnn_lm_amd as L
import oracle
from linear_rnn_lm_amd.inputs import Inputs, make_inputs
from tests.gpu_util import TOL, note, rel

pytestmark = pytest.mark.gpu

NAMES = ("dr", "dw", "dk", "dv", "da", "db", "dh0")
F32 = torch.float32


def _gpu(x, dhT, restart):
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in x.tensors()]
    h0 = None if x.h0 is None else x.h0.to(dev)
    dy = x.dy.to(dev)
    dh = None if dhT is None else dhT.to(dev)
    y, ck, hT = L.fwd(*ins, h0)
    div = L.bwd_division(dy, *ins, ck, hT, dh, restart=restart)
    rec = L.bwd(dy, *ins, ck, dh)
    torch.cuda.synchronize()
    to = lambda g: {n: t.double().cpu().numpy() for n, t in zip(NAMES, g)}
    return to(div), to(rec)


def _oracle(x, dhT):
    return dict(zip(NAMES, oracle.bwd(*x.tensors(), x.dy, x.h0, dhT)))


def _worst(g, ref):
    errs = {n: (rel(g[n], ref[n]) if np.all(np.isfinite(g[n])) else float("inf")) for n in NAMES}
    return max(errs.values()), errs


def _well_conditioned(B, T, H, seed):
    """Decays in [0.97, 1] and small gates: each undone step is close to the identity."""
    g = torch.Generator().manual_seed(seed)
    sh = (B, T, H, 64)
    n = lambda *s: torch.randn(*s, generator=g)
    r, k, v = n(*sh), n(*sh) / 8, n(*sh)
    w = 0.97 + 0.03 * torch.rand(*sh, generator=g)
    kap = n(*sh)
    kap = kap / kap.norm(dim=-1, keepdim=True)
    b = kap * 0.3 * torch.rand(*sh, generator=g)
    return Inputs(r, w, k, v, -kap, b, n(B, H, 64, 64) * 0.1, n(*sh))


@pytest.mark.parametrize("restart", [True, False], ids=["restart-every-chunk", "one-walk"])
def test_division_walk_matches_oracle_when_well_conditioned(restart):
    x = _well_conditioned(2, 100, 2, seed=800)
    dhT = torch.randn(2, 2, 64, 64, generator=torch.Generator().manual_seed(801)) * 0.1
    note(f"division walk, well conditioned, restart={restart}")
    div, _ = _gpu(x, dhT, restart)
    worst, errs = _worst(div, _oracle(x, dhT))
    note(f"rel-L2 {errs}")
    assert worst <= TOL[F32]["bwd"], errs


def test_division_error_grows_with_the_walk_at_workload_decay():
    """Workload distributions (w in (0.545, 1)), T = 512, fp32: restarting from
    the exact state at every chunk end bounds the walk to 32 divisions; one walk
    over all 512 tokens loses the gradients entirely.  The recompute backward
    on the same inputs stays within the fp32 tolerance."""
    x = make_inputs(1, 512, 2, F32, seed=802, with_h0=True)
    ref = _oracle(x, None)
    note("division walk at workload decay, restart every chunk")
    div32, rec = _gpu(x, None, True)
    note("division walk at workload decay, one walk")
    div512, _ = _gpu(x, None, False)
    e32, errs32 = _worst(div32, ref)
    e512, errs512 = _worst(div512, ref)
    erec, _ = _worst(rec, ref)
    note(f"worst rel-L2: recompute {erec:.2e}, division restarted every 32 tokens {e32:.2e}, "
         f"one walk of 512 tokens {e512:.2e}")
    note(f"restart every chunk {errs32}")
    note(f"one walk {errs512}")
    assert erec <= TOL[F32]["bwd"]
    assert e32 > 10 * erec                # even 32 divisions in a row cost accuracy
    assert not (e512 <= 1e3 * e32)        # 512 in a row: orders of magnitude worse, or not finite
