"""Long sequences in segments (state passed forward, state gradient passed
backward) through the C ABI: the segmented results equal one call over the
whole sequence, and both match the oracle on a sampled head."""
import pytest
import torch

import linear_rnn_lm_amd as L
from linear_rnn_lm_amd.inputs import make_inputs
from linear_rnn_lm_amd.segments import bwd_segments, fwd_segments
from tests.gpu_util import compare, note, run_oracle, slice_heads

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
NAMES = ("dr", "dw", "dk", "dv", "da", "db", "dh0")


def _rel(x, ref):
    x, ref = x.double(), ref.double()
    return ((x - ref).norm() / ref.norm()).item()


def _run(x, dhT, seg):
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in (x.r, x.w, x.k, x.v, x.a, x.b)]
    h0, dy, dh = x.h0.to(dev), x.dy.to(dev), dhT.to(dev)
    if seg is None:
        y, ck, hT = L.fwd(*ins, h0)
        g = L.bwd(dy, *ins, ck, dh)
    else:
        y, cks, hT = fwd_segments(*ins, seg, h0)
        g = bwd_segments(dy, *ins, cks, seg, dh)
    torch.cuda.synchronize()
    out = {"y": y.cpu(), "hT": hT.cpu()}
    out.update({n: t.cpu() for n, t in zip(NAMES, g)})
    return out


@pytest.mark.parametrize("T,seg", [(65536, 4096), (16384 + 40, 1000)])
def test_segments_match_one_call(T, seg):
    """Segments of a multiple of 32 tokens give the chunks of one call (results
    equal up to the order of a few sums); other segment lengths move the chunk
    boundaries and agree within the fp32 tolerance."""
    x = make_inputs(1, T, 2, BF16, seed=600 + seg, with_h0=True)
    dhT = torch.randn(1, 2, 64, 64, generator=torch.Generator().manual_seed(601)) * 0.1
    note(f"long context T{T} seg{seg}: one call")
    full = _run(x, dhT, None)
    note(f"long context T{T} seg{seg}: segments")
    segd = _run(x, dhT, seg)
    tol = 1e-6 if seg % 32 == 0 else 1e-4
    errs = {n: _rel(segd[n], full[n]) for n in full}
    note(f"rel {errs}")
    assert all(e <= tol for e in errs.values()), errs


def test_segments_match_oracle_16k():
    """T = 16384 in four segments against the oracle on one head."""
    T, seg = 16384, 4096
    x = make_inputs(1, T, 2, BF16, seed=602, with_h0=True)
    dhT = torch.randn(1, 2, 64, 64, generator=torch.Generator().manual_seed(603)) * 0.1
    note(f"long context T{T} seg{seg} vs oracle")
    segd = _run(x, dhT, seg)
    xs = slice_heads(x, [0], [1])
    ref = run_oracle(xs, dhT[:, 1:2].contiguous())
    gpu = {n: (v[:, :, 1:2] if n not in ("hT", "dh0") else v[:, 1:2]) for n, v in segd.items()}
    errs, bad = compare(gpu, ref, BF16, names=["y", "hT", *NAMES])
    note(f"rel-L2 {errs}")
    assert not bad, errs
