"""wkv7_fwd_noalloc, the forward whose chunk operands live in the library's
static device scratch (for callers that cannot allocate), through the C ABI
against wkv7_fwd with a caller-supplied workspace on the same inputs: two
calls in a row, the second smaller (so it runs over what the first left in
the scratch), each bitwise equal; the one-token path; and the host-side
refusal of a call whose operands would not fit the scratch."""
import pytest
import torch

import linear_rnn_lm_amd as L
from linear_rnn_lm_amd.inputs import make_inputs
from tests.gpu_util import note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
WKV7_ERR_WORKSPACE = 7


def _fwd_pair(B, T, H, dtype, seed):
    lib = L.lib()
    x = make_inputs(B, T, H, dtype, seed=seed, with_h0=True)
    ins = [t.to(DEV) for t in x.tensors()]
    h0 = x.h0.to(DEV)
    p = [t.data_ptr() for t in ins]
    code = 1 if dtype == torch.bfloat16 else 0
    s = torch.cuda.current_stream().cuda_stream
    nc = L.num_chunks(T)
    outs = []
    for noalloc in (False, True):
        y = torch.full((B, T, H, 64), float("nan"), device=DEV)
        ck = torch.full((B, H, nc, 64, 64), float("nan"), device=DEV)
        hT = torch.full((B, H, 64, 64), float("nan"), device=DEV)
        if noalloc:
            note(f"noalloc fwd B{B} T{T} H{H} {dtype}")
            st = lib.wkv7_fwd_noalloc(B, T, H, 64, code, *p, h0.data_ptr(), y.data_ptr(), ck.data_ptr(),
                                      hT.data_ptr(), s)
        else:
            wsb = L.fwd_workspace_bytes(B, T, H)
            ws = torch.empty(max(wsb, 16) // 4, device=DEV)
            note(f"fwd with workspace B{B} T{T} H{H} {dtype}")
            st = lib.wkv7_fwd(B, T, H, 64, code, *p, h0.data_ptr(), y.data_ptr(), ck.data_ptr(), hT.data_ptr(),
                              ws.data_ptr(), wsb, s)
        assert st == 0, lib.wkv7_status_str(st)
        outs.append((y, ck, hT))
    torch.cuda.synchronize()
    return outs


def test_noalloc_matches_fwd_two_calls_in_a_row():
    # the training-shape layer (94 MB of chunk operands, within the 128 MiB scratch),
    # then a smaller, ragged fp32 call over what it left behind
    for B, T, H, dtype, seed in ((12, 1024, 6, torch.bfloat16, 31), (2, 75, 3, torch.float32, 32)):
        (y, ck, hT), (y2, ck2, hT2) = _fwd_pair(B, T, H, dtype, seed)
        assert torch.isfinite(y2).all() and torch.isfinite(ck2).all() and torch.isfinite(hT2).all()
        assert torch.equal(y, y2) and torch.equal(ck, ck2) and torch.equal(hT, hT2)


def test_noalloc_one_token_and_refusal():
    (y, ck, hT), (y2, ck2, hT2) = _fwd_pair(4, 1, 5, torch.bfloat16, 33)
    assert torch.equal(y, y2) and torch.equal(ck, ck2) and torch.equal(hT, hT2)
    # 16 x 8 heads x 32 chunks = 4096 chunks of operands: more than the scratch holds
    lib = L.lib()
    B, T, H = 16, 1024, 8
    assert L.fwd_workspace_bytes(B, T, H) > lib.wkv7_fwd_noalloc_max_bytes()
    ins = [torch.zeros(B, T, H, 64, device=DEV, dtype=torch.bfloat16) for _ in range(6)]
    y = torch.empty(B, T, H, 64, device=DEV)
    note("noalloc refusal B16 T1024 H8")
    st = lib.wkv7_fwd_noalloc(B, T, H, 64, 1, *[t.data_ptr() for t in ins], None, y.data_ptr(), None, None,
                              torch.cuda.current_stream().cuda_stream)
    assert st == WKV7_ERR_WORKSPACE
