"""Host-side validation in the Python binding (CPU only): every tensor is
checked for shape, dtype, device and layout before a pointer reaches the
library, and a well-formed call on CPU tensors is refused at the end because
the library works on GPU memory only.  No library compute call is made."""
import pytest
import torch

import linear_rnn_lm_amd as L

BF, F32 = torch.bfloat16, torch.float32


def toks(B=2, T=40, H=3, dtype=BF):
    g = torch.Generator().manual_seed(0)
    return [torch.randn(B, T, H, 64, generator=g).to(dtype) for _ in range(6)]


def test_well_formed_cpu_call_is_refused_as_not_on_gpu():
    with pytest.raises(ValueError, match="GPU tensors"):
        L.fwd(*toks())
    with pytest.raises(ValueError, match="GPU tensors"):
        L.fwd_sequential(*toks())


@pytest.mark.parametrize("fn", [L.fwd, L.fwd_sequential, L.fwd_proj])
def test_token_inputs_must_agree(fn):
    x = toks()
    bad = list(x)
    bad[1] = x[1][:, :20].contiguous()                     # w shorter than r
    with pytest.raises(ValueError, match="shape and dtype"):
        fn(*bad)
    bad = list(x)
    bad[4] = x[4].float()                                  # a fp32, r bf16
    with pytest.raises(ValueError, match="shape and dtype"):
        fn(*bad)
    bad = list(x)
    bad[3] = x[3].transpose(1, 2).contiguous().transpose(1, 2)   # right shape, wrong strides
    with pytest.raises(ValueError, match="contiguous"):
        fn(*bad)
    with pytest.raises(TypeError, match="float32 or bfloat16"):
        fn(*[t.half() for t in x])
    with pytest.raises(ValueError, match=r"\(B, T, H, 64\)"):
        fn(*[t[..., :32].contiguous() for t in x])


def test_state_tensors_are_checked():
    x = toks()
    B, T, H = 2, 40, 3
    with pytest.raises(ValueError, match="h0"):
        L.fwd(*x, torch.zeros(B, H, 64, 64, dtype=BF))     # bf16 initial state
    with pytest.raises(ValueError, match="h0"):
        L.fwd(*x, torch.zeros(B, H + 1, 64, 64))
    with pytest.raises(ValueError, match="ckpt"):
        L.fwd(*x, ckpt=torch.empty(B, H, 1, 64, 64))       # too few chunks (T = 40 has 2)
    with pytest.raises(ValueError, match="y"):
        L.fwd(*x, y=torch.empty(B, T, H, 64, dtype=BF))
    one = toks(T=1)
    with pytest.raises(ValueError, match="state"):
        L.step(*one, torch.zeros(B, H, 64, 64, dtype=BF))  # bf16 state: half the bytes the step writes
    with pytest.raises(ValueError, match="state"):
        L.step(*one, torch.zeros(B, H, 64, 64).transpose(2, 3))


def test_backward_tensors_are_checked():
    x = toks()
    B, T, H = 2, 40, 3
    dy = torch.randn(B, T, H, 64)
    ck = torch.empty(B, H, 2, 64, 64)
    with pytest.raises(ValueError, match="dy"):
        L.bwd(dy.to(BF), *x, ck)
    with pytest.raises(ValueError, match="ckpt"):
        L.bwd(dy, *x, ck[:, :, :1].contiguous())
    with pytest.raises(ValueError, match="ckpt"):
        L.bwd(dy, *x, None)
    with pytest.raises(ValueError, match="dhT"):
        L.bwd(dy, *x, ck, torch.zeros(B, H, 64, 32))
    with pytest.raises(ValueError, match="workspace"):
        L.bwd(dy, *x, ck, workspace=torch.empty(16))
    with pytest.raises(ValueError, match="out"):
        L.bwd(dy, *x, ck, out=[torch.empty(B, T, H, 64)] * 5)
    with pytest.raises(ValueError, match="GPU tensors"):
        L.bwd(dy, *x, ck)


def test_staged_calls_are_checked():
    x = toks()
    B, T, H = 2, 40, 3
    r, w, k, v, a, b = x
    with pytest.raises(ValueError, match="out"):
        L.chunk_prepare(r, w, k, a, b, out=torch.empty(100))
    ops = torch.empty(L.chunk_ops_bytes(B, T, H) // 4)
    with pytest.raises(ValueError, match="chunk_ops"):
        L.fwd_scan(v, ops[:100])
    dy = torch.randn(B, T, H, 64)
    with pytest.raises(TypeError, match="in_dtype"):
        L.bwd_scan(dy, ops, in_dtype=torch.float16)
    with pytest.raises(TypeError, match="dy must be float32"):
        L.bwd_scan(dy.to(BF), ops, in_dtype=BF)
    with pytest.raises(ValueError, match="dh_ckpt"):
        L.bwd_scan(dy, ops, in_dtype=BF, dh_ckpt=torch.empty(B, H, 1, 64, 64))
    ck = torch.empty(B, H, 2, 64, 64)
    with pytest.raises(ValueError, match="dh_ckpt"):
        L.bwd_inputs(dy, *x, ops, ck, ck[:, :1].contiguous())
    with pytest.raises(ValueError, match="hT"):
        L.bwd_division(dy, *x, ck, torch.empty(B, H, 64, 64, dtype=BF))
