"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case draws seeded inputs once on the CPU, runs both implementations on
the identical (rounded) values and compares every output, head by head, by
rel-L2.
"""
import numpy as np
import pytest
import torch

import linear_rnn_lm_amd as L
from linear_rnn_lm_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from tests.gpu_util import compare, note, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16

# (B, T, H, dtype, with_h0, with_dhT): several chunks, ragged tails, one token,
# head counts on every scan launch shape (on 256 CUs: workgroups of 16 state
# rows up to 64 heads, of 32 rows up to 128 heads, of 64 rows beyond).
SMALL = [
    (1, 64, 1, F32, False, False),
    (2, 1, 3, F32, True, True),
    (2, 2, 3, BF16, True, True),
    (2, 31, 3, F32, True, True),
    (2, 32, 3, BF16, True, True),
    (2, 33, 3, F32, True, True),
    (2, 95, 3, BF16, True, True),
    (3, 200, 5, BF16, True, True),
    (4, 130, 4, F32, True, False),
    # the scan launch boundaries on 256 CUs: 64 heads (four workgroups per head) and 65 (two)
    (4, 70, 16, BF16, True, True),
    (5, 70, 13, F32, True, True),
    (8, 40, 16, BF16, True, True),
    (16, 40, 16, BF16, False, True),
    (1, 257, 8, F32, True, True),
    # more chunks than CUs: the gradient kernel's workgroups take several
    # chunks each (uneven counts), on the XCD-grouped (40 heads) and the
    # plain (300 heads) block order
    (3, 300, 40, BF16, True, True),
    # more than 128 heads: one scan workgroup per head (64 state rows); fp32 token rows of 256
    # bytes, so the scans' up-front read of v and dy (token tensors up to 32 MiB) takes two lines
    # per row (the full-size B8 T4096 H32 case covers scans without that read)
    (1, 200, 300, F32, False, True),
]


@pytest.mark.parametrize("B,T,H,dtype,with_h0,with_dhT", SMALL,
                         ids=[f"B{c[0]}T{c[1]}H{c[2]}-{str(c[3])[6:]}" for c in SMALL])
def test_small_shapes(B, T, H, dtype, with_h0, with_dhT):
    x = make_inputs(B, T, H, dtype, seed=100 + B * 7 + T * 3 + H, with_h0=with_h0)
    dhT = torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(T)) if with_dhT else None
    note(f"small B{B} T{T} H{H} {dtype}")
    g = run_gpu(x, dhT)
    o = run_oracle(x, dhT)
    errs, bad = compare(g, o, dtype)
    note(f"rel-L2 {errs}")
    assert not bad, f"over tolerance: {bad}; errors {errs}"


def test_tiny_fp32_workload():
    wl = WORKLOADS["tiny_fp32"]
    x = workload_inputs(wl)
    note("workload tiny_fp32")
    errs, bad = compare(run_gpu(x), run_oracle(x), wl.dtype)
    note(f"rel-L2 {errs}")
    assert not bad, errs


@pytest.mark.parametrize("name", ["debug_36m", "rwkv_0b1"])
def test_training_workload_full(name):
    """Every output of the full-size workload against the oracle."""
    wl = WORKLOADS[name]
    x = workload_inputs(wl)
    note(f"workload {name} full")
    g = run_gpu(x)
    o = run_oracle(x)
    errs, bad = compare(g, o, wl.dtype)
    note(f"rel-L2 {errs}")
    assert not bad, errs


def test_rwkv_1b5_all_heads():
    """Full-size B8 T4096 H32 (h0 != 0): every output of all 256 heads against
    the oracle, head by head."""
    wl = WORKLOADS["rwkv_1b5"]
    x = workload_inputs(wl)
    note("workload rwkv_1b5 full")
    g = run_gpu(x)
    note("workload rwkv_1b5: oracle on all 256 heads")
    o = run_oracle(x)
    errs, bad = compare(g, o, wl.dtype)
    note(f"rel-L2 (worst head) {errs}")
    assert not bad, errs


@pytest.mark.parametrize("layer", [0, 13, 31])
def test_rwkv_7b_step_layer(layer):
    """One layer of the 7B recurrent step: T=1, B=256, H=64, state updated in
    place (hT is h0), compared on every head."""
    wl = WORKLOADS["rwkv_7b_step"]
    x = workload_inputs(wl, layer)
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in x.tensors()]
    state = x.h0.to(dev).clone()
    note(f"7b step layer {layer}")
    y = L.step(*ins, state)
    torch.cuda.synchronize()
    o = run_oracle(x, bwd=False)
    errs, bad = compare({"y": y.double().cpu().numpy(), "hT": state.double().cpu().numpy()}, o, wl.dtype,
                        names=["y", "hT"])
    note(f"rel-L2 {errs}")
    assert not bad, errs


@pytest.mark.parametrize("T", [1, 7, 33, 95])
def test_sequential_path_matches_oracle(T):
    x = make_inputs(2, T, 3, BF16, seed=900 + T, with_h0=True)
    note(f"sequential T{T}")
    g = run_gpu(x, sequential=True, bwd=False)
    o = run_oracle(x, bwd=False)
    errs, bad = compare(g, o, BF16)
    note(f"rel-L2 {errs}")
    assert not bad, errs


def test_split_sequence_state_passing():
    """fwd over T1 tokens, then T2 tokens from the handed-over state, equals
    one fwd over T1+T2 tokens."""
    x = make_inputs(2, 150, 3, F32, seed=77, with_h0=True)
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in x.tensors()]
    h0 = x.h0.to(dev)
    note("split sequence")
    y, _, hT = L.fwd(*ins, h0)
    T1 = 70
    y1, _, h1 = L.fwd(*[t[:, :T1].contiguous() for t in ins], h0)
    y2, _, h2 = L.fwd(*[t[:, T1:].contiguous() for t in ins], h1)
    torch.cuda.synchronize()
    cat = torch.cat([y1, y2], dim=1)
    assert (cat - y).norm() / y.norm() < 1e-5
    assert (h2 - hT).norm() / hT.norm() < 1e-5


@pytest.mark.parametrize("dtype,T", [(F32, 70), (BF16, 64), (BF16, 5)])
def test_chunk_inverse_matches_direct_solve(dtype, T):
    """(I - L)^-1 of every chunk against numpy's inverse of the same L built in
    float64 from the same (rounded) inputs."""
    x = make_inputs(2, T, 3, dtype, seed=300 + T)
    dev = torch.device("cuda:0")
    note(f"chunk inverse {dtype} T{T}")
    B, _, H, D = x.w.shape
    ops = L.chunk_prepare(*(t.to(dev) for t in (x.r, x.w, x.k, x.a, x.b)))
    inv = L.chunk_inverse(ops, B, T, H).double().cpu().numpy()
    w, a, b = (t.double().numpy() for t in (x.w, x.a, x.b))
    worst = 0.0
    for bb in range(B):
        for hh in range(H):
            for c in range(inv.shape[2]):
                sl = slice(32 * c, min(T, 32 * c + 32))
                n = sl.stop - sl.start
                W = np.ones((32, D)); A = np.zeros((32, D)); Bv = np.zeros((32, D))
                W[:n], A[:n], Bv[:n] = w[bb, sl, hh], a[bb, sl, hh], b[bb, sl, hh]
                g = np.cumprod(W, axis=0)
                gp = np.vstack([np.ones((1, D)), g[:-1]])
                Lm = np.tril((A * gp) @ (Bv / g).T, -1)
                ref = np.linalg.inv(np.eye(32) - Lm)
                worst = max(worst, np.linalg.norm(inv[bb, hh, c] - ref) / np.linalg.norm(ref))
    assert worst < (1e-6 if dtype == F32 else 2e-5), worst
