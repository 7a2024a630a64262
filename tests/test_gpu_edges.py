"""The recurrence at the edges of its domain, through the C ABI, against the
oracle on identical inputs (every output, head by head), plus the exact
zeros that the definition forces:

* w = 1/8 everywhere, the smallest decay the library accepts (a chunk's
  running decay products reach 2^-96 and their reciprocals 2^96);
* w in [0.999, 1] over 4096 tokens with h0 and dhT (the state barely decays;
  the RWKV-LM README page's reason for an fp32 state);
* w = 1, a = b = 0: the state is the running sum of v k^T (causal linear
  attention), so sa = 0 and dsa = 0, hence da = db = 0 exactly;
* a = 0: sa = 0 for every token, hence db = 0 exactly;
* the delta rule (w = 1, r = k = kh, a = -kh, b = kh, kh a unit vector):
  every token writes v along kh and reads it back, so y = v.

Forward and update: rwkv-mlx page, "Metal kernel architecture", forward
block; gradients: its backward block."""
import numpy as np
import pytest
import torch

from linear_rnn_lm_amd.inputs import make_edge_inputs
from tests.gpu_util import compare, note, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16

# (kind, B, T, H, dtype): several chunks and a ragged tail in every case
CASES = [
    ("w_eighth", 2, 96, 3, F32),
    ("w_eighth", 2, 100, 3, BF16),
    ("w_near_one", 2, 4096, 2, F32),
    ("w_near_one", 1, 4096 + 17, 3, BF16),
    ("linear_attn", 2, 100, 3, F32),
    ("linear_attn", 2, 77, 2, BF16),
    ("a_zero", 2, 90, 3, F32),
    ("a_zero", 3, 70, 2, BF16),
    ("delta_rule", 2, 80, 3, F32),
    ("delta_rule", 2, 64, 2, BF16),
]


def _run(kind, B, T, H, dtype, seed):
    x = make_edge_inputs(kind, B, T, H, dtype, seed=seed, with_h0=True)
    dhT = torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(seed + 7)) * 0.1
    note(f"edge {kind} B{B} T{T} H{H} {dtype}")
    g = run_gpu(x, dhT)
    o = run_oracle(x, dhT)
    return x, g, o


@pytest.mark.parametrize("kind,B,T,H,dtype", CASES,
                         ids=[f"{c[0]}-B{c[1]}T{c[2]}H{c[3]}-{str(c[4])[6:]}" for c in CASES])
def test_edge_matches_oracle(kind, B, T, H, dtype):
    x, g, o = _run(kind, B, T, H, dtype, seed=1000 + T + H)
    errs, bad = compare(g, o, dtype)
    note(f"rel-L2 (worst head) {errs}")
    assert not bad, errs
    for n, v in g.items():
        assert np.isfinite(v).all(), n
    if kind == "linear_attn":
        assert np.all(g["da"] == 0.0) and np.all(g["db"] == 0.0)
        assert np.all(o["da"] == 0.0) and np.all(o["db"] == 0.0)
    if kind == "a_zero":
        assert np.all(g["db"] == 0.0) and np.all(o["db"] == 0.0)
        assert np.abs(g["da"]).max() > 0          # da itself is not forced to zero
    if kind == "delta_rule" and dtype == F32:
        # y_t = S_t kh_t = v_t up to the rounding of |kh| = 1
        v = x.v.double().numpy()
        assert np.linalg.norm(g["y"] - v) / np.linalg.norm(v) < 1e-5
