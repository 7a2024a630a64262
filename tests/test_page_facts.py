"""The workloads and readings against numbers printed on the pages (CPU only)."""
import json
import math
import os

import numpy as np

from linear_rnn_lm_amd.inputs import WORKLOADS

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_workload_shapes_follow_the_pages():
    dbg = GOLDEN["debug_training_shape"]
    wl = WORKLOADS["debug_36m"]
    assert (wl.B, wl.T, wl.H) == (dbg["batch"], dbg["ctx"], dbg["heads"])
    hd = dbg["head_dim"]
    widths = GOLDEN["model_widths"]
    assert WORKLOADS["rwkv_0b1"].H * hd == widths["rwkv_0b1"]["n_embd"]
    assert WORKLOADS["rwkv_1b5"].H * hd == widths["rwkv_1b5"]["n_embd"]
    st = GOLDEN["rwkv7_7b_state"]
    step = WORKLOADS["rwkv_7b_step"]
    assert step.layers == st["layers"] and step.H == st["heads_per_layer"]
    assert st["layers"] * st["heads_per_layer"] * st["state_rows"] * st["state_cols"] == st["state_floats"]
    assert st["heads_per_layer"] * hd == widths["rwkv_7b"]["n_embd"]


def test_division_amplification_reading():
    """The page's two amplification figures are one decay raised to two powers:
    the w that gives the factor at 32 tokens gives the stated order at 512."""
    g = GOLDEN["division_amplification"]
    w = g["factor_at_32"] ** (-1.0 / GOLDEN["checkpoint_interval"]["tokens"])
    assert 0.85 < w < 0.95
    assert abs(math.log10(w ** -512) - g["order_of_magnitude_at_512"]) < 1.0


def test_division_reconstruction_is_unusable_at_workload_decay():
    """Negative control for the recompute design: undoing the update by dividing
    by w (fp32) loses the state within a few chunks at the workload's decay."""
    import oracle
    from linear_rnn_lm_amd.inputs import make_inputs
    import torch
    x = make_inputs(1, 128, 1, torch.float32, seed=5, with_h0=True)
    r, w, k, v, a, b = (t.double().numpy()[0, :, 0] for t in x.tensors())
    y, ck, hT = oracle.fwd(*x.tensors(), x.h0)
    S = hT[0, 0].astype(np.float32)
    T = r.shape[0]
    err_at = {}
    for t in range(T - 1, -1, -1):
        # S currently approximates S_t; solve S_t = S_{t-1}(diag w + a b^T) + v k^T for S_{t-1}
        M = (np.diag(w[t]) + np.outer(a[t], b[t])).astype(np.float32)
        S = np.linalg.solve(M.T, (S - np.outer(v[t], k[t]).astype(np.float32)).T).T.astype(np.float32)
        n = T - t
        if t % 32 == 0:
            ref = ck[0, 0, t // 32]
            err_at[n] = np.linalg.norm(S - ref) / np.linalg.norm(ref)
    assert err_at[32] < err_at[128]
    assert err_at[128] > 1e-2
