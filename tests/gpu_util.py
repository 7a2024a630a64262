"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare output by output, head by head (relative
L2 in fp64 over each (b, h) head's part of an output)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import linear_rnn_lm_amd as L
import oracle

# Tolerances on rel-L2 (|x - ref|_2 / |ref|_2 in fp64), required of every
# (b, h) head's part of every output separately, so that one wrong head is not
# diluted by the others: fp32 inputs 1e-5 on forward outputs and 1e-4 on
# gradients; bf16 inputs (the oracle receives the same rounded values) 2e-3 on
# everything.
TOL = {
    torch.float32: {"fwd": 1e-5, "bwd": 1e-4},
    torch.bfloat16: {"fwd": 2e-3, "bwd": 2e-3},
}
FWD_NAMES = ("y", "ckpt", "hT")
BWD_NAMES = ("dr", "dw", "dk", "dv", "da", "db", "dh0")


def note(msg):
    """Name the case before a GPU step, flushed, so a crash log says what ran."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def _np(t):
    return None if t is None else t.detach().double().cpu().numpy()


def run_gpu(x, dhT=None, sequential=False, bwd=True):
    dev = torch.device("cuda:0")
    ins = [t.to(dev) for t in x.tensors()]
    h0 = None if x.h0 is None else x.h0.to(dev)
    f = L.fwd_sequential if sequential else L.fwd
    y, ck, hT = f(*ins, h0)
    out = {"y": y, "ckpt": ck, "hT": hT}
    if bwd:
        dy = x.dy.to(dev)
        dh = None if dhT is None else dhT.to(dev)
        g = L.bwd(dy, *ins, ck, dh)
        out.update(dict(zip(BWD_NAMES, g)))
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


def run_oracle(x, dhT=None, bwd=True):
    y, ck, hT = oracle.fwd(*x.tensors(), x.h0)
    out = {"y": y, "ckpt": ck, "hT": hT}
    if bwd:
        g = oracle.bwd(*x.tensors(), x.dy, x.h0, dhT)
        out.update(dict(zip(BWD_NAMES, g)))
    return out


# outputs laid out head-major, (B, H, ...); every other output is a token
# tensor (B, T, H, D)
STATE_NAMES = ("ckpt", "hT", "dh0")


def by_head(name, x):
    """An output as a (B*H, n) array, one row per (b, h) head."""
    x = np.asarray(x, dtype=np.float64)
    if name in STATE_NAMES:
        return x.reshape(x.shape[0] * x.shape[1], -1)
    B, T, H, D = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * H, T * D)


def rel_heads(name, x, ref):
    """Largest rel-L2 over the heads (a head whose reference is all zero
    contributes the norm of its error)."""
    xh, rh = by_head(name, x), by_head(name, ref)
    num = np.linalg.norm(xh - rh, axis=1)
    den = np.linalg.norm(rh, axis=1)
    per = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(per.max())


def compare(gpu, ref, dtype, names=None):
    """Return {name: worst per-head rel-L2} and the list of names over tolerance."""
    names = names or [n for n in FWD_NAMES + BWD_NAMES if n in gpu and n in ref]
    errs, bad = {}, []
    for n in names:
        e = rel_heads(n, gpu[n], ref[n])
        errs[n] = e
        tol = TOL[dtype]["fwd" if n in FWD_NAMES else "bwd"]
        if not (e <= tol):
            bad.append(n)
    return errs, bad


def slice_heads(x, bsel, hsel):
    """Sub-workload of heads (b, h) for b in bsel, h in hsel (index lists)."""
    from linear_rnn_lm_amd.inputs import Inputs
    bi = torch.tensor(bsel)
    hi = torch.tensor(hsel)
    tok = lambda t: t.index_select(0, bi).index_select(2, hi).contiguous()
    st = lambda t: None if t is None else t.index_select(0, bi).index_select(1, hi).contiguous()
    return Inputs(*(tok(t) for t in x.tensors()), st(x.h0), tok(x.dy))


def select_heads(out, bsel, hsel):
    bi, hi = np.asarray(bsel), np.asarray(hsel)
    res = {}
    for n, v in out.items():
        if v is None:
            continue
        if n in ("ckpt", "hT", "dh0"):
            res[n] = v[bi][:, hi]
        else:
            res[n] = v[bi][:, :, hi]
    return res
