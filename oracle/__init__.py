"""fp64 CPU oracle for the WKV7 recurrence (forward and backward).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports,
links or executes anything here, and nothing here imports the HIP library.

The arithmetic lives in ``wkv7_oracle.c`` (plain scalar C, fp64, one head per
thread).  This module compiles it with gcc when the shared object is missing
or older than the source, and marshals numpy arrays through ctypes.

Method: rwkv-mlx page, section "Metal kernel architecture" (forward block
for the per-token update and output; backward block for the reverse walk that
yields dr, dw, dk, dv, da, db).  Readings of the page are listed in the C
file's header comment.

Every function here is pinned by CPU tests against closed forms, special
cases and finite differences (tests/test_oracle_*.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv7_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CHUNK = 32

_default = None


def build(force: bool = False) -> str:
    """Compile the oracle shared library with gcc; returns its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source into a shared object at ``out``."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, src, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleLib:
    """ctypes view of one compiled oracle shared object."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_wkv7_fwd.argtypes = [i, i, i, i] + [dp] * 7 + [dp] * 3 + [i]
        lib.oracle_wkv7_fwd.restype = i
        lib.oracle_wkv7_bwd.argtypes = [i, i, i, i] + [dp] * 9 + [dp] * 7 + [i]
        lib.oracle_wkv7_bwd.restype = i
        lib.oracle_proj_fwd.argtypes = [ctypes.c_long, i] + [dp] * 6
        lib.oracle_proj_fwd.restype = i
        lib.oracle_proj_bwd.argtypes = [ctypes.c_long, i] + [dp] * 9
        lib.oracle_proj_bwd.restype = i
        self.lib = lib
        self.path = path

    def fwd(self, r, w, k, v, a, b, h0=None, want_ckpt=True, threads=None):
        return _fwd(self.lib, r, w, k, v, a, b, h0, want_ckpt, threads)

    def bwd(self, r, w, k, v, a, b, dy, h0=None, dhT=None, threads=None):
        return _bwd(self.lib, r, w, k, v, a, b, dy, h0, dhT, threads)

    def proj_fwd(self, w_raw, kappa, alpha):
        return _proj_fwd(self.lib, w_raw, kappa, alpha)

    def proj_bwd(self, w_raw, kappa, alpha, dw, da, db):
        return _proj_bwd(self.lib, w_raw, kappa, alpha, dw, da, db)


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib(build())
    return _default


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


MAX_THREADS = 16   # worker threads at most (one head each; each holds all states of its head)


def default_threads() -> int:
    """Host cores available to this process, at most MAX_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def num_chunks(T: int) -> int:
    return (T + CHUNK - 1) // CHUNK


def fwd(r, w, k, v, a, b, h0=None, want_ckpt=True, threads=None):
    """Forward over (B,T,H,D) inputs with the default oracle build; see _fwd."""
    return default().fwd(r, w, k, v, a, b, h0, want_ckpt, threads)


def bwd(r, w, k, v, a, b, dy, h0=None, dhT=None, threads=None):
    """Backward with the default oracle build; see _bwd."""
    return default().bwd(r, w, k, v, a, b, dy, h0, dhT, threads)


def proj_fwd(w_raw, kappa, alpha):
    """Time-mix prologue with the default oracle build; see _proj_fwd."""
    return default().proj_fwd(w_raw, kappa, alpha)


def proj_bwd(w_raw, kappa, alpha, dw, da, db):
    """Backward of the prologue with the default oracle build; see _proj_bwd."""
    return default().proj_bwd(w_raw, kappa, alpha, dw, da, db)


def _proj_fwd(lib, w_raw, kappa, alpha):
    """(w, a, b) from raw projections of any shape (..., D): steps P1-P5 of
    the C source's prologue comment."""
    w_raw, kappa, alpha = (_as64(x) for x in (w_raw, kappa, alpha))
    assert w_raw.shape == kappa.shape == alpha.shape
    D = w_raw.shape[-1]
    outs = [np.empty(w_raw.shape) for _ in range(3)]
    rc = lib.oracle_proj_fwd(w_raw.size // D, D, *map(_ptr, (w_raw, kappa, alpha)), *map(_ptr, outs))
    if rc != 0:
        raise RuntimeError(f"oracle_proj_fwd failed with code {rc}")
    return tuple(outs)


def _proj_bwd(lib, w_raw, kappa, alpha, dw, da, db):
    """(dw_raw, dkappa, dalpha) from the gradients on (w, a, b): steps Q1-Q4."""
    w_raw, kappa, alpha, dw, da, db = (_as64(x) for x in (w_raw, kappa, alpha, dw, da, db))
    for x in (kappa, alpha, dw, da, db):
        assert x.shape == w_raw.shape
    D = w_raw.shape[-1]
    outs = [np.empty(w_raw.shape) for _ in range(3)]
    rc = lib.oracle_proj_bwd(w_raw.size // D, D, *map(_ptr, (w_raw, kappa, alpha, dw, da, db)),
                             *map(_ptr, outs))
    if rc != 0:
        raise RuntimeError(f"oracle_proj_bwd failed with code {rc}")
    return tuple(outs)


def _fwd(lib, r, w, k, v, a, b, h0=None, want_ckpt=True, threads=None):
    """Forward over (B,T,H,D) inputs.

    Returns (y, ckpt, hT): y (B,T,H,D), ckpt (B,H,NC,D,D) with ckpt[...,c,:,:]
    the state entering chunk c (None if want_ckpt is False), hT (B,H,D,D).
    """
    r, w, k, v, a, b, h0 = (_as64(x) for x in (r, w, k, v, a, b, h0))
    B, T, H, D = r.shape
    for x in (w, k, v, a, b):
        assert x.shape == (B, T, H, D)
    if h0 is not None:
        assert h0.shape == (B, H, D, D)
    y = np.empty((B, T, H, D))
    ckpt = np.empty((B, H, num_chunks(T), D, D)) if want_ckpt else None
    hT = np.empty((B, H, D, D))
    rc = lib.oracle_wkv7_fwd(B, T, H, D, *map(_ptr, (r, w, k, v, a, b, h0)),
                                 _ptr(y), _ptr(ckpt), _ptr(hT),
                                 threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_wkv7_fwd failed with code {rc}")
    return y, ckpt, hT


def _bwd(lib, r, w, k, v, a, b, dy, h0=None, dhT=None, threads=None):
    """Backward: returns (dr, dw, dk, dv, da, db, dh0) for loss gradient dy on y
    and dhT on the final state (None = zero)."""
    r, w, k, v, a, b, dy, h0, dhT = (_as64(x) for x in (r, w, k, v, a, b, dy, h0, dhT))
    B, T, H, D = r.shape
    assert dy.shape == (B, T, H, D)
    outs = [np.empty((B, T, H, D)) for _ in range(6)]
    dh0 = np.empty((B, H, D, D))
    rc = lib.oracle_wkv7_bwd(B, T, H, D, *map(_ptr, (r, w, k, v, a, b, h0, dy, dhT)),
                                 *map(_ptr, outs), _ptr(dh0),
                                 threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_wkv7_bwd failed with code {rc}")
    return (*outs, dh0)
