"""linear_rnn_lm_amd -- the RWKV-7 WKV7 recurrence on AMD Instinct MI355X.

Thin Python binding of ``libwkv7.so`` (C ABI in ``include/wkv7.h``).  It only
marshals arguments: torch supplies device memory and the current HIP stream,
every step of the computation runs in the library's HIP kernels.  There is no
CPU fallback; if the library is missing, calls raise.

    y, ckpt, hT = fwd(r, w, k, v, a, b, h0)            # (B,T,H,64) inputs
    dr, dw, dk, dv, da, db, dh0 = bwd(dy, r, w, k, v, a, b, ckpt, dhT)
    WKV7.apply(r, w, k, v, a, b, h0)                   # autograd op -> (y, hT)
    WKV7.apply(r, w, k, v, a, b, h0, False)            # the same, chunk operands not kept

The recurrence (rwkv-mlx page, section "Metal kernel architecture"): per
head a 64x64 fp32 state S; per token sa = S a, S = S diag(w) + v k^T + sa b^T,
y = S r.  Inputs r, w, k, v, a, b are fp32 or bf16; all outputs are fp32.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["lib", "fwd", "fwd_sequential", "fwd_scan", "chunk_prepare", "chunk_inverse", "bwd", "bwd_scan",
           "bwd_inputs", "step", "WKV7", "Wkv7Error",
           "num_chunks", "workspace_bytes", "chunk_ops_bytes", "CHUNK", "HEAD_SIZE"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv7.so")
CHUNK = 32
HEAD_SIZE = 64
F32, BF16 = 0, 1

_lib = None


class Wkv7Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def lib():
    """Load libwkv7.so (built by ``python -m linear_rnn_lm_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m linear_rnn_lm_amd.build` "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.wkv7_version.restype = i
        L.wkv7_chunk_len.restype = i
        L.wkv7_num_chunks.argtypes = [i64]
        L.wkv7_num_chunks.restype = i64
        L.wkv7_status_str.argtypes = [i]
        L.wkv7_status_str.restype = ctypes.c_char_p
        for q in ("wkv7_bwd_workspace_bytes", "wkv7_fwd_workspace_bytes", "wkv7_chunk_ops_bytes"):
            getattr(L, q).argtypes = [i, i, i, i]
            getattr(L, q).restype = sz
        L.wkv7_chunk_prepare.argtypes = [i, i, i, i, i] + [vp] * 5 + [vp] + [vp]
        L.wkv7_chunk_prepare.restype = i
        L.wkv7_fwd.argtypes = [i, i, i, i, i] + [vp] * 6 + [vp] * 4 + [vp, sz] + [vp]
        L.wkv7_fwd.restype = i
        L.wkv7_fwd_scan.argtypes = [i, i, i, i, i] + [vp] * 2 + [vp] * 4 + [vp]
        L.wkv7_fwd_scan.restype = i
        L.wkv7_fwd_sequential.argtypes = [i, i, i, i, i] + [vp] * 6 + [vp] * 4 + [vp]
        L.wkv7_fwd_sequential.restype = i
        L.wkv7_bwd.argtypes = [i, i, i, i, i] + [vp] * 2 + [vp] * 6 + [vp] + [vp] * 7 + [vp, sz, vp]
        L.wkv7_bwd.restype = i
        L.wkv7_bwd_scan.argtypes = [i, i, i, i, i] + [vp] * 3 + [vp] * 3 + [vp]
        L.wkv7_bwd_scan.restype = i
        L.wkv7_bwd_inputs.argtypes = [i, i, i, i, i] + [vp] * 2 + [vp] * 6 + [vp] * 3 + [vp] * 5 + [vp]
        L.wkv7_bwd_inputs.restype = i
        L.wkv7_fwd_proj.argtypes = L.wkv7_fwd.argtypes
        L.wkv7_fwd_proj.restype = i
        L.wkv7_bwd_proj.argtypes = L.wkv7_bwd.argtypes
        L.wkv7_bwd_proj.restype = i
        L.wkv7_fwd_noalloc.argtypes = [i, i, i, i, i] + [vp] * 6 + [vp] * 4 + [vp]
        L.wkv7_fwd_noalloc.restype = i
        L.wkv7_fwd_noalloc_max_bytes.restype = sz
        L.wkv7_bwd_division.argtypes = [i, i, i, i, i] + [vp] * 2 + [vp] * 6 + [vp] * 2 + [i] + [vp] * 7 + [vp]
        L.wkv7_bwd_division.restype = i
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise Wkv7Error(fn, status, lib().wkv7_status_str(status).decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"inputs must be float32 or bfloat16, got {t.dtype}")


def _stream(device):
    """The current HIP stream of `device`.  Evaluated as the last argument of
    every library call, after the tensors have been validated, so it is also
    where a call on tensors outside a GPU is refused."""
    import torch
    if device.type != "cuda":
        raise ValueError(f"libwkv7 works on GPU tensors; got tensors on {device}")
    return torch.cuda.current_stream(device).cuda_stream


def _shape(r):
    if r.dim() != 4:
        raise ValueError("inputs must be (B, T, H, D)")
    return tuple(r.shape)


# ---------------------------------------------------------------------------
# Host-side validation of every tensor a call hands to the library, before
# any pointer is passed: the kernels trust shapes, dtypes and devices, so a
# CPU tensor, an undersized buffer or a strided view must never reach them.

def _where(t):
    return f"{tuple(t.shape)} {t.dtype} on {t.device}"


def _dense_on(fn, name, t, dev):
    if t.device != dev:
        raise ValueError(f"{fn}: {name} is on {t.device}, expected {dev} (the device of the inputs)")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous (got strides {t.stride()})")


def _check_tokens(fn, names, tensors):
    """Token inputs: (B, T, H, 64), one dtype (fp32 or bf16), one device,
    contiguous.  Returns (B, T, H, D).  (That the device is a GPU is checked
    by _stream, after every other check.)"""
    import torch
    r = tensors[0]
    if r.dim() != 4 or r.shape[-1] != HEAD_SIZE:
        raise ValueError(f"{fn}: {names[0]} must be (B, T, H, {HEAD_SIZE}), got {tuple(r.shape)}")
    if r.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{fn}: {names[0]} must be float32 or bfloat16, got {r.dtype}")
    for n, t in zip(names, tensors):
        if t.shape != r.shape or t.dtype != r.dtype:
            raise ValueError(f"{fn}: {n} is {_where(t)}, expected the shape and dtype of {names[0]} ({_where(r)})")
        _dense_on(fn, n, t, r.device)
    return tuple(r.shape)


def _check_f32(fn, name, t, shape, dev, required=True):
    """An fp32 tensor of exactly `shape` on `dev`, contiguous (None allowed
    unless required)."""
    import torch
    if t is None:
        if required:
            raise ValueError(f"{fn}: {name} is required")
        return
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {name} is {_where(t)}, expected {tuple(shape)} torch.float32")
    _dense_on(fn, name, t, dev)


def _check_bytes(fn, name, t, nbytes, dev):
    """A scratch or operand buffer of at least `nbytes` bytes on `dev`, contiguous."""
    _dense_on(fn, name, t, dev)
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{fn}: {name} holds {have} bytes, needs {nbytes}")


def _state_shape(B, H):
    return (B, H, HEAD_SIZE, HEAD_SIZE)


def _ckpt_shape(B, T, H):
    return (B, H, num_chunks(T), HEAD_SIZE, HEAD_SIZE)


def num_chunks(T: int) -> int:
    return int(lib().wkv7_num_chunks(T))


def workspace_bytes(B: int, T: int, H: int, D: int = HEAD_SIZE) -> int:
    """Workspace bytes of wkv7_bwd."""
    return int(lib().wkv7_bwd_workspace_bytes(B, T, H, D))


def fwd_workspace_bytes(B: int, T: int, H: int, D: int = HEAD_SIZE) -> int:
    return int(lib().wkv7_fwd_workspace_bytes(B, T, H, D))


def chunk_ops_bytes(B: int, T: int, H: int, D: int = HEAD_SIZE) -> int:
    return int(lib().wkv7_chunk_ops_bytes(B, T, H, D))


def _f32_bytes(nbytes, device):
    import torch
    return torch.empty(max(nbytes, 16) // 4, device=device, dtype=torch.float32)


def _fwd_outputs(r, want_y, want_ckpt, want_hT, y, ckpt, hT):
    import torch
    B, T, H, D = _shape(r)
    f32 = dict(device=r.device, dtype=torch.float32)
    if want_y and y is None:
        y = torch.empty((B, T, H, D), **f32)
    if want_ckpt and ckpt is None:
        ckpt = torch.empty((B, H, num_chunks(T), D, D), **f32)
    if want_hT and hT is None:
        hT = torch.empty((B, H, D, D), **f32)
    return y, ckpt, hT


def _check_fwd_states(fn, r, h0, y, ckpt, hT):
    B, T, H, D = r.shape
    _check_f32(fn, "h0", h0, _state_shape(B, H), r.device, required=False)
    _check_f32(fn, "y", y, (B, T, H, D), r.device, required=False)
    _check_f32(fn, "ckpt", ckpt, _ckpt_shape(B, T, H), r.device, required=False)
    _check_f32(fn, "hT", hT, _state_shape(B, H), r.device, required=False)


def fwd(r, w, k, v, a, b, h0=None, *, want_y=True, want_ckpt=True, want_hT=True,
        y=None, ckpt=None, hT=None, workspace=None):
    """Forward.  Returns (y, ckpt, hT); entries not wanted are None.
    Pre-allocated outputs may be passed; hT may be h0 (in-place update)."""
    B, T, H, D = _check_tokens("wkv7_fwd", "rwkvab", (r, w, k, v, a, b))
    y, ckpt, hT = _fwd_outputs(r, want_y, want_ckpt, want_hT, y, ckpt, hT)
    _check_fwd_states("wkv7_fwd", r, h0, y, ckpt, hT)
    need = fwd_workspace_bytes(B, T, H, D)
    if workspace is None and need:
        workspace = _f32_bytes(need, r.device)
    if workspace is not None:
        _check_bytes("wkv7_fwd", "workspace", workspace, need, r.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().wkv7_fwd(B, T, H, D, _dtype_code(r), *map(_ptr, (r, w, k, v, a, b)), _ptr(h0),
                        _ptr(y), _ptr(ckpt), _ptr(hT), _ptr(workspace), wsb, _stream(r.device))
    _check("wkv7_fwd", st)
    return y, ckpt, hT


def fwd_noalloc(r, w, k, v, a, b, h0=None, *, y, ckpt=None, hT=None):
    """Forward whose chunk operands live in the library's static device scratch
    (wkv7_fwd_noalloc): nothing is allocated, so the outputs must be passed.
    Calls that overlap in time on one GPU race on that scratch."""
    B, T, H, D = _check_tokens("wkv7_fwd_noalloc", "rwkvab", (r, w, k, v, a, b))
    _check_fwd_states("wkv7_fwd_noalloc", r, h0, y, ckpt, hT)
    st = lib().wkv7_fwd_noalloc(B, T, H, D, _dtype_code(r), *map(_ptr, (r, w, k, v, a, b)), _ptr(h0),
                                _ptr(y), _ptr(ckpt), _ptr(hT), _stream(r.device))
    _check("wkv7_fwd_noalloc", st)
    return y, ckpt, hT


def chunk_prepare(r, w, k, a, b, out=None):
    """Per-chunk operands of r, w, k, a, b (see include/wkv7.h), as a flat
    fp32 tensor of chunk_ops_bytes(...) bytes; the forward and the backward of
    one step may share it."""
    B, T, H, D = _check_tokens("wkv7_chunk_prepare", "rwkab", (r, w, k, a, b))
    if out is None:
        out = _f32_bytes(chunk_ops_bytes(B, T, H, D), r.device)
    _check_bytes("wkv7_chunk_prepare", "out", out, chunk_ops_bytes(B, T, H, D), r.device)
    st = lib().wkv7_chunk_prepare(B, T, H, D, _dtype_code(r), *map(_ptr, (r, w, k, a, b)), _ptr(out),
                                  _stream(r.device))
    _check("wkv7_chunk_prepare", st)
    return out


def chunk_inverse(chunk_ops, B, T, H):
    """View of the (I - L)^-1 part of chunk operands: (B, H, NC, 32, 32) fp32."""
    n = B * H * num_chunks(T) * CHUNK * CHUNK
    return chunk_ops[:n].view(B, H, num_chunks(T), CHUNK, CHUNK)


def fwd_scan(v, chunk_ops, h0=None, *, want_y=True, want_ckpt=True, want_hT=True, y=None, ckpt=None, hT=None):
    """Forward given the chunk operands of the same r, w, k, a, b."""
    B, T, H, D = _check_tokens("wkv7_fwd_scan", "v", (v,))
    y, ckpt, hT = _fwd_outputs(v, want_y, want_ckpt, want_hT, y, ckpt, hT)
    _check_fwd_states("wkv7_fwd_scan", v, h0, y, ckpt, hT)
    _check_bytes("wkv7_fwd_scan", "chunk_ops", chunk_ops, chunk_ops_bytes(B, T, H, D), v.device)
    st = lib().wkv7_fwd_scan(B, T, H, D, _dtype_code(v), _ptr(v), _ptr(chunk_ops), _ptr(h0), _ptr(y),
                             _ptr(ckpt), _ptr(hT), _stream(v.device))
    _check("wkv7_fwd_scan", st)
    return y, ckpt, hT


def fwd_sequential(r, w, k, v, a, b, h0=None, *, want_y=True, want_ckpt=True, want_hT=True,
                   y=None, ckpt=None, hT=None):
    """Token-by-token forward (same results as ``fwd``)."""
    B, T, H, D = _check_tokens("wkv7_fwd_sequential", "rwkvab", (r, w, k, v, a, b))
    y, ckpt, hT = _fwd_outputs(r, want_y, want_ckpt, want_hT, y, ckpt, hT)
    _check_fwd_states("wkv7_fwd_sequential", r, h0, y, ckpt, hT)
    st = lib().wkv7_fwd_sequential(B, T, H, D, _dtype_code(r), *map(_ptr, (r, w, k, v, a, b)), _ptr(h0),
                                   _ptr(y), _ptr(ckpt), _ptr(hT), _stream(r.device))
    _check("wkv7_fwd_sequential", st)
    return y, ckpt, hT


def step(r, w, k, v, a, b, state, y=None):
    """One recurrent call updating ``state`` (B,H,64,64) in place; returns y."""
    B, T, H, D = _check_tokens("wkv7_fwd", "rwkvab", (r, w, k, v, a, b))
    _check_f32("wkv7_fwd", "state", state, _state_shape(B, H), r.device)
    y, _, _ = fwd(r, w, k, v, a, b, state, want_ckpt=False, y=y, hT=state)
    return y


def _check_bwd_tensors(fn, r, dy, ckpt, dhT, out, n_out):
    B, T, H, D = r.shape
    _check_f32(fn, "dy", dy, (B, T, H, D), r.device)
    _check_f32(fn, "ckpt", ckpt, _ckpt_shape(B, T, H), r.device)
    _check_f32(fn, "dhT", dhT, _state_shape(B, H), r.device, required=False)
    if len(out) != n_out:
        raise ValueError(f"{fn}: out must hold {n_out} tensors, got {len(out)}")
    for i, o in enumerate(out):
        _check_f32(fn, f"out[{i}]", o, (B, T, H, D), r.device)


def bwd(dy, r, w, k, v, a, b, ckpt, dhT=None, *, want_dh0=True, workspace=None, out=None):
    """Backward.  Returns (dr, dw, dk, dv, da, db, dh0) as fp32 tensors."""
    import torch
    B, T, H, D = _check_tokens("wkv7_bwd", "rwkvab", (r, w, k, v, a, b))
    dev = r.device
    f32 = dict(device=dev, dtype=torch.float32)
    if out is None:
        out = [torch.empty((B, T, H, D), **f32) for _ in range(6)]
    dh0 = torch.empty((B, H, D, D), **f32) if want_dh0 else None
    need = workspace_bytes(B, T, H, D)
    if workspace is None:
        workspace = torch.empty(need // 4, **f32)
    _check_bwd_tensors("wkv7_bwd", r, dy, ckpt, dhT, out, 6)
    _check_bytes("wkv7_bwd", "workspace", workspace, need, dev)
    st = lib().wkv7_bwd(B, T, H, D, _dtype_code(r), _ptr(dy), _ptr(dhT),
                        *map(_ptr, (r, w, k, v, a, b)), _ptr(ckpt), *map(_ptr, out), _ptr(dh0),
                        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check("wkv7_bwd", st)
    return (*out, dh0)


def fwd_proj(r, w_raw, k, v, kappa, alpha, h0=None, *, want_y=True, want_ckpt=True, want_hT=True,
             y=None, ckpt=None, hT=None, workspace=None):
    """Forward of the layer with its time-mix prologue (w, a, b formed in the
    kernels from w_raw, kappa, alpha; see wkv7_fwd_proj).  Returns (y, ckpt, hT)."""
    names = ("r", "w_raw", "k", "v", "kappa", "alpha")
    B, T, H, D = _check_tokens("wkv7_fwd_proj", names, (r, w_raw, k, v, kappa, alpha))
    y, ckpt, hT = _fwd_outputs(r, want_y, want_ckpt, want_hT, y, ckpt, hT)
    _check_fwd_states("wkv7_fwd_proj", r, h0, y, ckpt, hT)
    need = fwd_workspace_bytes(B, T, H, D)
    if workspace is None and need:
        workspace = _f32_bytes(need, r.device)
    if workspace is not None:
        _check_bytes("wkv7_fwd_proj", "workspace", workspace, need, r.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().wkv7_fwd_proj(B, T, H, D, _dtype_code(r), *map(_ptr, (r, w_raw, k, v, kappa, alpha)), _ptr(h0),
                             _ptr(y), _ptr(ckpt), _ptr(hT), _ptr(workspace), wsb, _stream(r.device))
    _check("wkv7_fwd_proj", st)
    return y, ckpt, hT


def bwd_proj(dy, r, w_raw, k, v, kappa, alpha, ckpt, dhT=None, *, want_dh0=True, workspace=None, out=None):
    """Backward of ``fwd_proj``: (dr, dw_raw, dk, dv, dkappa, dalpha, dh0), fp32."""
    import torch
    names = ("r", "w_raw", "k", "v", "kappa", "alpha")
    B, T, H, D = _check_tokens("wkv7_bwd_proj", names, (r, w_raw, k, v, kappa, alpha))
    dev = r.device
    f32 = dict(device=dev, dtype=torch.float32)
    if out is None:
        out = [torch.empty((B, T, H, D), **f32) for _ in range(6)]
    dh0 = torch.empty((B, H, D, D), **f32) if want_dh0 else None
    if workspace is None:
        workspace = torch.empty(workspace_bytes(B, T, H, D) // 4, **f32)
    _check_bwd_tensors("wkv7_bwd_proj", r, dy, ckpt, dhT, out, 6)
    _check_bytes("wkv7_bwd_proj", "workspace", workspace, workspace_bytes(B, T, H, D), dev)
    st = lib().wkv7_bwd_proj(B, T, H, D, _dtype_code(r), _ptr(dy), _ptr(dhT),
                             *map(_ptr, (r, w_raw, k, v, kappa, alpha)), _ptr(ckpt), *map(_ptr, out), _ptr(dh0),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check("wkv7_bwd_proj", st)
    return (*out, dh0)


def bwd_division(dy, r, w, k, v, a, b, ckpt, hT, dhT=None, *, restart=True, want_dh0=True):
    """Diagnostic backward that rebuilds earlier states by dividing by w (see
    wkv7_bwd_division): (dr, dw, dk, dv, da, db, dh0).  restart=True walks each
    chunk from the exact state at its end; False walks the whole sequence from hT."""
    import torch
    B, T, H, D = _check_tokens("wkv7_bwd_division", "rwkvab", (r, w, k, v, a, b))
    f32 = dict(device=r.device, dtype=torch.float32)
    out = [torch.empty((B, T, H, D), **f32) for _ in range(6)]
    dh0 = torch.empty((B, H, D, D), **f32) if want_dh0 else None
    _check_bwd_tensors("wkv7_bwd_division", r, dy, ckpt, dhT, out, 6)
    _check_f32("wkv7_bwd_division", "hT", hT, _state_shape(B, H), r.device)
    st = lib().wkv7_bwd_division(B, T, H, D, _dtype_code(r), _ptr(dy), _ptr(dhT),
                                 *map(_ptr, (r, w, k, v, a, b)), _ptr(ckpt), _ptr(hT), 1 if restart else 0,
                                 *map(_ptr, out), _ptr(dh0), _stream(r.device))
    _check("wkv7_bwd_division", st)
    return (*out, dh0)


def bwd_scan(dy, chunk_ops, dhT=None, *, in_dtype=None, want_dv=True, want_dh0=True, dh_ckpt=None):
    """First backward stage: returns (dh_ckpt, dv, dh0); dh_ckpt[:, :, c] is the
    gradient w.r.t. checkpoint c.  in_dtype: the dtype of the forward's inputs
    (it fixes the operand format), a torch dtype."""
    import torch
    B, T, H, D = _check_tokens("wkv7_bwd_scan", ("dy",), (dy,))
    if dy.dtype != torch.float32:
        raise TypeError(f"wkv7_bwd_scan: dy must be float32, got {dy.dtype}")
    if in_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"wkv7_bwd_scan: in_dtype must be torch.float32 or torch.bfloat16, got {in_dtype}")
    f32 = dict(device=dy.device, dtype=torch.float32)
    if dh_ckpt is None:
        dh_ckpt = torch.empty((B, H, num_chunks(T), D, D), **f32)
    dv = torch.empty((B, T, H, D), **f32) if want_dv else None
    dh0 = torch.empty((B, H, D, D), **f32) if want_dh0 else None
    _check_f32("wkv7_bwd_scan", "dh_ckpt", dh_ckpt, _ckpt_shape(B, T, H), dy.device)
    _check_f32("wkv7_bwd_scan", "dhT", dhT, _state_shape(B, H), dy.device, required=False)
    _check_bytes("wkv7_bwd_scan", "chunk_ops", chunk_ops, chunk_ops_bytes(B, T, H, D), dy.device)
    code = BF16 if in_dtype == torch.bfloat16 else F32
    st = lib().wkv7_bwd_scan(B, T, H, D, code, _ptr(dy), _ptr(dhT), _ptr(chunk_ops), _ptr(dh_ckpt), _ptr(dv),
                             _ptr(dh0), _stream(dy.device))
    _check("wkv7_bwd_scan", st)
    return dh_ckpt, dv, dh0


def bwd_inputs(dy, r, w, k, v, a, b, chunk_ops, ckpt, dh_ckpt, dhT=None, *, out=None):
    """Second backward stage: returns (dr, dw, dk, da, db)."""
    import torch
    B, T, H, D = _check_tokens("wkv7_bwd_inputs", "rwkvab", (r, w, k, v, a, b))
    if out is None:
        out = [torch.empty((B, T, H, D), device=r.device, dtype=torch.float32) for _ in range(5)]
    _check_bwd_tensors("wkv7_bwd_inputs", r, dy, ckpt, dhT, out, 5)
    _check_f32("wkv7_bwd_inputs", "dh_ckpt", dh_ckpt, _ckpt_shape(B, T, H), r.device)
    _check_bytes("wkv7_bwd_inputs", "chunk_ops", chunk_ops, chunk_ops_bytes(B, T, H, D), r.device)
    st = lib().wkv7_bwd_inputs(B, T, H, D, _dtype_code(r), _ptr(dy), _ptr(dhT),
                               *map(_ptr, (r, w, k, v, a, b)), _ptr(chunk_ops), _ptr(ckpt), _ptr(dh_ckpt),
                               *map(_ptr, out), _stream(r.device))
    _check("wkv7_bwd_inputs", st)
    return tuple(out)


def _make_autograd():
    import torch

    class WKV7(torch.autograd.Function):
        """Differentiable op: (r, w, k, v, a, b, h0, keep_ops) -> (y, hT), gradients by
        wkv7_bwd.  keep_ops (default True): keep the chunk operands (1,152 B per
        head-token, plus the chunk inverses) from the forward for the backward; False
        keeps only the checkpoints (512 B per head-token) and the backward prepares
        the operands again (one more pass of the prepare kernel)."""

        @staticmethod
        def forward(ctx, r, w, k, v, a, b, h0=None, keep_ops=True):
            ins = [x.contiguous() for x in (r, w, k, v, a, b)]
            h0c = None if h0 is None else h0.contiguous().float()
            T = ins[0].shape[1]
            if T > 1 and keep_ops:   # one set of chunk operands serves forward and backward
                ops = chunk_prepare(ins[0], ins[1], ins[2], ins[4], ins[5])
                y, ckpt, hT = fwd_scan(ins[3], ops, h0c)
            else:
                ops = None
                y, ckpt, hT = fwd(*ins, h0c)
            ctx.save_for_backward(*ins, ckpt, ops)
            ctx.has_h0 = h0 is not None
            return y, hT

        @staticmethod
        def backward(ctx, dy, dhT):
            *ins, ckpt, ops = ctx.saved_tensors
            if dy is None:
                dy = torch.zeros(ins[0].shape, dtype=torch.float32, device=ins[0].device)
            else:
                dy = dy.contiguous().float()
            dhT = None if dhT is None else dhT.contiguous().float()
            if ops is None:
                dr, dw, dk, dv, da, db, dh0 = bwd(dy, *ins, ckpt, dhT)
            else:
                r, w, k, v, a, b = ins
                dh_ck, dv, dh0 = bwd_scan(dy, ops, dhT, in_dtype=r.dtype)
                dr, dw, dk, da, db = bwd_inputs(dy, r, w, k, v, a, b, ops, ckpt, dh_ck, dhT)
            cast = lambda g, x: g.to(x.dtype)
            grads = [cast(g, x) for g, x in zip((dr, dw, dk, dv, da, db), ins)]
            return (*grads, dh0 if ctx.has_h0 else None, None)

    class WKV7Proj(torch.autograd.Function):
        """Differentiable op with the fused time-mix prologue: (r, w_raw, k, v, kappa, alpha, h0)
        -> (y, hT), gradients by wkv7_bwd_proj (w, a, b are formed inside the kernels)."""

        @staticmethod
        def forward(ctx, r, w_raw, k, v, kappa, alpha, h0=None):
            ins = [x.contiguous() for x in (r, w_raw, k, v, kappa, alpha)]
            h0c = None if h0 is None else h0.contiguous().float()
            y, ckpt, hT = fwd_proj(*ins, h0c)
            ctx.save_for_backward(*ins, ckpt)
            ctx.has_h0 = h0 is not None
            return y, hT

        @staticmethod
        def backward(ctx, dy, dhT):
            *ins, ckpt = ctx.saved_tensors
            if dy is None:
                dy = torch.zeros(ins[0].shape, dtype=torch.float32, device=ins[0].device)
            else:
                dy = dy.contiguous().float()
            dhT = None if dhT is None else dhT.contiguous().float()
            *g, dh0 = bwd_proj(dy, *ins, ckpt, dhT)
            grads = [gi.to(x.dtype) for gi, x in zip(g, ins)]
            return (*grads, dh0 if ctx.has_h0 else None)

    return WKV7, WKV7Proj


class _LazyOp:
    _classes = None

    def __init__(self, index):
        self._index = index

    def __getattr__(self, name):
        if _LazyOp._classes is None:
            _LazyOp._classes = _make_autograd()
        return getattr(_LazyOp._classes[self._index], name)


WKV7 = _LazyOp(0)
WKV7Proj = _LazyOp(1)
