"""Long sequences in segments, by passing the state between calls.

The recurrence carries everything about the past in the D x D state per head,
so a sequence can be cut into segments that are processed one after the
other: the forward of segment s starts from the state the forward of segment
s - 1 ended in, and the backward runs the segments in reverse, handing the
gradient w.r.t. a segment's initial state to the previous segment as the
gradient w.r.t. its final state.  (RWKV-LM project page: the RNN-mode example
that calls the model on a few tokens at a time with the returned state, and
the pointer to infinite-context training.)

Memory: the forward keeps each segment's checkpoints (one state per 32 tokens)
and nothing else, so the whole sequence needs T/32 states per head plus one
segment's work buffers.  With segment lengths that are multiples of 32 the
chunks are the same as in one call over the whole sequence, and so are the
results.  Every step runs in the library's kernels; this module only loops
over the segments.
"""
from __future__ import annotations

from . import bwd, fwd


def _segments(T, seg):
    if seg < 1:
        raise ValueError("segment length must be positive")
    return [(s, min(T, s + seg)) for s in range(0, T, seg)]


def fwd_segments(r, w, k, v, a, b, seg, h0=None):
    """Forward over (B, T, H, 64) inputs in segments of ``seg`` tokens.

    Returns (y, ckpts, hT): y (B, T, H, 64) fp32, the list of each segment's
    checkpoints (what ``bwd_segments`` needs) and the final state.
    """
    import torch
    B, T, H, D = r.shape
    y = torch.empty((B, T, H, D), device=r.device, dtype=torch.float32)
    ckpts, h = [], h0
    for t0, t1 in _segments(T, seg):
        part = [x[:, t0:t1].contiguous() for x in (r, w, k, v, a, b)]
        ys, ck, h = fwd(*part, h)
        y[:, t0:t1] = ys
        ckpts.append(ck)
    return y, ckpts, h


def bwd_segments(dy, r, w, k, v, a, b, ckpts, seg, dhT=None):
    """Backward of ``fwd_segments`` (same ``seg``): (dr, dw, dk, dv, da, db, dh0)."""
    import torch
    B, T, H, D = r.shape
    spans = _segments(T, seg)
    if len(ckpts) != len(spans):
        raise ValueError("checkpoints do not match the segments")
    grads = [torch.empty((B, T, H, D), device=r.device, dtype=torch.float32) for _ in range(6)]
    g = dhT
    for (t0, t1), ck in zip(reversed(spans), reversed(ckpts)):
        part = [x[:, t0:t1].contiguous() for x in (r, w, k, v, a, b)]
        *gs, g = bwd(dy[:, t0:t1].contiguous(), *part, ck, g)
        for dst, src in zip(grads, gs):
            dst[:, t0:t1] = src
    return (*grads, g)
