"""Seeded synthetic inputs for the WKV7 recurrence (shared by tests, smoke and bench).

This module holds no part of the recurrence itself: it only draws the six
(B,T,H,D) input tensors, the optional initial state and the output gradient,
with the shapes and value distributions of the workloads on the pages:

* shapes: the rwkv-mlx page's "debug" training config (ctx 1024, batch 12,
  6 heads of 64, section "Конфигурация" table and the usage example of
  section "wkv7_checkpoint.py"); the 0.1B and 1.5B model sizes of the RWKV-LM
  README page (n_embd 768 and 2048 with 64-wide heads); the 7B state geometry
  of the RWKV-7 news page (32 layers x 64 heads x 64x64 state per sequence).
* values, drawn in this fixed order with a CPU torch.Generator, fp32:
    1. r ~ N(0,1)
    2. w = exp(-exp(-0.5) * sigmoid(N(0,1)))          -> w in (0.545, 1)
    3. k ~ N(0,1) / 8
    4. v ~ N(0,1)
    5. kappa = N(0,1) normalised to unit L2 norm over D; a = -kappa
    6. b = kappa * sigmoid(N(0,1))
    7. h0 ~ N(0, 0.1) (standard deviation 0.1), only where the workload has one
    8. dy ~ N(0,1), fp32, shape of y
  then r, w, k, v, a, b are rounded once (round-to-nearest-even) to bf16 for
  the bf16 workloads.  Both the HIP path and the oracle receive the identical
  rounded tensors.

No dataset, checkpoint or trained weight is involved: the pages' training
corpora and weights stand in as these synthetic draws of the same shapes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

D = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dtype: torch.dtype          # storage dtype of r, w, k, v, a, b
    seed: int
    with_h0: bool
    layers: int = 1             # recurrent-step workload: one call per layer
    description: str = ""

    @property
    def heads(self) -> int:
        return self.B * self.H

    @property
    def head_tokens(self) -> int:
        return self.B * self.T * self.H


# Five workloads.  Shapes and distributions as listed in the module docstring.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 64, 1, torch.float32, 0, False,
                          description="B1 T64 H1 D64, fp32 inputs"),
    "debug_36m": Workload("debug_36m", 12, 1024, 6, torch.bfloat16, 1, False,
                          description="B12 T1024 H6 D64, bf16 inputs (36M debug training layer)"),
    "rwkv_0b1": Workload("rwkv_0b1", 4, 512, 12, torch.bfloat16, 2, False,
                         description="B4 T512 H12 D64, bf16 inputs (0.1B class, n_embd 768)"),
    "rwkv_1b5": Workload("rwkv_1b5", 8, 4096, 32, torch.bfloat16, 3, True,
                         description="B8 T4096 H32 D64, bf16 inputs, h0 ~ N(0,0.1) (1.5B class)"),
    "rwkv_7b_step": Workload("rwkv_7b_step", 256, 1, 64, torch.bfloat16, 4000, True, layers=32,
                             description="32 layers x (B256 T1 H64 D64), bf16 inputs, "
                                         "fp32 state updated in place (7B recurrent step)"),
}


@dataclasses.dataclass
class Inputs:
    r: torch.Tensor
    w: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    h0: Optional[torch.Tensor]
    dy: torch.Tensor

    def tensors(self):
        return (self.r, self.w, self.k, self.v, self.a, self.b)

    def to(self, device):
        f = lambda x: None if x is None else x.to(device)
        return Inputs(*(f(getattr(self, n)) for n in ("r", "w", "k", "v", "a", "b", "h0", "dy")))


def make_inputs(B: int, T: int, H: int, dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                with_h0: bool = False, h0_std: float = 0.1, device: str = "cpu") -> Inputs:
    """Draw one set of inputs (on the CPU unless `device` says otherwise; a
    device generator gives a different, equally seeded stream, for shapes too
    large to draw on the host).  Deterministic for a given seed and device."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (B, T, H, D)

    def n01(*s):
        return torch.randn(*s, generator=g, dtype=torch.float32, device=device)

    r = n01(*shape)
    w = torch.exp(-math.exp(-0.5) * torch.sigmoid(n01(*shape)))
    k = n01(*shape) / 8.0
    v = n01(*shape)
    kappa = n01(*shape)
    kappa = kappa / kappa.norm(dim=-1, keepdim=True)
    a = -kappa
    b = kappa * torch.sigmoid(n01(*shape))
    h0 = n01(B, H, D, D) * h0_std if with_h0 else None
    dy = n01(*shape)
    cast = lambda x: x.to(dtype).contiguous()
    return Inputs(cast(r), cast(w), cast(k), cast(v), cast(a), cast(b),
                  None if h0 is None else h0.contiguous(), dy.contiguous())


# Inputs at the edges of the recurrence's domain.  Each kind starts from the
# draws of make_inputs (same seed, same order) and replaces some of them:
#   w_eighth     w = 1/8 everywhere: the smallest decay the library accepts, so
#                a chunk's running decay products reach 2^-96
#   w_near_one   w ~ U[0.999, 1]: the state barely decays and grows over T
#   linear_attn  w = 1, a = b = 0: the state is the running sum of v k^T
#   a_zero       a = 0 (b as drawn): no state-dependent term, sa = 0
#   delta_rule   w = 1, r = k = kh, a = -kh, b = kh for a unit vector kh:
#                each token writes v along kh and reads it back
EDGE_KINDS = ("w_eighth", "w_near_one", "linear_attn", "a_zero", "delta_rule")


def make_edge_inputs(kind: str, B: int, T: int, H: int, dtype: torch.dtype = torch.float32, seed: int = 0,
                     with_h0: bool = False) -> Inputs:
    if kind not in EDGE_KINDS:
        raise ValueError(f"unknown edge kind {kind!r}; one of {EDGE_KINDS}")
    x = make_inputs(B, T, H, torch.float32, seed, with_h0)
    r, w, k, v, a, b = x.tensors()
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 1)
    if kind == "w_eighth":
        w = torch.full_like(w, 0.125)
    elif kind == "w_near_one":
        w = 1.0 - 0.001 * torch.rand(w.shape, generator=g)
    elif kind == "linear_attn":
        w, a, b = torch.ones_like(w), torch.zeros_like(a), torch.zeros_like(b)
    elif kind == "a_zero":
        a = torch.zeros_like(a)
    else:
        kh = -a                      # the recipe's unit vector kappa
        w, r, k, b = torch.ones_like(w), kh.clone(), kh.clone(), kh.clone()
    cast = lambda t: t.to(dtype).contiguous()
    return Inputs(cast(r), cast(w), cast(k), cast(v), cast(a), cast(b), x.h0, x.dy)


@dataclasses.dataclass
class ProjInputs:
    """Inputs of the layer with its time-mix prologue: raw projections in
    place of w, a and b."""
    r: torch.Tensor
    w_raw: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    kappa: torch.Tensor
    alpha: torch.Tensor
    h0: Optional[torch.Tensor]
    dy: torch.Tensor

    def tensors(self):
        return (self.r, self.w_raw, self.k, self.v, self.kappa, self.alpha)

    def to(self, device):
        f = lambda x: None if x is None else x.to(device)
        return ProjInputs(*(f(getattr(self, n)) for n in ("r", "w_raw", "k", "v", "kappa", "alpha", "h0", "dy")))


def make_proj_inputs(B: int, T: int, H: int, dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                     with_h0: bool = False, h0_std: float = 0.1) -> ProjInputs:
    """The draws of make_inputs, in the same order, with w_raw, kappa and alpha
    left as drawn (N(0,1)): the layer's prologue derives w, a and b from them."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, T, H, D)

    def n01(*s):
        return torch.randn(*s, generator=g, dtype=torch.float32)

    r = n01(*shape)
    w_raw = n01(*shape)
    k = n01(*shape) / 8.0
    v = n01(*shape)
    kappa = n01(*shape)
    alpha = n01(*shape)
    h0 = n01(B, H, D, D) * h0_std if with_h0 else None
    dy = n01(*shape)
    cast = lambda x: x.to(dtype).contiguous()
    return ProjInputs(cast(r), cast(w_raw), cast(k), cast(v), cast(kappa), cast(alpha),
                      None if h0 is None else h0.contiguous(), dy.contiguous())


def workload_inputs(wl: Workload, layer: int = 0) -> Inputs:
    """Inputs of one workload (for the recurrent-step workload: of one layer)."""
    return make_inputs(wl.B, wl.T, wl.H, wl.dtype, wl.seed + layer, wl.with_h0)
