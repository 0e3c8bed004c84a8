"""Seeded synthetic inputs for the gated delta rule forward.

This module draws random tensors only. It holds none of the method's
arithmetic, so both the fp64 oracle (test side) and the HIP path (product
side) take their inputs from here and from nowhere else.

Value distributions follow the workloads the library is measured on:
  * q, k ~ N(0, 1) in fp32, L2-normalised over the feature axis per
    (token, head), then rounded to the storage dtype (round-to-nearest-even);
  * v ~ N(0, 1), rounded to the storage dtype;
  * beta = sigmoid(N(0, 1)) in fp32, per (token, head);
  * log_alpha = -softplus(N(-3, 1)) in fp32, per (token, head); absent for
    DeltaNet (alpha = 1); with ``gate_channels`` one such value per key
    channel, [B, T, H, Dk] (the per-channel gate), drawn in the same place;
  * S0 ~ N(0, 0.1^2) in fp32, shape [N, H, Dv, Dk], or absent (zero state).
Draw order is fixed: [sequence lengths], q, k, v, beta logits, alpha logits,
S0.  All draws use a CPU ``torch.Generator`` so that a seed gives the same
tensors on every machine.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "GdnInputs", "make_inputs", "draw_lengths",
           "workload_inputs"]


@dataclass(frozen=True)
class Workload:
    """A named input shape. ``lengths_total`` > 0 selects a packed varlen batch."""
    name: str
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    C: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v and O
    gated: bool           # False: DeltaNet, log_alpha absent (alpha = 1)
    s0: bool              # True: random initial state, False: zero state
    seed: int
    lengths_total: int = 0
    len_lo: int = 256
    len_hi: int = 8192


# The five measured/parity workloads.  Sizes per (batch, head) unit.
WORKLOADS = {
    w.name: w for w in [
        Workload("deltanet_f32_b1_h1_t128_d16", B=1, H=1, T=128, Dk=16, Dv=16, C=16,
                 dtype="f32", gated=False, s0=False, seed=1),
        Workload("gdn_f32_b2_h4_t1024_d64", B=2, H=4, T=1024, Dk=64, Dv=64, C=64,
                 dtype="f32", gated=True, s0=True, seed=2),
        Workload("gdn_bf16_b4_h16_t4096_d128", B=4, H=16, T=4096, Dk=128, Dv=128, C=64,
                 dtype="bf16", gated=True, s0=False, seed=3),
        Workload("gdn_bf16_long_b1_h32_t32768_d128", B=1, H=32, T=32768, Dk=128, Dv=128,
                 C=64, dtype="bf16", gated=True, s0=True, seed=4),
        Workload("gdn_bf16_varlen_65536_h16_dk128_dv256", B=1, H=16, T=65536, Dk=128,
                 Dv=256, C=64, dtype="bf16", gated=True, s0=True, seed=5,
                 lengths_total=65536),
    ]
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class GdnInputs:
    """Tensors of one call (on the CPU unless drawn on a device). Token-major
    layout [B, T, H, D]."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    beta: torch.Tensor                      # [B, T, H] fp32
    log_alpha: Optional[torch.Tensor]       # [B, T, H] (or [B, T, H, Dk]) fp32, or None
    S0: Optional[torch.Tensor]              # [N, H, Dv, Dk] fp32 or None
    cu_seqlens: Optional[torch.Tensor]      # [N+1] int32 or None
    C: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    def to(self, device) -> "GdnInputs":
        f = lambda t: None if t is None else t.to(device)
        return GdnInputs(f(self.q), f(self.k), f(self.v), f(self.beta), f(self.log_alpha),
                         f(self.S0), f(self.cu_seqlens), self.C, dict(self.meta))


def draw_lengths(total: int, lo: int, hi: int, gen: torch.Generator) -> list[int]:
    """Integer lengths uniform on [lo, hi] until their sum reaches ``total``;
    the last one is shortened so that the sum is exactly ``total``."""
    lens: list[int] = []
    s = 0
    while s < total:
        n = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
        lens.append(n)
        s += n
    lens[-1] -= s - total
    return lens


def _unit_norm(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(B: int, T: int, H: int, Dk: int, Dv: int, *, dtype: str = "bf16",
                gated: bool = True, s0: bool = True, seed: int = 0, C: int = 64,
                lengths: Optional[list[int]] = None, normalize_qk: bool = True,
                beta_fill: Optional[float] = None, gate_channels: bool = False,
                device: str = "cpu") -> GdnInputs:
    """Draw one call's inputs.

    With ``lengths`` the batch is packed: B must be 1, T must equal
    sum(lengths), and ``cu_seqlens`` holds the prefix offsets.
    ``beta_fill`` replaces the drawn beta by a constant (special cases).
    ``gate_channels`` draws log_alpha per key channel, [B, T, H, Dk].
    ``device`` draws the tensors there, from that device's generator (same
    distributions, other values than a CPU draw of the same seed): for inputs
    too large to draw on the host in reasonable time."""
    g = torch.Generator(device=device).manual_seed(seed)
    td = _TORCH_DTYPE[dtype]
    if lengths is not None:
        assert B == 1 and sum(lengths) == T
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.tensor(lengths, dtype=torch.int64).cumsum(0).to(torch.int32)
        cu = cu.to(device)
        N = len(lengths)
    else:
        cu, N = None, B

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device)

    # q and k rounded as soon as they are drawn: on a device the fp32 draws of
    # the largest inputs are the bulk of the memory
    q = randn(B, T, H, Dk)
    if normalize_qk:
        q = _unit_norm(q)
    q = q.to(td).contiguous()
    k = randn(B, T, H, Dk)
    if normalize_qk:
        k = _unit_norm(k)
    k = k.to(td).contiguous()
    v = randn(B, T, H, Dv).to(td).contiguous()
    beta = torch.sigmoid(randn(B, T, H))
    if beta_fill is not None:
        beta = torch.full_like(beta, beta_fill)
    log_alpha = None
    if gated:
        la_shape = (B, T, H, Dk) if gate_channels else (B, T, H)
        log_alpha = -torch.nn.functional.softplus(randn(*la_shape) - 3.0)
    S0 = randn(N, H, Dv, Dk) * 0.1 if s0 else None
    return GdnInputs(q, k, v, beta.contiguous(), None if log_alpha is None else log_alpha.contiguous(),
                     S0, cu, C, {"dtype": dtype, "seed": seed})


def workload_inputs(name: str, seed: Optional[int] = None, gate_channels: bool = False) -> GdnInputs:
    """Inputs of a named workload; ``seed`` overrides its default seed;
    ``gate_channels`` draws its gate per key channel instead (same shapes and
    distributions otherwise)."""
    w = WORKLOADS[name]
    s = w.seed if seed is None else seed
    lengths = None
    if w.lengths_total:
        lengths = draw_lengths(w.lengths_total, w.len_lo, w.len_hi,
                               torch.Generator().manual_seed(s))
    inp = make_inputs(w.B, w.T, w.H, w.Dk, w.Dv, dtype=w.dtype, gated=w.gated, s0=w.s0,
                      seed=s, C=w.C, lengths=lengths, gate_channels=gate_channels)
    inp.meta["workload"] = name
    return inp
