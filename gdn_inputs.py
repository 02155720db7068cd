"""Seeded synthetic inputs for the gated-delta SSM layer core.

This module only draws random tensors; it holds none of the method's
arithmetic.  Both sides of every parity check (the HIP library and the fp64
oracle) consume the identical fp32 arrays it returns, and the benchmark times
the same tensors.

Workloads (all fp32; "std" is a standard deviation):

* ``tiny``     1 seq x 64 tokens, 4 heads, 32x32 zero state, conv 384 ch
               (256 Q/K), d_conv 4, head_dim 32.  Seed 0.
* ``decode``   1 seq x 1 token, 32 value heads / 16 q-k heads, 128x128 state
               (std 0.05), conv 8192 ch (4096 Q/K), history std 1.  Seed 1.
* ``decode64`` 64 seq x 1 token, 48 / 16 heads, 128x128 state per head,
               conv 10240 ch read from rows 20480 apart, written 10240 apart.
               Seed 2.
* ``prefill``  1 seq x 4096 tokens, 32 / 16 heads, zero state, conv 8192 ch,
               zero history.  Seed 3.
* ``verify2``  16 seq x 2 tokens, 32 / 16 heads, 128x128 state, conv 8192 ch.
               Seed 4.

Distributions: alpha ~ N(0,1), dt ~ U(0,1), A_log ~ U(0, ln 16), beta =
sigmoid(N(0,1)), a = -exp(A_log); q, k, v, x, z, norm input ~ N(0,1) with
q, k scaled to unit length per head; conv weight std 0.25; norm weight
N(0,1).  Tensors a workload does not describe take the ``tiny`` workload's
distribution.  Draw order is fixed (see ``make_inputs``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    n_tok: int
    H: int          # value heads
    Hk: int         # query/key heads
    S: int          # state is S x S per head
    conv_dim: int
    qk_channels: int
    d_conv: int
    head_dim: int   # width of an L2 / RMS norm head
    x_stride: int   # elements between consecutive conv-input rows
    out_stride: int  # elements between consecutive conv-output rows
    state_std: float
    hist_std: float
    seed: int
    l2_eps: float = 1e-6
    norm_eps: float = 1e-6
    chunk: int = 64

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.S)

    @property
    def rows(self) -> int:
        return self.n_seq * self.n_tok

    @property
    def state_bytes(self) -> int:
        return self.n_seq * self.H * self.S * self.S * 4


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 4, 4, 32, 384, 256, 4, 32, 384, 384, 0.0, 0.0, 0),
    "decode": Workload("decode", 1, 1, 32, 16, 128, 8192, 4096, 4, 128, 8192, 8192,
                       0.05, 1.0, 1),
    "decode64": Workload("decode64", 64, 1, 48, 16, 128, 10240, 4096, 4, 128, 20480, 10240,
                         0.05, 1.0, 2),
    "prefill": Workload("prefill", 1, 4096, 32, 16, 128, 8192, 4096, 4, 128, 8192, 8192,
                        0.0, 0.0, 3),
    "verify2": Workload("verify2", 16, 2, 32, 16, 128, 8192, 4096, 4, 128, 8192, 8192,
                        0.05, 1.0, 4),
}


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Scale every vector along the last axis to unit Euclidean length."""
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(wl: Workload | str, seed: int | None = None, **overrides) -> dict:
    """Draw every input of one workload on the CPU, in a fixed order.

    Returns fp32 CPU tensors:
      alpha [rows][H], dt [H], A_log [H], a [H], beta [n_seq][n_tok][H],
      q, k [n_seq][n_tok][Hk][S], v [n_seq][n_tok][H][S], z [rows][H][head_dim],
      conv_w [C][d_conv], conv_hist [n_seq][C][d_conv-1],
      x [n_seq][n_tok][x_stride] (the conv reads columns [0, C)),
      state [n_seq][H][S (value j)][S (key i)], norm_w [head_dim],
      norm_y [rows][H][head_dim].
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if overrides:
        wl = Workload(**{**wl.__dict__, **overrides})
    gen = torch.Generator("cpu").manual_seed(wl.seed if seed is None else seed)

    def normal(*shape, std=1.0):
        t = torch.randn(*shape, generator=gen, dtype=torch.float32)
        return t * std if std != 1.0 else t

    def uniform(lo, hi, *shape):
        return lo + (hi - lo) * torch.rand(*shape, generator=gen, dtype=torch.float32)

    hd_heads = wl.H
    out = {"wl": wl}
    out["alpha"] = normal(wl.rows, wl.H)
    out["dt"] = uniform(0.0, 1.0, wl.H)
    out["A_log"] = uniform(0.0, math.log(16.0), wl.H)
    beta_logit = normal(wl.n_seq, wl.n_tok, wl.H)
    out["q"] = _unit_rows(normal(wl.n_seq, wl.n_tok, wl.Hk, wl.S))
    out["k"] = _unit_rows(normal(wl.n_seq, wl.n_tok, wl.Hk, wl.S))
    out["v"] = normal(wl.n_seq, wl.n_tok, wl.H, wl.S)
    out["z"] = normal(wl.rows, hd_heads, wl.head_dim)
    out["conv_w"] = normal(wl.conv_dim, wl.d_conv, std=0.25)
    out["conv_hist"] = normal(wl.n_seq, wl.conv_dim, wl.d_conv - 1, std=wl.hist_std) \
        if wl.hist_std > 0 else torch.zeros(wl.n_seq, wl.conv_dim, wl.d_conv - 1)
    out["x"] = normal(wl.n_seq, wl.n_tok, wl.x_stride)
    out["state"] = normal(wl.n_seq, wl.H, wl.S, wl.S, std=wl.state_std) \
        if wl.state_std > 0 else torch.zeros(wl.n_seq, wl.H, wl.S, wl.S)
    out["norm_w"] = normal(wl.head_dim)
    out["norm_y"] = normal(wl.rows, hd_heads, wl.head_dim)
    # the two pre-baked per-head inputs the layer contract asks for
    out["a"] = -torch.exp(out["A_log"])
    out["beta"] = torch.sigmoid(beta_logit)
    return out


def make_mamba2_inputs(n_seq: int, n_tok: int, H: int, G: int, P: int, N: int, seed: int,
                       state_std: float = 0.0) -> dict:
    """Seeded fp32 inputs of one Mamba-2 selective-scan layer (the chunked SSD
    scan's operands).  Draw order: dt_raw, dt_bias, A_log, D, x, B, C, state.

      dt_raw [n_seq][n_tok][H] ~ N(0, 1);  dt_bias [H] ~ U(-7, -2.3)
      A_log [H] ~ U(0, ln 16);  D [H] ~ N(0, 1)
      x [n_seq][n_tok][H][P] ~ N(0, 1);  B, C [n_seq][n_tok][G][N] ~ N(0, 1)
      state [n_seq][H][P][N] ~ N(0, state_std) (zero when state_std is 0)
    dt_min, dt_max = 1e-3, 1e-1 are returned with them.
    """
    gen = torch.Generator("cpu").manual_seed(seed)

    def normal(*shape, std=1.0):
        return (torch.randn(*shape, generator=gen) * std).float()

    def uniform(lo, hi, *shape):
        return (lo + (hi - lo) * torch.rand(*shape, generator=gen)).float()

    out = {"dt_raw": normal(n_seq, n_tok, H), "dt_bias": uniform(-7.0, -2.3, H),
           "A_log": uniform(0.0, math.log(16.0), H), "D": normal(H),
           "x": normal(n_seq, n_tok, H, P), "B": normal(n_seq, n_tok, G, N),
           "C": normal(n_seq, n_tok, G, N)}
    out["state"] = normal(n_seq, H, P, N, std=state_std) if state_std > 0 else \
        torch.zeros(n_seq, H, P, N)
    out["dt_min"], out["dt_max"] = 1e-3, 1e-1
    return out
