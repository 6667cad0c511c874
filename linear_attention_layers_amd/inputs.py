"""Seeded synthetic inputs for the GDN layer hot path.

This module only draws random tensors of the shapes and distributions of the
five workloads (tiny f32 layer, bf16 varlen prefill, 36-layer speculative
verify, 32k-token prefill, 24-layer mixed serving step).  It holds none of the
method's arithmetic; both the HIP path and the CPU oracle consume what it
returns.  Everything is drawn on the CPU with torch's seeded generator, so
the same seed gives the same bits on every machine.

Distribution readings: N(m, s2) names mean and variance (N(0, 0.25) has
standard deviation 0.5, N(0, 0.1) has 0.316); the decay gate is passed as
g = log a_t; where a workload leaves gates or initial states unstated, g =
-softplus(N(0,1)), beta = sigmoid(N(0,1)) and states ~ N(0, 0.1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass(frozen=True)
class Geometry:
    Hk: int
    Hv: int
    dk: int = 128
    dv: int = 128

    @property
    def C(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


@dataclass
class LayerBatch:
    """One GDN layer's inputs for one batch of sequences (CPU tensors)."""
    act: str                       # "f32" or "bf16": activation storage dtype
    geo: Geometry
    cu_seqlens: torch.Tensor       # int32 [nseq+1]
    x: torch.Tensor                # act [N, C]  packed q|k|v conv input
    conv_w: torch.Tensor           # f32 [C, 4]
    conv_b: Optional[torch.Tensor] # f32 [C] or None
    conv_state: torch.Tensor       # f32 [nseq, 3, C]
    has_init: torch.Tensor         # uint8 [nseq]
    g: torch.Tensor                # f32 [N, Hv]   log of the decay gate a_t
    beta: torch.Tensor             # f32 [N, Hv]
    state: torch.Tensor            # f32 [nseq, Hv, dv, dk]
    n_keep: Optional[torch.Tensor] = None   # int32 [nseq] (verify windows only)
    meta: dict = field(default_factory=dict)

    @property
    def nseq(self) -> int:
        return int(self.cu_seqlens.numel() - 1)

    @property
    def N(self) -> int:
        return int(self.x.shape[0])


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(shape, std: float, seed: int) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32) * std


def _to_act(t: torch.Tensor, act: str) -> torch.Tensor:
    if act == "f32":
        return t.to(torch.float32)
    if act == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(act)


def cu_from_lengths(lengths: List[int]) -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def make_layer(geo: Geometry, lengths: List[int], act: str, seed: int, *,
               x_std: float = 1.0, w_std: float = 0.5, bias_std: float = 0.0,
               conv_state_std: float = 1.0, state_std: float = 0.0,
               has_init=None, gate: str = "softplus",
               x_row_pad: int = 0) -> LayerBatch:
    """Draw one layer's inputs.  Tensor ids (added to seed): 1 x, 2 conv_w,
    3 conv_b, 4 conv_state, 5 g, 6 beta, 7 state.  gate = "softplus" draws
    g = -softplus(N(0,1)); gate = "uniform" draws g = -U(0.001, 0.5).
    x_row_pad > 0 allocates rows of C + x_row_pad elements and returns the
    [N, C] view (a row stride above C)."""
    C = geo.C
    cu = cu_from_lengths(lengths)
    N = int(cu[-1])
    nseq = len(lengths)
    xf = _normal((N, C + x_row_pad), x_std, seed + 1)
    x = _to_act(xf, act)[:, :C]
    w = _normal((C, 4), w_std, seed + 2)
    b = _normal((C,), bias_std, seed + 3) if bias_std > 0 else None
    cs = _normal((nseq, 3, C), conv_state_std, seed + 4)
    if gate == "softplus":
        g = -torch.nn.functional.softplus(_normal((N, geo.Hv), 1.0, seed + 5))
    elif gate == "uniform":
        u = torch.rand(N, geo.Hv, generator=_gen(seed + 5), dtype=torch.float32)
        g = -(0.001 + (0.5 - 0.001) * u)
    else:
        raise ValueError(gate)
    beta = torch.sigmoid(_normal((N, geo.Hv), 1.0, seed + 6))
    st = _normal((nseq, geo.Hv, geo.dv, geo.dk), state_std, seed + 7) if state_std > 0 \
        else torch.zeros(nseq, geo.Hv, geo.dv, geo.dk)
    if has_init is None:
        hi = torch.ones(nseq, dtype=torch.uint8)
    else:
        hi = torch.tensor([int(bool(h)) for h in has_init], dtype=torch.uint8)
    return LayerBatch(act=act, geo=geo, cu_seqlens=cu, x=x, conv_w=w, conv_b=b,
                      conv_state=cs, has_init=hi, g=g.contiguous(), beta=beta.contiguous(),
                      state=st)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

GEO_TINY = Geometry(Hk=2, Hv=4)          # C = 1024
GEO_8192 = Geometry(Hk=16, Hv=32)        # C = 8192, 2 v-heads per k-head
GEO_6144 = Geometry(Hk=16, Hv=16)        # C = 6144


def tiny_f32(seed: int = 1000) -> LayerBatch:
    """Tiny float32 layer: 1 sequence of 64 tokens, C = 1024 (2 q, 2 k, 4 v
    heads of 128), conv weights ~N(0, 0.25), bias 0, x ~N(0,1), initial
    conv_state ~N(0,1); recurrent state starts at zero (flag set, zero
    buffer)."""
    return make_layer(GEO_TINY, [64], "f32", seed, conv_state_std=1.0, state_std=0.0,
                      has_init=[1])


def varlen_lengths(seed: int = 2000, nseq: int = 8, lo: int = 128, hi: int = 2048) -> List[int]:
    return torch.randint(lo, hi + 1, (nseq,), generator=_gen(seed)).tolist()


def varlen_prefill(seed: int = 2000) -> LayerBatch:
    """bf16 varlen prefill: 8 sequences with lengths uniform in [128, 2048],
    C = 8192 (16 q, 16 k, 32 v heads of 128), even-indexed sequences carry an
    initial conv_state and recurrent state ~N(0, 0.1)."""
    lengths = varlen_lengths(seed)
    hi = [1 if s % 2 == 0 else 0 for s in range(len(lengths))]
    lb = make_layer(GEO_8192, lengths, "bf16", seed + 10, conv_state_std=math.sqrt(0.1),
                    state_std=math.sqrt(0.1), has_init=hi)
    lb.meta["workload"] = "varlen_prefill_bf16"
    return lb


def spec_verify_window(seed: int = 3000, nseq: int = 32, max_T: int = 8):
    """Window shape of the speculative-verify workload: draft lengths T_s
    uniform in 1..8 and n_keep uniform in 0..T_s, shared by all layers."""
    gen = _gen(seed)
    lengths = torch.randint(1, max_T + 1, (nseq,), generator=gen).tolist()
    n_keep = [int(torch.randint(0, T + 1, (1,), generator=gen)) for T in lengths]
    return lengths, n_keep


def spec_verify_layer(layer: int, seed: int = 3000) -> LayerBatch:
    """One layer of the 36-layer speculative-verify workload (32 sequences,
    bf16, C = 8192, all with conv_state and recurrent state ~N(0, 0.1))."""
    lengths, n_keep = spec_verify_window(seed)
    lb = make_layer(GEO_8192, lengths, "bf16", seed + 10 * (layer + 1),
                    conv_state_std=math.sqrt(0.1), state_std=math.sqrt(0.1))
    lb.n_keep = torch.tensor(n_keep, dtype=torch.int32)
    lb.meta["workload"] = "spec_verify_36L"
    return lb


def long_prefill(seed: int = 4000, T: int = 32768) -> LayerBatch:
    """Single 32768-token bf16 prefill, C = 8192, x ~N(0,1),
    log a_t ~ -U(0.001, 0.5), no initial state."""
    lb = make_layer(GEO_8192, [T], "bf16", seed, conv_state_std=0.0, state_std=0.0,
                    has_init=[0], gate="uniform")
    lb.meta["workload"] = "long_prefill_32k"
    return lb


def mixed_lengths(seed: int = 5000, n_prefill: int = 8, n_decode: int = 24,
                  lo: int = 256, hi: int = 8192) -> List[int]:
    u = torch.rand(n_prefill, generator=_gen(seed), dtype=torch.float64)
    pre = [int(round(math.exp(math.log(lo) + float(t) * (math.log(hi) - math.log(lo))))) for t in u]
    return pre + [1] * n_decode


def mixed_serving_layer(layer: int, seed: int = 5000) -> LayerBatch:
    """One layer of the mixed serving step: 8 prefill sequences with lengths
    log-uniform in [256, 8192] followed by 24 single-token decode sequences,
    C = 6144 (16 q, 16 k, 16 v heads of 128), all with initial state."""
    lengths = mixed_lengths(seed)
    lb = make_layer(GEO_6144, lengths, "bf16", seed + 10 * (layer + 1),
                    conv_state_std=math.sqrt(0.1), state_std=math.sqrt(0.1))
    lb.meta["workload"] = "mixed_serving_24L"
    lb.meta["n_prefill"] = 8
    return lb
