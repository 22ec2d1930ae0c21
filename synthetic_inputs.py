"""Seeded synthetic inputs for the q4gsw linear layer.

This module is shared by the CPU oracle's tests, the GPU parity tests, the smoke
check and the benchmark.  It only draws random numbers and rounds them to the
storage dtype; it holds none of the method's arithmetic (no dequantisation, no
products, no sums), so neither side of a parity comparison depends on the other
through it.

Recipe (the same for every workload):
  * one ``torch.Generator('cpu')`` seeded with ``seed`` (default 0);
  * activations: ``randn`` in fp32, times sigma, then rounded to the activation
    dtype with round-to-nearest-even (``Tensor.to``);
  * 4-bit codes: ``randint(0, 16)`` stored one code per byte (uint8), shape [N, K];
  * scales: ``rand * (hi - lo) + lo`` in fp32, then rounded to the scale dtype,
    shape [num_groups, N] with num_groups = K / group_size;
  * token ids (embedding gather): ``randint(0, N)`` int64, shape [M];
  * low-rank adapter factors (fp32): A [r, K] = ``randn / sqrt(K)``,
    B [N, r] = ``randn * b_std`` (b_std 0.02 by default; B is nonzero so that both
    factors' gradients are exercised);
  * AdamW state (fp32, n values): param ``randn``, grad ``randn * 0.1``, first
    moment ``randn * 0.01``, second moment ``rand * 1e-3`` (zero moments at step 1);
  * draw order: activation(s) or ids first, then (codes, scales) per weight, then
    the adapter factors A, B.

Shapes are those of Llama-3.2-1B projections: MLP up/gate [8192, 2048], down
[2048, 8192], Q [2048, 2048], K and V [512, 2048]; its tied embedding / output
projection table is [128256, 2048].  Random codes and scales stand
in for trained weights (no checkpoint is used).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def draw_activation(g: torch.Generator, rows: int, cols: int, dtype: str, sigma: float = 1.0) -> torch.Tensor:
    """[rows, cols] normal samples (std sigma) rounded to ``dtype``."""
    t = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        t = t * sigma
    return t.to(DTYPES[dtype]).contiguous()


def draw_codes(g: torch.Generator, n: int, k: int) -> torch.Tensor:
    """[n, k] uniform integer codes in 0..15, one per byte."""
    return torch.randint(0, 16, (n, k), generator=g, dtype=torch.int64).to(torch.uint8).contiguous()


def draw_ids(g: torch.Generator, t: int, n: int) -> torch.Tensor:
    """[t] uniform token ids in 0..n-1 (int64)."""
    return torch.randint(0, n, (t,), generator=g, dtype=torch.int64).contiguous()


def draw_scales(g: torch.Generator, groups: int, n: int, dtype: str, lo: float, hi: float) -> torch.Tensor:
    """[groups, n] uniform samples in [lo, hi) rounded to ``dtype``."""
    t = torch.rand(groups, n, generator=g, dtype=torch.float32) * (hi - lo) + lo
    return t.to(DTYPES[dtype]).contiguous()


@dataclass
class Weight:
    codes: torch.Tensor          # uint8 [N, K]
    scales: torch.Tensor         # f16/f32 [K // group_size, N]
    group_size: int

    @property
    def N(self) -> int:
        return self.codes.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[1]

    @property
    def scale_dtype(self) -> str:
        return {torch.float16: "f16", torch.float32: "f32"}[self.scales.dtype]


@dataclass
class Case:
    name: str
    M: int
    x: Optional[torch.Tensor]            # [M, K] activation (forward / QKV input)
    d_out: Optional[torch.Tensor]        # [M, N] output gradient (backward input)
    weights: List[Weight] = field(default_factory=list)
    ids: Optional[torch.Tensor] = None   # [M] token ids (embedding gather input)
    A: Optional[torch.Tensor] = None     # [r, K] fp32 adapter factor
    B: Optional[torch.Tensor] = None     # [N, r] fp32 adapter factor

    @property
    def w(self) -> Weight:
        return self.weights[0]


def make_weight(g: torch.Generator, n: int, k: int, group_size: int, scale_dtype: str,
                s_lo: float, s_hi: float) -> Weight:
    if k % group_size:
        raise ValueError("K must be a multiple of group_size")
    codes = draw_codes(g, n, k)
    scales = draw_scales(g, k // group_size, n, scale_dtype, s_lo, s_hi)
    return Weight(codes, scales, group_size)


def make_linear(M: int, K: int, N: int, group_size: int, act_dtype: str, scale_dtype: str,
                seed: int = 0, sigma: float = 1.0, s_lo: float = 0.002, s_hi: float = 0.02,
                fwd: bool = True, bwd: bool = False, name: str = "linear") -> Case:
    """One weight with a forward activation x [M, K] and/or an output gradient d_out [M, N]."""
    g = torch.Generator().manual_seed(seed)
    x = draw_activation(g, M, K, act_dtype, sigma) if fwd else None
    d_out = draw_activation(g, M, N, act_dtype, sigma) if bwd else None
    w = make_weight(g, N, K, group_size, scale_dtype, s_lo, s_hi)
    return Case(name, M, x, d_out, [w])


def draw_factors(g: torch.Generator, rank: int, n: int, k: int, b_std: float = 0.02):
    """Low-rank adapter factors A [rank, k] ~ N(0, 1/k) and B [n, rank] ~ N(0, b_std^2), fp32."""
    A = (torch.randn(rank, k, generator=g, dtype=torch.float32) / float(k) ** 0.5).contiguous()
    B = (torch.randn(n, rank, generator=g, dtype=torch.float32) * b_std).contiguous()
    return A, B


def make_adapter(M: int, K: int, N: int, group_size: int, act_dtype: str, scale_dtype: str, rank: int,
                 seed: int = 0, sigma: float = 1.0, s_lo: float = 0.002, s_hi: float = 0.02,
                 b_std: float = 0.02, name: str = "adapter") -> Case:
    """The adapter step's inputs: x [M, K] and d_out [M, N] in one dtype, the frozen weight
    [N, K] and the factors A [rank, K], B [N, rank]."""
    g = torch.Generator().manual_seed(seed)
    x = draw_activation(g, M, K, act_dtype, sigma)
    d_out = draw_activation(g, M, N, act_dtype, sigma)
    w = make_weight(g, N, K, group_size, scale_dtype, s_lo, s_hi)
    A, B = draw_factors(g, rank, N, K, b_std)
    return Case(name, M, x, d_out, [w], A=A, B=B)


def make_adamw_state(n: int, step: int, seed: int = 0):
    """(param, grad, exp_avg, exp_avg_sq), fp32 [n]; the moments are zero at step 1."""
    g = torch.Generator().manual_seed(seed)
    p = torch.randn(n, generator=g, dtype=torch.float32)
    gr = torch.randn(n, generator=g, dtype=torch.float32) * 0.1
    if step <= 1:
        return p, gr, torch.zeros(n), torch.zeros(n)
    m = torch.randn(n, generator=g, dtype=torch.float32) * 0.01
    v = torch.rand(n, generator=g, dtype=torch.float32) * 1e-3
    return p, gr, m, v


def make_qkv(M: int, K: int, Ns: Sequence[int], group_size: int, act_dtype: str, scale_dtype: str,
             seed: int = 0, sigma: float = 1.0, s_lo: float = 0.002, s_hi: float = 0.02,
             name: str = "qkv") -> Case:
    """One activation x [M, K] and three weights [N_i, K] sharing K and group_size."""
    g = torch.Generator().manual_seed(seed)
    x = draw_activation(g, M, K, act_dtype, sigma)
    ws = [make_weight(g, n, K, group_size, scale_dtype, s_lo, s_hi) for n in Ns]
    return Case(name, M, x, None, ws)


def make_embedding(M: int, K: int, N: int, group_size: int, scale_dtype: str, seed: int = 0,
                   s_lo: float = 0.002, s_hi: float = 0.02, name: str = "embedding") -> Case:
    """M token ids and one [N, K] table (a packed linear weight serving as the embedding)."""
    g = torch.Generator().manual_seed(seed)
    ids = draw_ids(g, M, N)
    w = make_weight(g, N, K, group_size, scale_dtype, s_lo, s_hi)
    return Case(name, M, None, None, [w], ids=ids)


# The five workloads of the Llama-1B-shaped suite.
#   tiny    : fwd+bwd, M=4 K=64 N=32 gs=16, fp32 x/d_out N(0,1), fp32 scales U[0.005,0.02]
#   decode  : fwd, M=1 K=2048 N=8192 gs=32, fp16 x, fp16 scales U[0.002,0.02]
#   prefill : fwd, M=512 K=8192 N=2048 gs=128, bf16 x, fp16 scales
#   qkv     : M in {128,508,512}, K=2048, N=(2048,512,512), gs=32, fp16 x and scales
#   bwd     : d_out fp32 N(0, 0.1) [512,8192], W [8192,2048] gs=128, fp16 scales
# and the row gather of the tied embedding / output projection table:
#   embedding: M=512 uniform ids, table [128256, 2048] gs=32, fp16 scales
# and the adapter step around the frozen MLP up projection:
#   adapter : M=512 K=2048 N=8192 gs=128, bf16 x and d_out, fp16 scales, rank 16, alpha 2
WORKLOADS: Dict[str, dict] = {
    "tiny": dict(kind="linear", M=4, K=64, N=32, group_size=16, act_dtype="f32", scale_dtype="f32",
                 sigma=1.0, s_lo=0.005, s_hi=0.02, fwd=True, bwd=True),
    "decode": dict(kind="linear", M=1, K=2048, N=8192, group_size=32, act_dtype="f16",
                   scale_dtype="f16", sigma=1.0, s_lo=0.002, s_hi=0.02, fwd=True, bwd=False),
    "prefill": dict(kind="linear", M=512, K=8192, N=2048, group_size=128, act_dtype="bf16",
                    scale_dtype="f16", sigma=1.0, s_lo=0.002, s_hi=0.02, fwd=True, bwd=False),
    "qkv": dict(kind="qkv", M=512, K=2048, Ns=(2048, 512, 512), group_size=32, act_dtype="f16",
                scale_dtype="f16", sigma=1.0, s_lo=0.002, s_hi=0.02),
    "bwd": dict(kind="linear", M=512, K=2048, N=8192, group_size=128, act_dtype="f32",
                scale_dtype="f16", sigma=0.1, s_lo=0.002, s_hi=0.02, fwd=False, bwd=True),
    "embedding": dict(kind="embedding", M=512, K=2048, N=128256, group_size=32, scale_dtype="f16",
                      s_lo=0.002, s_hi=0.02),
    "adapter": dict(kind="adapter", M=512, K=2048, N=8192, group_size=128, act_dtype="bf16",
                    scale_dtype="f16", rank=16, sigma=1.0, s_lo=0.002, s_hi=0.02),
}
ADAPTER_ALPHA = 2.0

QKV_MS: Tuple[int, ...] = (128, 508, 512)


def make_workload(name: str, seed: int = 0, M: Optional[int] = None, act_dtype: Optional[str] = None) -> Case:
    """Build one of the named workloads; ``M`` and ``act_dtype`` may be overridden."""
    spec = dict(WORKLOADS[name])
    kind = spec.pop("kind")
    if M is not None:
        spec["M"] = M
    if act_dtype is not None:
        spec["act_dtype"] = act_dtype
    if kind == "qkv":
        return make_qkv(seed=seed, name=name, **spec)
    if kind == "embedding":
        return make_embedding(seed=seed, name=name, **spec)
    if kind == "adapter":
        return make_adapter(seed=seed, name=name, **spec)
    return make_linear(seed=seed, name=name, **spec)
