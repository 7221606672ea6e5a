"""Seeded synthetic inputs for the KDA forward workloads.

This module is shared by the tests, the benchmark and the smoke check. It draws
random tensors and nothing else: it holds none of the method's arithmetic (no
normalisation, gating, decay or recurrence), so the CPU oracle and the HIP path
both receive exactly the same bits and never share computation.

Workloads follow the shapes the FlashInfer `kda_backward` page admits
("Supported contract", the admitted-shape list) and the value distributions
stated for the five standard configurations:

  small      : B=1, T=17, H=1, everything fp32, chunk 16, zero initial state
  varlen     : packed lengths [17, 33, 65], H=4, bf16 q/k/v, chunk 32,
               initial states ~ N(0, 0.1^2)
  prefill    : B=1, T=4096, H=32, bf16 q/k/v, g ~ N(0, 2^2), chunk 64
  large      : B=1, T=8192, H=96, bf16, g ~ N(0, 2^2), chunk 64, h0 ~ N(0, 0.1^2)
  large_varlen: packed lengths [1300, 547, 2048, 963, 271, 3063], H=96, as large
  packed_8x1024: eight packed sequences of 1024 tokens, H=96, as large
  decode     : 256 requests, H=32, 64 consecutive T=1 steps, state ~ N(0, 0.1^2)
  epilogue   : output-gate logits ~ N(0, 2^2) in the token dtype and an output-norm
               weight ~ U(0.5, 1.5) (stand-ins for the model's projection and weight)
  front end  : projection outputs ~ N(0, 1) in the token dtype, conv weights
               ~ U(-1/sqrt(W), 1/sqrt(W)), carried-in conv states ~ N(0, 1)

"N(0, s)" in the configuration text is read as standard deviation s.
All values are drawn in fp32 from a CPU `torch.Generator` seeded with the
workload's seed, in the fixed order q, k, v, g, beta_raw, A_log, dt_bias, h0,
then cast to bf16 where the workload says so.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

K_DIM = 128
V_DIM = 128
LN16 = math.log(16.0)


@dataclass
class PrefillInputs:
    name: str
    q: torch.Tensor          # [T, H, K]  bf16 or fp32 (CPU)
    k: torch.Tensor          # [T, H, K]
    v: torch.Tensor          # [T, H, V]
    g: torch.Tensor          # [T, H, K]  fp32 raw gate
    beta_raw: torch.Tensor   # [T, H]     fp32
    A_log: torch.Tensor      # [H]        fp32
    dt_bias: torch.Tensor    # [H, K]     fp32
    cu_seqlens: torch.Tensor  # [N+1]     int64
    h0: Optional[torch.Tensor]  # [N, H, V, K] fp32 or None
    chunk: int
    scale: float
    lower_bound: float = -5.0

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.numel() - 1)


@dataclass
class DecodeInputs:
    name: str
    state: torch.Tensor       # [B, H, V, K] fp32 (initial state)
    A_log: torch.Tensor       # [H]
    dt_bias: torch.Tensor     # [H, K]
    steps: List[dict] = field(default_factory=list)  # each: q,k,v [B,H,*] bf16; g [B,H,K]; beta_raw [B,H]
    scale: float = 1.0 / math.sqrt(128.0)
    lower_bound: float = -5.0


def _randn(gen, shape, std=1.0):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _uniform(gen, shape, lo, hi):
    return torch.rand(*shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo


def make_prefill(lengths, H, *, token_dtype=torch.bfloat16, g_std=1.0, h0_std=None,
                 chunk=64, seed=0, K=K_DIM, V=V_DIM, name="custom",
                 scale=None) -> PrefillInputs:
    """Draw one packed-varlen prefill problem.

    lengths : per-sequence token counts (zeros allowed); packed along T.
    h0_std  : None for a zero initial state, else the std of the fp32 h0.
    """
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    N = len(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int64)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    q = _randn(gen, (T, H, K))
    k = _randn(gen, (T, H, K))
    v = _randn(gen, (T, H, V))
    g = _randn(gen, (T, H, K), g_std)
    beta_raw = _randn(gen, (T, H))
    A_log = _uniform(gen, (H,), 0.0, LN16)
    dt_bias = _uniform(gen, (H, K), -1.0, 1.0)
    h0 = None if h0_std is None else _randn(gen, (N, H, V, K), h0_std)
    if token_dtype != torch.float32:
        q, k, v = q.to(token_dtype), k.to(token_dtype), v.to(token_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    return PrefillInputs(name, q, k, v, g, beta_raw, A_log, dt_bias, cu, h0,
                         int(chunk), float(scale))


def make_decode(B, H, n_steps, *, seed=0, state_std=0.1, K=K_DIM, V=V_DIM,
                name="custom") -> DecodeInputs:
    """Draw a batched-decode problem: an initial state and n_steps token sets."""
    gen = torch.Generator().manual_seed(int(seed))
    A_log = _uniform(gen, (H,), 0.0, LN16)
    dt_bias = _uniform(gen, (H, K), -1.0, 1.0)
    state = _randn(gen, (B, H, V, K), state_std)
    steps = []
    for _ in range(int(n_steps)):
        q = _randn(gen, (B, H, K)).to(torch.bfloat16)
        k = _randn(gen, (B, H, K)).to(torch.bfloat16)
        v = _randn(gen, (B, H, V)).to(torch.bfloat16)
        g = _randn(gen, (B, H, K))
        beta_raw = _randn(gen, (B, H))
        steps.append(dict(q=q, k=k, v=v, g=g, beta_raw=beta_raw))
    return DecodeInputs(name, state, A_log, dt_bias, steps, 1.0 / math.sqrt(K))


# ---- the named standard workloads --------------------------------------------

LARGE_VARLEN_LENGTHS = [1300, 547, 2048, 963, 271, 3063]


def small():
    return make_prefill([17], 1, token_dtype=torch.float32, chunk=16, seed=1000,
                        name="small T=17 H=1 fp32 C=16")


def varlen():
    return make_prefill([17, 33, 65], 4, h0_std=0.1, chunk=32, seed=1001,
                        name="varlen [17,33,65] H=4 bf16 C=32")


def prefill_4k():
    return make_prefill([4096], 32, g_std=2.0, chunk=64, seed=1002,
                        name="prefill T=4096 H=32 bf16 C=64")


def large():
    return make_prefill([8192], 96, g_std=2.0, h0_std=0.1, chunk=64, seed=1003,
                        name="prefill T=8192 H=96 bf16 C=64")


def large_varlen():
    return make_prefill(LARGE_VARLEN_LENGTHS, 96, g_std=2.0, h0_std=0.1, chunk=64,
                        seed=1013, name="prefill varlen[1300..3063] H=96 bf16 C=64")


def packed_8x1024():
    return make_prefill([1024] * 8, 96, g_std=2.0, h0_std=0.1, chunk=64, seed=1014,
                        name="prefill packed 8x1024 H=96 bf16 C=64")


def decode(n_steps=64):
    return make_decode(256, 32, n_steps, seed=1004,
                       name="decode B=256 H=32 T=1")


def make_epilogue(shape, *, token_dtype=torch.bfloat16, z_std=2.0, seed=0, D=V_DIM):
    """Synthetic inputs of the output epilogue: gate logits z (shape `shape`, last
    axis D, in the token dtype, ~ N(0, z_std)) and the norm weight [D] fp32 ~ U(0.5, 1.5).
    The gate projection and the trained norm weight need model weights; these stand in."""
    gen = torch.Generator().manual_seed(int(seed))
    z = _randn(gen, tuple(shape), z_std).to(token_dtype)
    w = _uniform(gen, (D,), 0.5, 1.5)
    return z, w


def make_short_conv(lengths, H, W, *, token_dtype=torch.bfloat16, with_state=True, seed=0,
                    D=K_DIM):
    """Synthetic inputs of the q/k/v front end for one of q, k, v: a projection
    output x [T, H, D] ~ N(0, 1) in the token dtype, conv weights [H, D, W] fp32 ~
    U(-1/sqrt(W), 1/sqrt(W)) (the default init range of a depthwise conv1d with
    W taps), and carried-in conv states [N, W-1, H, D] ~ N(0, 1) in the token
    dtype (or None). Returns (x, w, cu_seqlens, state)."""
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(n) for n in lengths]
    T, N = sum(lengths), len(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int64)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    x = _randn(gen, (T, H, D)).to(token_dtype)
    bound = 1.0 / math.sqrt(W)
    w = _uniform(gen, (H, D, W), -bound, bound)
    state = _randn(gen, (N, W - 1, H, D)).to(token_dtype) if with_state else None
    return x, w, cu, state
