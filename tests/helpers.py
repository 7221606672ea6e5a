"""Shared test helpers: error metrics and tensor plumbing (no method arithmetic)."""
import math

import numpy as np
import torch


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return math.sqrt(float(np.mean(x * x))) if x.size else 0.0


def max_err_rel_rms(gpu, ref) -> float:
    """max |gpu - ref| / rms(ref): the tolerance metric, for fp32 results."""
    g, r = to_np(gpu), np.asarray(ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r))) / max(rms(r), 1e-300)


def bf16_half_ulp(x) -> np.ndarray:
    """Half the bf16 spacing at |x| (normal range): 2^(floor(log2|x|) - 8)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.exp2(e - 8.0)


def max_err_bf16_out(gpu_bf16, ref) -> float:
    """Error of a bf16-stored result beyond its own storage rounding, over rms(ref).

    If the kernel's fp32 value y has |y - ref| <= eps, its bf16 rounding b
    satisfies |b - ref| <= eps + half_ulp(b); so max(|b - ref| - half_ulp(b), 0)
    is a lower bound of the pre-rounding error, and it is 0 for an exact y.
    """
    g, r = to_np(gpu_bf16), np.asarray(ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    ex = np.maximum(np.abs(g - r) - bf16_half_ulp(g), 0.0)
    return float(np.max(ex)) / max(rms(r), 1e-300)


def raw_err(gpu, ref) -> float:
    return max_err_rel_rms(gpu, ref)


def prefill_to_device(p, dev):
    return dict(q=p.q.to(dev), k=p.k.to(dev), v=p.v.to(dev), g=p.g.to(dev),
                beta_raw=p.beta_raw.to(dev), A_log=p.A_log.to(dev), dt_bias=p.dt_bias.to(dev),
                cu_seqlens=p.cu_seqlens.to(dev),
                h0=None if p.h0 is None else p.h0.to(dev))
