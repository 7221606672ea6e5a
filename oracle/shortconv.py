"""Causal short depthwise convolution + SiLU on q, k, v, fp64. TEST INFRASTRUCTURE ONLY.

kimi_k3 FusedKDAChunkwise page, "CUDA-only forward and causal preprocessing":
after the Q/K/V projections each of the H*D channels is left-padded by
kernel_size - 1 along time and filtered by its own kernel (depthwise), then SiLU
is applied. For packed sequences the history restarts at every sequence start:
the W - 1 positions before it hold the sequence's carried-in conv state (the
last W - 1 inputs of its previous part) or zeros. Tap W - 1 multiplies the
current token:

    y[t, h, c] = silu( sum_{i=0}^{W-1} w[h, c, i] * x[t - (W - 1) + i, h, c] ),  silu(u) = u sigmoid(u)

The page gives no kernel size; it is an argument here. Written from that
description; shares no code with the HIP path.
"""
from __future__ import annotations

import numpy as np

from . import _f64, _i64
from .epilogue import sigmoid


def silu(u):
    u = np.asarray(u, dtype=np.float64)
    return u * sigmoid(u)


def short_conv_silu(x, w, cu_seqlens, *, state=None):
    """x: [T, H, D]; w: [H, D, W]; cu_seqlens: [N+1]; state: [N, W-1, H, D] or None.

    A conv state is W - 1 input rows, oldest first. Returns (y [T, H, D],
    final_state [N, W-1, H, D]): the final state of a sequence is its last
    W - 1 inputs, reaching back into its initial state when the sequence is
    shorter than W - 1 (an empty sequence keeps it).
    """
    x, w, cu = _f64(x), _f64(w), _i64(cu_seqlens)
    T, H, D = x.shape
    W = w.shape[2]
    N = cu.shape[0] - 1
    assert w.shape == (H, D, W) and int(cu[-1]) == T
    st = np.zeros((N, W - 1, H, D)) if state is None else _f64(state)
    assert st.shape == (N, W - 1, H, D)
    y = np.zeros((T, H, D))
    final = np.zeros((N, W - 1, H, D))
    for n in range(N):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        # history rows (W - 1 of them) followed by the sequence's own inputs
        seq = np.concatenate([st[n], x[s0:s1]], axis=0)                     # [W-1+L, H, D]
        for t in range(s1 - s0):
            win = seq[t:t + W]                                              # [W, H, D]
            pre = np.einsum("ihd,hdi->hd", win, w)
            y[s0 + t] = silu(pre)
        final[n] = seq[seq.shape[0] - (W - 1):]
    return y, final
