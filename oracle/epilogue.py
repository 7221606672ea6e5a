"""Output epilogue of the attention block, fp64. TEST INFRASTRUCTURE ONLY.

kimi_k3 FusedKDAChunkwise page, "Output handling": after the recurrence returns
its per-head outputs, each head's feature vector is RMS-normalised (the
per-head norm named in the page's constructor summary, with a learned weight)
and then multiplied elementwise by a sigmoid output gate whose logits come from
a projection of the hidden states (the projection itself needs model weights
and stays outside; its output z is an input here):

    y[r, c] = o[r, c] / sqrt(mean_c' o[r, c']^2 + eps) * weight[c] * sigmoid(z[r, c])

The page gives no epsilon; it is an argument (the GPU binding defaults to 1e-5).
Written from that description; shares no code with the HIP path.
"""
from __future__ import annotations

import numpy as np

from . import _f64


def sigmoid(z):
    """Logistic function, evaluated without overflow for any finite z."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))                      # in (0, 1]
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def output_norm_gate(o, z, weight, *, eps: float) -> np.ndarray:
    """Per-row RMS normalisation over the last axis, channel weight, sigmoid gate (fp64).

    o, z: [..., D]; weight: [D]. Returns y with o's shape.
    """
    o, z, w = _f64(o), _f64(z), _f64(weight)
    assert o.shape == z.shape and w.shape == (o.shape[-1],)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * w * sigmoid(z)
