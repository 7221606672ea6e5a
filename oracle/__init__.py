"""CPU oracle for the KDA forward (fp64). TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It never imports the HIP package and shares no code with
it; both sides take their inputs from the seeded generators in kda_inputs.py.

Formulations here:
  * `kda_recurrent` — the token-by-token recurrence (kda_oracle.c), the plain
    definition of what the method computes;
  * `kda_chunked`   — the chunkwise WY form (chunked.py), derived separately and
    used to pin the recurrence and to check the GPU's intra-chunk stage;
  * `output_norm_gate` — the output epilogue (epilogue.py): per-head RMS norm
    and sigmoid output gate applied to the recurrence's outputs;
  * `short_conv_silu` — the front end (shortconv.py): causal depthwise short
    convolution + SiLU applied to q, k, v before the recurrence;
  * `kda_backward` — the gradients of the recurrence (backward.py) for an
    output adjoint and an optional final-state adjoint.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

LOWER_BOUND = -5.0   # gate floor fixed by the FlashInfer kda_backward contract
L2_EPS = 1e-6        # epsilon of the q/k L2 normalisation, same contract


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc -O2 -fopenmp (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Bind the oracle's C entry points in the shared library at `path`."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_kda_recurrent.restype = ctypes.c_int
    lib.oracle_kda_recurrent.argtypes = [
        P, P, P, P, P, P, P,
        ctypes.c_double, ctypes.c_double, ctypes.c_double,
        P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        P, P, P, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f32(x) -> np.ndarray:
    """Exact upcast of a bf16/fp32 torch tensor or array to a C-contiguous fp32 array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype != torch.float32:
                x = x.to(torch.float32)      # bf16 -> fp32 is exact
            return np.ascontiguousarray(x.numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").to(torch.float64)
            return np.ascontiguousarray(x.numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu").to(torch.int64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def kda_recurrent(q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, *,
                  scale: float, lower_bound: float = LOWER_BOUND,
                  eps: float = L2_EPS, h0=None, nthreads: int = 0,
                  lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token KDA forward in fp64.

    q, k, g: [T,H,K]; v: [T,H,V]; beta_raw: [T,H]; A_log: [H]; dt_bias: [H,K];
    cu_seqlens: [N+1] int64; h0: [N,H,V,K] or None.
    Returns (o [T,H,V] fp64, ht [N,H,V,K] fp64). `lib` selects another build
    of kda_oracle.c (used by the tests that plant mistakes in a copy of it).
    """
    lib = _load() if lib is None else lib
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    beta_raw, A_log, dt_bias = _f32(beta_raw), _f32(A_log), _f32(dt_bias)
    cu = _i64(cu_seqlens)
    T, H, K = q.shape
    V = v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T, H, K) and g.shape == (T, H, K) and v.shape[:2] == (T, H)
    assert beta_raw.shape == (T, H) and A_log.shape == (H,) and dt_bias.shape == (H, K)
    assert N >= 0 and int(cu[-1]) == T
    h0a = None
    if h0 is not None:
        h0a = _f64(h0)
        assert h0a.shape == (N, H, V, K)
    o = np.zeros((T, H, V), dtype=np.float64)
    ht = np.zeros((N, H, V, K), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.oracle_kda_recurrent(
        ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta_raw), ptr(A_log), ptr(dt_bias),
        float(scale), float(lower_bound), float(eps),
        ptr(cu), N, H, K, V, ptr(h0a), ptr(o), ptr(ht), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_kda_recurrent failed with code %d" % rc)
    return o, ht


def kda_decode_steps(steps, state, A_log, dt_bias, *, scale: float,
                     lower_bound: float = LOWER_BOUND, eps: float = L2_EPS,
                     nthreads: int = 0):
    """Consecutive T=1 steps over B independent requests (fp64 state carried).

    steps: list of dicts with q,k,v [B,H,*], g [B,H,K], beta_raw [B,H].
    Returns (list of o [B,H,V] fp64, final state [B,H,V,K] fp64).
    A decode step is the recurrence with every sequence of length one.
    """
    S = _f64(state)
    B = S.shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    outs = []
    for st in steps:
        o, S = kda_recurrent(st["q"], st["k"], st["v"], st["g"], st["beta_raw"],
                             A_log, dt_bias, cu, scale=scale,
                             lower_bound=lower_bound, eps=eps, h0=S,
                             nthreads=nthreads)
        outs.append(o)
    return outs, S


from .chunked import kda_chunked  # noqa: E402  (pure numpy, no library)
from .epilogue import output_norm_gate  # noqa: E402  (pure numpy, no library)
from .shortconv import short_conv_silu  # noqa: E402  (pure numpy, no library)
from .backward import kda_backward  # noqa: E402  (pure numpy, no library)

__all__ = ["build", "kda_recurrent", "kda_decode_steps", "kda_chunked",
           "output_norm_gate", "short_conv_silu", "kda_backward", "max_threads", "LOWER_BOUND", "L2_EPS"]
