"""Chunkwise (WY) form of the KDA forward in fp64 numpy. TEST INFRASTRUCTURE ONLY.

The Trainium kda-neuron-kernels commit log names an exact per-channel prefill
built from 16-row sub-chunks and a WY representation
(`kda_chunk_step_exact`). The pages give no formulas for it, so the chunk
algebra below is derived from the recurrence itself:

Inside one chunk of L tokens starting from state S0 ([V,K]) write
G_t = sum_{s<=t} lambda_s (per key channel, inclusive, restarting at the chunk
start) and Gamma_t = exp(G_t). Then, with q and k already normalised,

  B[i,j] = sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])          (i > j)
  A      = diag(beta) * strictly_lower(B)
  T      = (I + A)^-1 diag(beta)
  W      = T (K * Gamma)        U_base = T V
  U      = U_base - W S0^T                          (the per-token delta writes)
  qg     = Q * Gamma            M[i,j] = sum_c q_i[c] k_j[c] exp(G_i[c]-G_j[c]) (i >= j)
  O      = qg S0^T + M U
  kg     = K * exp(G_L - G)     Gamma_C = exp(G_L)
  S_L    = S0 diag(Gamma_C) + U^T kg

Here every exponent is a difference G_i - G_j with i >= j, or a cumulative sum,
so it is <= 0 and fp64 needs no sub-chunk rescaling. The system (I + A) is
solved by plain forward substitution. Chunks restart at every sequence start;
the last chunk of a sequence may be shorter than the chunk size.

This module does not call the C recurrence: the two formulations agree only if
both are right, which is what the tests check.
"""
from __future__ import annotations

import numpy as np


def _np64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _logistic(x):
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ez = np.exp(x[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def _forward_substitution_unit_lower(Lmat, rhs):
    """Solve Lmat X = rhs for unit-lower-triangular Lmat, row by row."""
    n = Lmat.shape[0]
    X = np.zeros_like(rhs)
    for i in range(n):
        X[i] = rhs[i] - Lmat[i, :i] @ X[:i]
    return X


def chunk_step(qh, kh, v, lam, beta, S0):
    """One chunk of the WY form.

    qh, kh: [L,K] normalised (qh carries the output scale); v: [L,V];
    lam: [L,K] per-token log-decay; beta: [L]; S0: [V,K].
    Returns (o [L,V], S_L [V,K], intermediates dict).
    """
    L, K = kh.shape
    G = np.cumsum(lam, axis=0)                       # [L,K]
    Gamma = np.exp(G)
    # pairwise decay exp(G_i - G_j) for every (i, j, c); only i >= j is used
    D = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))
    lower_strict = np.tril(np.ones((L, L)), -1)
    lower_incl = np.tril(np.ones((L, L)), 0)
    Bm = np.einsum("ic,jc,ijc->ij", kh, kh, D) * lower_strict
    A = beta[:, None] * Bm
    T = _forward_substitution_unit_lower(np.eye(L) + A, np.diag(beta))
    W = T @ (kh * Gamma)
    U_base = T @ v
    U = U_base - W @ S0.T
    qg = qh * Gamma
    M = np.einsum("ic,jc,ijc->ij", qh, kh, D) * lower_incl
    O = qg @ S0.T + M @ U
    G_last = G[-1] if L > 0 else np.zeros(K)
    kg = kh * np.exp(G_last[None, :] - G)
    Gamma_C = np.exp(G_last)
    S_L = S0 * Gamma_C[None, :] + U.T @ kg
    inter = dict(G=G, A=A, T=T, W=W, U_base=U_base, qg=qg, kg=kg, M=M,
                 Gamma_C=Gamma_C, U=U)
    return O, S_L, inter


def kda_chunked(q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, *, scale,
                chunk, lower_bound=-5.0, eps=1e-6, h0=None, keep=False):
    """KDA forward by the chunkwise WY form (fp64, tiny inputs only).

    Same argument layout as the recurrence. Returns (o, ht) and, when keep is
    true, a dict {(n, j, h): intermediates} for chunk j of sequence n.
    """
    q, k, v, g = _np64(q), _np64(k), _np64(v), _np64(g)
    beta_raw, A_log, dt_bias = _np64(beta_raw), _np64(A_log), _np64(dt_bias)
    cu = np.asarray(_np64(cu_seqlens), dtype=np.int64)
    T, H, K = q.shape
    V = v.shape[2]
    N = cu.shape[0] - 1
    o = np.zeros((T, H, V))
    ht = np.zeros((N, H, V, K))
    saved = {}
    # per-token transforms (normalisation, gate, beta)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps) * scale
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    lam = lower_bound * _logistic(np.exp(A_log)[None, :, None] * (g + dt_bias[None]))
    beta = _logistic(beta_raw)
    for n in range(N):
        for h in range(H):
            S = np.zeros((V, K)) if h0 is None else _np64(h0)[n, h].copy()
            t = int(cu[n])
            j = 0
            while t < int(cu[n + 1]):
                e = min(t + chunk, int(cu[n + 1]))
                O, S, inter = chunk_step(qn[t:e, h], kn[t:e, h], v[t:e, h],
                                         lam[t:e, h], beta[t:e, h], S)
                o[t:e, h] = O
                if keep:
                    saved[(n, j, h)] = inter
                t = e
                j += 1
            ht[n, h] = S
    if keep:
        return o, ht, saved
    return o, ht
