"""Gradients of the KDA recurrence, fp64 numpy. TEST INFRASTRUCTURE ONLY.

The FlashInfer kda_backward page ("Supported contract") defines the training
backward as the gradient of the frozen recurrence with respect to q, k, v, the
raw gate g, raw beta, A_log, dt_bias and the initial state, given the output
adjoint. The kda-neuron-kernels commit log asks for the gradient of the exact
forward (its chunked backward must equal the recurrent one). This module writes
that gradient out by reverse-mode differentiation of the recurrence, one token
at a time, derived by hand from the forward (notation of kda_recurrent):

  forward, per token t (S is [V, K], value-first):
    qh = scale q / sqrt(|q|^2 + eps)        kh = k / sqrt(|k|^2 + eps)
    x  = exp(A_log) (g + dt_bias)           alpha = exp(lb sigmoid(x))
    b  = sigmoid(beta_raw)
    S' = S diag(alpha)     u = b (v - S' kh)     S <- S' + u kh^T     o = S qh

  reverse, with dS the adjoint of the state after token t:
    dS  += do qh^T               dqh = S^T do
    du   = dS kh                 dkh = dS^T u - b S'^T du
    dv   = b du                  db  = du . (v - S' kh)
    dS'  = dS - b du kh^T        dalpha = column sums of dS' * S_prev
    dS   = dS' diag(alpha)       (the adjoint of the state before token t)

  then the elementwise chains back to the raw inputs:
    dq = scale (r dqh - r^3 (q . dqh) q)   with r = 1/sqrt(|q|^2 + eps); dk alike (no scale)
    dx = dalpha alpha lb sigmoid(x) (1 - sigmoid(x))
    dg = dx exp(A_log)     ddt_bias = sum over tokens of dg     dA_log = sum dg (g + dt_bias)
    dbeta_raw = db b (1 - b)        dh0 = dS after the first token (in reverse order)

The state before each token is needed in the reverse sweep. The states are
recomputed from a copy kept every `ckpt` tokens (the forward is deterministic,
so the recomputed states are the very values of the first pass); this only
bounds memory and changes no arithmetic. Shares no code with the HIP path.
"""
from __future__ import annotations

import numpy as np

from . import LOWER_BOUND, L2_EPS, _f64, _i64


def _sig(x):
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ez = np.exp(x[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def _token_vectors(q, k, g, beta_raw, A_log, dt_bias, scale, lb, eps):
    """Per-token transforms for a block of tokens [L, H, *]."""
    rq = 1.0 / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    rk = 1.0 / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    a = np.exp(A_log)[None, :, None]
    x = a * (g + dt_bias[None])
    sg = _sig(x)
    al = np.exp(lb * sg)
    b = _sig(beta_raw)
    return dict(qh=scale * q * rq, kh=k * rk, rq=rq, rk=rk, a=a, x=x, sg=sg, al=al, b=b)


def _step(S, tv, t, v):
    """One forward token on S [H, V, K]; returns (S', u, v - S' kh, S_new)."""
    Sp = S * tv["al"][t][:, None, :]
    w = v[t] - np.einsum("hvk,hk->hv", Sp, tv["kh"][t])
    u = tv["b"][t][:, None] * w
    return Sp, u, w, Sp + u[:, :, None] * tv["kh"][t][:, None, :]


def kda_backward(q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, do, *,
                 scale: float, lower_bound: float = LOWER_BOUND, eps: float = L2_EPS,
                 h0=None, dht=None, ckpt: int = 64):
    """Gradients of the recurrence for the output adjoint `do` [T, H, V] and an
    optional final-state adjoint `dht` [N, H, V, K] (zero if None).

    Returns a dict of fp64 arrays: dq, dk, dg [T,H,K]; dv [T,H,V]; dbeta [T,H];
    dA_log [H]; ddt_bias [H,K]; dh0 [N,H,V,K].
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    beta_raw, A_log, dt_bias, do = _f64(beta_raw), _f64(A_log), _f64(dt_bias), _f64(do)
    cu = _i64(cu_seqlens)
    T, H, K = q.shape
    V = v.shape[2]
    N = cu.shape[0] - 1
    lb = float(lower_bound)
    out = dict(dq=np.zeros((T, H, K)), dk=np.zeros((T, H, K)), dg=np.zeros((T, H, K)),
               dv=np.zeros((T, H, V)), dbeta=np.zeros((T, H)), dA_log=np.zeros(H),
               ddt_bias=np.zeros((H, K)), dh0=np.zeros((N, H, V, K)))
    h0a = np.zeros((N, H, V, K)) if h0 is None else _f64(h0)
    dhta = np.zeros((N, H, V, K)) if dht is None else _f64(dht)
    for n in range(N):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        L = s1 - s0
        sl = slice(s0, s1)
        tv = _token_vectors(q[sl], k[sl], g[sl], beta_raw[sl], A_log, dt_bias, scale, lb, eps)
        vv, dov = v[sl], do[sl]
        # forward: keep the state before every ckpt-th token
        marks = {}
        S = h0a[n].copy()
        for t in range(L):
            if t % ckpt == 0:
                marks[t] = S.copy()
            S = _step(S, tv, t, vv)[3]
        dS = dhta[n].copy()
        dqh = np.zeros((L, H, K))
        dkh = np.zeros((L, H, K))
        dal = np.zeros((L, H, K))
        db = np.zeros((L, H))
        dvv = np.zeros((L, H, V))
        for c0 in reversed(range(0, L, ckpt)):
            c1 = min(c0 + ckpt, L)
            prev = [marks[c0]]                    # state before each token of the block
            for t in range(c0, c1 - 1):
                prev.append(_step(prev[-1], tv, t, vv)[3])
            for t in reversed(range(c0, c1)):
                Sprev = prev[t - c0]
                Sp, u, w, Snew = _step(Sprev, tv, t, vv)
                kh, qh, b = tv["kh"][t], tv["qh"][t], tv["b"][t]
                dS = dS + dov[t][:, :, None] * qh[:, None, :]
                dqh[t] = np.einsum("hvk,hv->hk", Snew, dov[t])
                du = np.einsum("hvk,hk->hv", dS, kh)
                dkh[t] = (np.einsum("hvk,hv->hk", dS, u)
                          - np.einsum("hvk,hv->hk", Sp, b[:, None] * du))
                dvv[t] = b[:, None] * du
                db[t] = np.sum(du * w, axis=1)
                dSp = dS - (b[:, None] * du)[:, :, None] * kh[:, None, :]
                dal[t] = np.sum(dSp * Sprev, axis=1)
                dS = dSp * tv["al"][t][:, None, :]
        out["dh0"][n] = dS
        # elementwise chains to the raw inputs
        qs, ks = q[sl], k[sl]
        rq, rk = tv["rq"], tv["rk"]
        out["dq"][sl] = scale * (rq * dqh - rq ** 3 * np.sum(qs * dqh, axis=-1, keepdims=True) * qs)
        out["dk"][sl] = rk * dkh - rk ** 3 * np.sum(ks * dkh, axis=-1, keepdims=True) * ks
        dx = dal * tv["al"] * lb * tv["sg"] * (1.0 - tv["sg"])
        dgn = dx * tv["a"]
        out["dg"][sl] = dgn
        out["ddt_bias"] += np.sum(dgn, axis=0)
        out["dA_log"] += np.sum(dgn * (g[sl] + dt_bias[None]), axis=(0, 2))
        out["dv"][sl] = dvv
        out["dbeta"][sl] = db * tv["b"] * (1.0 - tv["b"])
    return out
