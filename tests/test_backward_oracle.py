"""Pins of the backward oracle (gradients of the KDA recurrence).

The gradient is checked against central finite differences of a different
forward: the chunkwise WY form (oracle.kda_chunked, fp64, derived separately
and itself pinned to the recurrence), along random directions, for every input
the FlashInfer kda_backward page lists (q, k, v, raw gate, raw beta, A_log,
dt_bias, initial state) and for the final-state adjoint. Also: the checkpoint
spacing changes nothing, packed = separate sequences, and planted slips in the
hand derivation are caught."""
import numpy as np
import pytest

import oracle
from oracle import backward as ob

SCALE = 1.0 / np.sqrt(8.0)


def problem(lengths=(5, 4), H=2, K=8, V=8, seed=0, g_std=1.0):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    return dict(q=rng.standard_normal((T, H, K)), k=rng.standard_normal((T, H, K)),
                v=rng.standard_normal((T, H, V)), g=g_std * rng.standard_normal((T, H, K)),
                beta_raw=rng.standard_normal((T, H)), A_log=rng.uniform(0, np.log(16), H),
                dt_bias=rng.uniform(-1, 1, (H, K)), h0=0.3 * rng.standard_normal((N, H, V, K)),
                cu=cu, do=rng.standard_normal((T, H, V)), dht=rng.standard_normal((N, H, V, K)))


def loss(p):
    o, ht = oracle.kda_chunked(p["q"], p["k"], p["v"], p["g"], p["beta_raw"], p["A_log"],
                               p["dt_bias"], p["cu"], scale=SCALE, chunk=4, h0=p["h0"])
    return float(np.sum(o * p["do"]) + np.sum(ht * p["dht"]))


def grads(p, fn=None):
    fn = fn or ob.kda_backward
    return fn(p["q"], p["k"], p["v"], p["g"], p["beta_raw"], p["A_log"], p["dt_bias"],
              p["cu"], p["do"], scale=SCALE, h0=p["h0"], dht=p["dht"], ckpt=3)


NAMES = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta_raw", "dbeta"),
         ("A_log", "dA_log"), ("dt_bias", "ddt_bias"), ("h0", "dh0")]


def directional_errors(p, gr, eps=1e-5, seed=1):
    rng = np.random.default_rng(seed)
    errs = {}
    for x, dx in NAMES:
        d = rng.standard_normal(p[x].shape)
        pp, pm = dict(p), dict(p)
        pp[x] = p[x] + eps * d
        pm[x] = p[x] - eps * d
        fd = (loss(pp) - loss(pm)) / (2 * eps)
        an = float(np.sum(gr[dx] * d))
        errs[dx] = abs(fd - an) / max(abs(fd), 1e-3)
    return errs


@pytest.mark.parametrize("seed,g_std", [(0, 1.0), (1, 3.0), (2, 0.1)])
def test_gradients_match_finite_differences_of_the_chunked_form(seed, g_std):
    p = problem(seed=seed, g_std=g_std)
    errs = directional_errors(p, grads(p))
    assert max(errs.values()) < 1e-6, errs


def test_checkpoint_spacing_changes_nothing():
    p = problem(lengths=(7, 1, 9), seed=3)
    a = ob.kda_backward(p["q"], p["k"], p["v"], p["g"], p["beta_raw"], p["A_log"], p["dt_bias"],
                        p["cu"], p["do"], scale=SCALE, h0=p["h0"], dht=p["dht"], ckpt=1)
    for c in (2, 4, 64):
        b = ob.kda_backward(p["q"], p["k"], p["v"], p["g"], p["beta_raw"], p["A_log"],
                            p["dt_bias"], p["cu"], p["do"], scale=SCALE, h0=p["h0"],
                            dht=p["dht"], ckpt=c)
        for key in a:
            np.testing.assert_array_equal(a[key], b[key])


def test_packed_equals_separate_sequences():
    p = problem(lengths=(6, 0, 3), seed=4)
    full = grads(p)
    cu = p["cu"]
    acc_A, acc_dt = np.zeros_like(full["dA_log"]), np.zeros_like(full["ddt_bias"])
    for n in range(3):
        s0, s1 = cu[n], cu[n + 1]
        sub = dict(p)
        for key in ("q", "k", "v", "g", "beta_raw", "do"):
            sub[key] = p[key][s0:s1]
        sub["h0"], sub["dht"] = p["h0"][n:n + 1], p["dht"][n:n + 1]
        sub["cu"] = np.array([0, s1 - s0])
        r = grads(sub)
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_array_equal(full[key][s0:s1], r[key])
        np.testing.assert_array_equal(full["dh0"][n], r["dh0"][0])
        acc_A += r["dA_log"]
        acc_dt += r["ddt_bias"]
    np.testing.assert_allclose(full["dA_log"], acc_A, rtol=1e-13)
    np.testing.assert_allclose(full["ddt_bias"], acc_dt, rtol=1e-13, atol=1e-15)


def test_empty_sequence_passes_the_final_adjoint_back():
    # no tokens: the initial state is the final state, so dh0 = dht
    p = problem(lengths=(0, 4), seed=5)
    r = grads(p)
    np.testing.assert_array_equal(r["dh0"][0], p["dht"][0])


@pytest.mark.parametrize("slip", ["no_decay_in_adjoint", "dkh_first_term_only", "db_uses_u",
                                  "dh0_before_decay", "dq_no_projection"])
def test_finite_differences_catch_planted_slips(slip):
    p = problem(seed=6)
    gr = ob_kda_backward_mutated(slip, p["q"], p["k"], p["v"], p["g"], p["beta_raw"],
                                 p["A_log"], p["dt_bias"], p["cu"], p["do"], scale=SCALE,
                                 h0=p["h0"], dht=p["dht"], ckpt=3)
    errs = directional_errors(p, gr)
    assert max(errs.values()) > 1e-3, (slip, errs)


def ob_kda_backward_mutated(slip, q, k, v, g, beta_raw, A_log, dt_bias, cu_seqlens, do, *,
                            scale, h0, dht, ckpt):
    """The oracle's reverse sweep re-run with one planted slip (test-local copy
    of the derivation's steps; each slip changes exactly one of them)."""
    lb, eps = oracle.LOWER_BOUND, oracle.L2_EPS
    cu = np.asarray(cu_seqlens)
    T, H, K = q.shape
    V = v.shape[2]
    N = len(cu) - 1
    out = {kk: np.zeros_like(vv) for kk, vv in grads_shapes(T, H, K, V, N).items()}
    for n in range(N):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        sl = slice(s0, s1)
        L = s1 - s0
        tv = ob._token_vectors(q[sl], k[sl], g[sl], beta_raw[sl], A_log, dt_bias, scale, lb, eps)
        states = [h0[n].copy()]
        for t in range(L):
            states.append(ob._step(states[-1], tv, t, v[sl])[3])
        dS = dht[n].copy()
        dqh, dkh, dal = np.zeros((L, H, K)), np.zeros((L, H, K)), np.zeros((L, H, K))
        db, dvv = np.zeros((L, H)), np.zeros((L, H, V))
        for t in reversed(range(L)):
            Sprev = states[t]
            Sp, u, w, Snew = ob._step(Sprev, tv, t, v[sl])
            kh, qh, b = tv["kh"][t], tv["qh"][t], tv["b"][t]
            dS = dS + do[sl][t][:, :, None] * qh[:, None, :]
            dqh[t] = np.einsum("hvk,hv->hk", Snew, do[sl][t])
            du = np.einsum("hvk,hk->hv", dS, kh)
            dkh[t] = np.einsum("hvk,hv->hk", dS, u)
            if slip != "dkh_first_term_only":
                dkh[t] -= np.einsum("hvk,hv->hk", Sp, b[:, None] * du)
            dvv[t] = b[:, None] * du
            db[t] = np.sum(du * (u if slip == "db_uses_u" else w), axis=1)
            dSp = dS - (b[:, None] * du)[:, :, None] * kh[:, None, :]
            dal[t] = np.sum(dSp * Sprev, axis=1)
            if slip == "dh0_before_decay" and t == 0:
                dS = dSp
            else:
                dS = dSp if slip == "no_decay_in_adjoint" else dSp * tv["al"][t][:, None, :]
        out["dh0"][n] = dS
        qs, ks, rq, rk = q[sl], k[sl], tv["rq"], tv["rk"]
        if slip == "dq_no_projection":
            out["dq"][sl] = scale * rq * dqh
        else:
            out["dq"][sl] = scale * (rq * dqh - rq ** 3 * np.sum(qs * dqh, -1, keepdims=True) * qs)
        out["dk"][sl] = rk * dkh - rk ** 3 * np.sum(ks * dkh, -1, keepdims=True) * ks
        dx = dal * tv["al"] * lb * tv["sg"] * (1.0 - tv["sg"])
        dgn = dx * tv["a"]
        out["dg"][sl] = dgn
        out["ddt_bias"] += dgn.sum(0)
        out["dA_log"] += np.sum(dgn * (g[sl] + dt_bias[None]), axis=(0, 2))
        out["dv"][sl] = dvv
        out["dbeta"][sl] = db * tv["b"] * (1.0 - tv["b"])
    return out


def grads_shapes(T, H, K, V, N):
    return dict(dq=np.zeros((T, H, K)), dk=np.zeros((T, H, K)), dg=np.zeros((T, H, K)),
                dv=np.zeros((T, H, V)), dbeta=np.zeros((T, H)), dA_log=np.zeros(H),
                ddt_bias=np.zeros((H, K)), dh0=np.zeros((N, H, V, K)))


def test_unmutated_copy_agrees():
    # the test-local copy without a slip reproduces the oracle (so each slip
    # above is the only difference)
    p = problem(seed=7)
    a = grads(p)
    b = ob_kda_backward_mutated("none", p["q"], p["k"], p["v"], p["g"], p["beta_raw"],
                                p["A_log"], p["dt_bias"], p["cu"], p["do"], scale=SCALE,
                                h0=p["h0"], dht=p["dht"], ckpt=3)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-13)
