"""Pins of the fp64 CPU oracle against facts it did not compute itself.

Each pin is written as a function of the recurrence under test so that the
same pins can be run against copies of the oracle with a planted mistake
(test_pins_catch_planted_mistakes): every planted mistake must fail at least
one pin.

Facts used (all from the FlashInfer kda_backward page, "Supported contract",
and the per-K decay fix in the kda-neuron-kernels commit log, unless noted):
decay exp(-5*sigmoid(exp(A_log)*(g+dt_bias))) per key channel, beta =
sigmoid(beta_raw), L2-normalised q/k with eps 1e-6, scale 1/sqrt(128),
value-first state.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import kda_inputs

EPS = 1e-6
LB = -5.0


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    rms = math.sqrt(float(np.mean(b * b))) if b.size else 1.0
    return float(np.max(np.abs(a - b))) / max(rms, 1e-300)


def problem(lengths, H, K, V, seed, g_std=1.0, h0_std=None, scale=None):
    p = kda_inputs.make_prefill(lengths, H, token_dtype=torch.float32, g_std=g_std,
                                h0_std=h0_std, chunk=16, seed=seed, K=K, V=V,
                                scale=scale)
    return p


def run(rec, p, **over):
    kw = dict(q=p.q, k=p.k, v=p.v, g=p.g, beta_raw=p.beta_raw, A_log=p.A_log,
              dt_bias=p.dt_bias, cu_seqlens=p.cu_seqlens, h0=p.h0)
    kw.update(over)
    h0 = kw.pop("h0")
    return rec(kw["q"], kw["k"], kw["v"], kw["g"], kw["beta_raw"], kw["A_log"],
               kw["dt_bias"], kw["cu_seqlens"], scale=p.scale, h0=h0)


# ---- transforms written with library routines (scipy expit, numpy norm) ----

def lib_transforms(p):
    q = p.q.double().numpy()
    k = p.k.double().numpy()
    g = p.g.double().numpy()
    nq = np.linalg.norm(q, axis=-1, keepdims=True)
    nk = np.linalg.norm(k, axis=-1, keepdims=True)
    qh = q / np.sqrt(nq ** 2 + EPS) * p.scale
    kh = k / np.sqrt(nk ** 2 + EPS)
    A = np.exp(p.A_log.double().numpy())
    lam = LB * expit(A[None, :, None] * (g + p.dt_bias.double().numpy()[None]))
    b = expit(p.beta_raw.double().numpy())
    return qh, kh, lam, b


# ---- pins --------------------------------------------------------------------

def pin_t1_closed_form(rec):
    """P1: one token from a random state, closed form for state and output."""
    for K, V, H in [(128, 128, 2), (5, 3, 3)]:
        p = problem([1], H, K, V, seed=11 + K, h0_std=0.5)
        o, ht = run(rec, p)
        qh, kh, lam, b = lib_transforms(p)
        for h in range(H):
            S0 = p.h0[0, h].double().numpy()
            alpha = np.exp(lam[0, h])
            Sd = S0 * alpha[None, :]                      # decay columns (key channels)
            err = p.v[0, h].double().numpy() - Sd @ kh[0, h]
            S1 = Sd + b[0, h] * np.outer(err, kh[0, h])
            assert rel_err(ht[0, h], S1) < 1e-12
            assert rel_err(o[0, h], S1 @ qh[0, h]) < 1e-12
    # with a zero state the read-after-write output is b (k.q) v
    p = problem([1], 1, 16, 7, seed=5)
    o, ht = run(rec, p)
    qh, kh, lam, b = lib_transforms(p)
    want = b[0, 0] * float(kh[0, 0] @ qh[0, 0]) * p.v[0, 0].double().numpy()
    assert rel_err(o[0, 0], want) < 1e-12


def pin_beta_zero_pure_decay(rec):
    """P2: beta = 0 leaves only the per-key-channel decay of h0."""
    p = problem([9, 4], 2, 6, 4, seed=21, g_std=1.5, h0_std=1.0)
    p.beta_raw.fill_(-1000.0)          # sigmoid(-1000) == 0 exactly in fp64
    o, ht = run(rec, p)
    qh, kh, lam, b = lib_transforms(p)
    cu = p.cu_seqlens.tolist()
    for n in range(2):
        for h in range(2):
            S0 = p.h0[n, h].double().numpy()
            G = np.cumsum(lam[cu[n]:cu[n + 1], h], axis=0)
            for i, t in enumerate(range(cu[n], cu[n + 1])):
                St = S0 * np.exp(G[i])[None, :]
                assert rel_err(o[t, h], St @ qh[t, h]) < 1e-12
            assert rel_err(ht[n, h], S0 * np.exp(G[-1])[None, :]) < 1e-12


def pin_orthonormal_write_recall(rec):
    """P3: alpha = 1, beta = 1, orthonormal keys: exact write, recall, overwrite."""
    K, V, T = 8, 5, 10
    p = problem([T], 1, K, V, seed=31)
    keys = [0, 1, 2, 3, 0, 4, 5, 1, 6, 7]
    qidx = [3, 0, 1, 2, 0, 4, 3, 1, 7, 6]
    p.k.zero_()
    p.q.zero_()
    for t in range(T):
        p.k[t, 0, keys[t]] = 1e3
        p.q[t, 0, qidx[t]] = 1e3     # eps effect ~1e-12
    p.g.fill_(-1e4)           # sigmoid -> 0, lambda = -0, alpha = 1 exactly
    p.beta_raw.fill_(1e4)     # sigmoid -> 1 exactly
    o, ht = run(rec, p)
    v = p.v[:, 0].double().numpy()
    S = np.zeros((V, K))
    for t in range(T):
        S[:, keys[t]] = v[t]                           # latest write wins
        last = [s for s in range(t + 1) if keys[s] == qidx[t]]
        want = v[last[-1]] * p.scale if last else np.zeros(V)
        assert np.max(np.abs(o[t, 0] - want)) < 1e-9
    assert np.max(np.abs(ht[0, 0] - S)) < 1e-9


def pin_beta_one_recalls_last_write(rec):
    """beta = 1 makes the state map the newest key to its value, whatever the decay."""
    p = problem([12], 2, 16, 9, seed=41, g_std=2.0, h0_std=1.0)
    p.beta_raw.fill_(1e4)
    p.q.copy_(p.k)            # read with the key just written
    o, ht = run(rec, p)
    want = p.v.double().numpy() * p.scale
    assert np.max(np.abs(o - want)) / np.sqrt(np.mean(want ** 2)) < 1e-6


def pin_constant_key_moving_average(rec):
    """P4: one fixed key and no decay: the state stays rank one and its value
    vector follows an exponential moving average."""
    K, V, T = 12, 7, 15
    p = problem([T], 1, K, V, seed=51)
    p.k.copy_(p.k[0:1].expand_as(p.k))
    p.g.fill_(-1e4)
    o, ht = run(rec, p)
    kk = p.k[0, 0].double().numpy()
    s = float(kk @ kk)
    kh = kk / math.sqrt(s + EPS)
    k2 = s / (s + EPS)
    b = expit(p.beta_raw[:, 0].double().numpy())
    qh = p.q[:, 0].double().numpy()
    qh = qh / np.sqrt((qh * qh).sum(-1, keepdims=True) + EPS) * p.scale
    pv = np.zeros(V)
    for t in range(T):
        pv = (1.0 - b[t] * k2) * pv + b[t] * p.v[t, 0].double().numpy()
        assert rel_err(o[t, 0], pv * float(kh @ qh[t])) < 1e-11
    assert rel_err(ht[0, 0], np.outer(pv, kh)) < 1e-11


def pin_varlen_equals_separate(rec):
    """P5: a packed batch equals its sequences run one by one (bitwise)."""
    lengths = [5, 0, 11, 1, 7]
    p = problem(lengths, 3, 8, 6, seed=61, h0_std=0.3)
    o, ht = run(rec, p)
    cu = p.cu_seqlens.tolist()
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        o1, ht1 = rec(p.q[sl], p.k[sl], p.v[sl], p.g[sl], p.beta_raw[sl], p.A_log,
                      p.dt_bias, torch.tensor([0, L]), scale=p.scale,
                      h0=p.h0[n:n + 1])
        assert np.array_equal(o[sl], o1)
        assert np.array_equal(ht[n:n + 1], ht1)
    # a zero-length sequence returns its initial state unchanged
    assert np.array_equal(ht[1], p.h0[1].double().numpy())


def pin_split_chaining(rec):
    """P6: running [0,t) then [t,T) from the first part's final state equals one run."""
    p = problem([23], 2, 8, 8, seed=71, g_std=1.0, h0_std=0.2)
    o, ht = run(rec, p)
    for t in [1, 9, 22]:
        a = slice(0, t)
        b = slice(t, 23)
        oa, hta = rec(p.q[a], p.k[a], p.v[a], p.g[a], p.beta_raw[a], p.A_log, p.dt_bias,
                      torch.tensor([0, t]), scale=p.scale, h0=p.h0)
        ob, htb = rec(p.q[b], p.k[b], p.v[b], p.g[b], p.beta_raw[b], p.A_log, p.dt_bias,
                      torch.tensor([0, 23 - t]), scale=p.scale, h0=hta)
        assert np.array_equal(np.concatenate([oa, ob]), o)
        assert np.array_equal(htb, ht)


def pin_linearity(rec):
    """P9: (o, ht) are jointly linear in (v, h0)."""
    p = problem([13], 2, 8, 5, seed=81, h0_std=1.0)
    gen = torch.Generator().manual_seed(82)
    # bf16-valued v so that 2 v + v2 is exact in the oracle's fp32 input format
    p.v.copy_(p.v.bfloat16().float())
    v2 = torch.randn(p.v.shape, generator=gen).bfloat16().float()
    h02 = torch.randn(p.h0.shape, generator=gen).double()
    o1, ht1 = run(rec, p)
    o2, ht2 = run(rec, p, v=v2, h0=h02)
    o3, ht3 = run(rec, p, v=p.v * 2.0 + v2, h0=p.h0.double() * 2.0 + h02)
    assert rel_err(o3, 2 * o1 + o2) < 1e-12
    assert rel_err(ht3, 2 * ht1 + ht2) < 1e-12


def pin_scalar_recurrence(rec):
    """P10: K = V = 1 reduces to s_t = alpha s_{t-1} (1 - b kh^2) + b v kh, o = s qh."""
    T = 9
    p = problem([T], 1, 1, 1, seed=91, g_std=1.0, h0_std=1.0)
    o, ht = run(rec, p)
    s = float(p.h0[0, 0, 0, 0])
    a = math.exp(float(p.A_log[0]))
    for t in range(T):
        qv, kv = float(p.q[t, 0, 0]), float(p.k[t, 0, 0])
        kh = kv / math.sqrt(kv * kv + EPS)
        qh = qv / math.sqrt(qv * qv + EPS) * p.scale
        x = a * (float(p.g[t, 0, 0]) + float(p.dt_bias[0, 0]))
        alpha = math.exp(LB / (1.0 + math.exp(-x)))
        b = 1.0 / (1.0 + math.exp(-float(p.beta_raw[t, 0])))
        s = alpha * s * (1.0 - b * kh * kh) + b * float(p.v[t, 0, 0]) * kh
        assert abs(o[t, 0, 0] - s * qh) <= 1e-13 * max(1.0, abs(s * qh))
    assert abs(ht[0, 0, 0, 0] - s) <= 1e-13 * max(1.0, abs(s))


def pin_chunked_agrees(rec):
    """P7: the independent chunkwise WY form agrees with the recurrence."""
    cases = [([37], 1, 4, 4, 16, 0.01), ([64, 1, 30], 2, 8, 8, 32, 2.0),
             ([130], 1, 8, 6, 64, 8.0), ([17, 0, 33, 65], 2, 16, 16, 16, 2.0),
             ([70], 1, 128, 128, 64, 2.0)]
    for i, (lengths, H, K, V, C, gs) in enumerate(cases):
        p = problem(lengths, H, K, V, seed=100 + i, g_std=gs, h0_std=0.3)
        o, ht = run(rec, p)
        oc, htc = oracle.kda_chunked(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log,
                                     p.dt_bias, p.cu_seqlens, scale=p.scale,
                                     chunk=C, h0=p.h0)
        assert rel_err(oc, o) < 1e-10, (lengths, C, gs)
        assert rel_err(htc, ht) < 1e-10, (lengths, C, gs)


def pin_decode_is_recurrence(rec):
    """P8: consecutive decode steps equal each request's tokens run as one sequence."""
    B, H, K, V, steps = 3, 2, 8, 4, 4
    d = kda_inputs.make_decode(B, H, steps, seed=7, K=K, V=V)
    outs, S = oracle.kda_decode_steps(d.steps, d.state, d.A_log, d.dt_bias, scale=d.scale)
    # repack: request b's tokens become sequence b
    cat = lambda key: torch.stack([st[key] for st in d.steps], 1).reshape(
        B * steps, *d.steps[0][key].shape[1:])
    o, ht = rec(cat("q"), cat("k"), cat("v"), cat("g"), cat("beta_raw"), d.A_log,
                d.dt_bias, torch.arange(0, B * steps + 1, steps), scale=d.scale,
                h0=d.state)
    o = o.reshape(B, steps, H, V)
    for s in range(steps):
        assert np.array_equal(outs[s], o[:, s])
    assert np.array_equal(S, ht)


PINS = [pin_t1_closed_form, pin_beta_zero_pure_decay, pin_orthonormal_write_recall,
        pin_beta_one_recalls_last_write, pin_constant_key_moving_average,
        pin_varlen_equals_separate, pin_split_chaining, pin_linearity,
        pin_scalar_recurrence, pin_chunked_agrees, pin_decode_is_recurrence]


@pytest.mark.parametrize("pin", PINS, ids=[f.__name__ for f in PINS])
def test_oracle_pin(pin):
    pin(oracle.kda_recurrent)


def test_contract_constants(golden_contract):
    c = golden_contract
    assert oracle.LOWER_BOUND == c["lower_bound"]["value"]
    assert oracle.L2_EPS == c["l2_eps"]["value"]
    assert abs(1.0 / math.sqrt(128) - c["scale"]["value"]) < 1e-16
    assert c["head_dims"]["K"] == kda_inputs.K_DIM == 128
    assert c["head_dims"]["V"] == kda_inputs.V_DIM == 128
    # the workloads reproduce the page's admitted shapes
    fixed = [tuple(x) for x in c["admitted_shapes"]["fixed"]]
    assert (1, 17, 1) in fixed and (1, 4096, 32) in fixed and (1, 8192, 96) in fixed
    packed = c["admitted_shapes"]["packed"]
    assert {"lengths": [17, 33, 65], "H": 4} in packed
    assert {"lengths": kda_inputs.LARGE_VARLEN_LENGTHS, "H": 96} in packed
    # 256 MiB fp32 checkpoint at T=1024, H=4 (consistency of the page's own figure)
    assert 1024 * 4 * 128 * 128 * 4 == c["checkpoint_bytes_T1024_H4"]["value"]


def test_sigmoid_extremes_are_finite():
    p = problem([6], 1, 4, 4, seed=3)
    p.beta_raw.copy_(torch.tensor([[-1e30], [1e30], [-800.0], [800.0], [0.0], [1.0]]))
    p.g[0].fill_(1e30)
    p.g[1].fill_(-1e30)
    o, ht = run(oracle.kda_recurrent, p)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))


def test_zero_vectors_are_finite():
    """q = k = 0 gives qh = kh = 0 (eps inside the root), so the state only decays."""
    p = problem([4], 1, 4, 3, seed=4, h0_std=1.0)
    p.q.zero_()
    p.k.zero_()
    o, ht = run(oracle.kda_recurrent, p)
    assert np.all(o == 0.0)
    qh, kh, lam, b = lib_transforms(p)
    want = p.h0[0, 0].double().numpy() * np.exp(lam[:, 0].sum(0))[None, :]
    assert rel_err(ht[0, 0], want) < 1e-13


def test_chunked_intermediates_definitions():
    """The chunk form's intermediates satisfy their defining identities."""
    p = problem([40], 1, 8, 6, seed=9, g_std=2.0, h0_std=0.5)
    o, ht, saved = oracle.kda_chunked(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                      p.cu_seqlens, scale=p.scale, chunk=32, h0=p.h0,
                                      keep=True)
    it = saved[(0, 0, 0)]
    L = it["A"].shape[0]
    # (I + A) T = diag(beta)
    qh, kh, lam, b = lib_transforms(p)
    assert rel_err((np.eye(L) + it["A"]) @ it["T"], np.diag(b[:L, 0])) < 1e-13
    assert np.all(np.triu(it["A"]) == 0.0) and np.all(np.triu(it["M"], 1) == 0.0)
    assert np.all(it["Gamma_C"] <= 1.0) and np.all(np.abs(it["kg"]) <= 1.0)


# ---- planted mistakes: every one must be caught by some pin ------------------

MUTANTS = {
    "decay_per_value_row": ("S[r * K + c] *= alpha[c];", "S[r * K + c] *= alpha[r % K];"),
    "gate_sign": ("alpha[c] = exp(lower_bound * sigmoid(x));",
                  "alpha[c] = exp(lower_bound * sigmoid(-x));"),
    "delta_sign": ("double u = b * ((double)vt[r] - p[r]);",
                   "double u = b * ((double)vt[r] + p[r]);"),
    "no_scale": ("qh[c] = (double)qt[c] * rq * scale;", "qh[c] = (double)qt[c] * rq;"),
    "no_key_norm": ("kh[c] = (double)kt[c] * rk;", "kh[c] = (double)kt[c];"),
    "beta_no_sigmoid": ("double b = sigmoid((double)beta_raw[t * H + h]);",
                        "double b = (double)beta_raw[t * H + h];"),
    "A_log_no_exp": ("double a = exp((double)A_log[h]);", "double a = (double)A_log[h];"),
    "dt_bias_head_index": ("(double)dt_bias[h * K + c]", "(double)dt_bias[c]"),
    "initial_state_ignored": ("S[i] = S0 ? S0[i] : 0.0;", "S[i] = 0.0;"),
    "read_with_key": ("acc += S[r * K + c] * qh[c];", "acc += S[r * K + c] * kh[c];"),
    "lower_bound_dropped": ("exp(lower_bound * sigmoid(x))", "exp(-sigmoid(x))"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="kda_oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, name
    path_c = os.path.join(mutant_dir, name + ".c")
    path_so = os.path.join(mutant_dir, name + ".so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                    path_so, path_c, "-lm"], check=True)
    lib = oracle.load_library(path_so)

    def rec(*a, **kw):
        return oracle.kda_recurrent(*a, lib=lib, **kw)

    caught = []
    for pin in PINS:
        if pin is pin_decode_is_recurrence:
            continue      # compares the oracle with itself through another path
        try:
            pin(rec)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %s passed every pin" % name
