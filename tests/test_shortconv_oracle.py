"""Pins of the front-end oracle (causal depthwise short conv + SiLU on q, k, v).

Definition (kimi_k3 FusedKDAChunkwise page, "CUDA-only forward and causal
preprocessing"): per channel, left-pad by W-1, filter, then SiLU; history
restarts at each packed sequence start (carried-in state or zeros). Pins come
from hand arithmetic, degenerate filters and chaining identities."""
import math

import numpy as np
import pytest

import oracle
from oracle.shortconv import silu


def sig(u):
    return 1.0 / (1.0 + math.exp(-u))


def test_worked_example_by_hand():
    # W = 2, taps [0.5, 1]: pre-activations 1*1, 2 + 0.5*1, 3 + 0.5*2 = 1, 2.5, 4
    x = np.array([1.0, 2.0, 3.0]).reshape(3, 1, 1)
    w = np.array([0.5, 1.0]).reshape(1, 1, 2)
    y, f = oracle.short_conv_silu(x, w, np.array([0, 3]))
    np.testing.assert_allclose(y.ravel(), [1 * sig(1), 2.5 * sig(2.5), 4 * sig(4)], rtol=1e-15)
    assert f.ravel().tolist() == [3.0]


def test_degenerate_filters():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((11, 2, 5))
    cu = np.array([0, 11])
    # current-tap-only filter of ones: plain SiLU
    w = np.zeros((2, 5, 4)); w[:, :, 3] = 1.0
    np.testing.assert_allclose(oracle.short_conv_silu(x, w, cu)[0], x * (1 / (1 + np.exp(-x))), rtol=1e-14)
    # oldest-tap-only filter: SiLU of the input three steps back, zero before the start
    w = np.zeros((2, 5, 4)); w[:, :, 0] = 1.0
    y, _ = oracle.short_conv_silu(x, w, cu)
    np.testing.assert_allclose(y[3:], silu(x[:-3]), rtol=1e-14)
    assert np.all(y[:3] == 0.0)
    # W = 1 is a per-channel scale
    w1 = rng.uniform(-2, 2, (2, 5, 1))
    np.testing.assert_allclose(oracle.short_conv_silu(x, w1, cu)[0], silu(x * w1[:, :, 0]), rtol=1e-14)


def test_current_tap_weight_scales_the_input():
    # a filter with only the current tap, of weight a, gives silu(a x) per token
    x = np.linspace(-3, 3, 8).reshape(8, 1, 1)
    w = np.array([0.0, 0.0, 0.0, 2.5]).reshape(1, 1, 4)
    y, _ = oracle.short_conv_silu(x, w, np.array([0, 8]))
    np.testing.assert_allclose(y.ravel(), [2.5 * v * sig(2.5 * v) for v in x.ravel()], rtol=1e-14)


def test_packed_equals_separate_and_chaining():
    rng = np.random.default_rng(4)
    lens = [5, 0, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((int(cu[-1]), 3, 4))
    w = rng.standard_normal((3, 4, 4))
    st = rng.standard_normal((4, 3, 3, 4))   # [N, W-1, H, D]
    y, f = oracle.short_conv_silu(x, w, cu, state=st)
    for n in range(4):
        ys, fs = oracle.short_conv_silu(x[cu[n]:cu[n + 1]], w, np.array([0, lens[n]]), state=st[n:n + 1])
        np.testing.assert_array_equal(y[cu[n]:cu[n + 1]], ys)
        np.testing.assert_array_equal(f[n], fs[0])
    # the empty sequence keeps its state; the 2-token one keeps its last state row
    np.testing.assert_array_equal(f[1], st[1])
    np.testing.assert_array_equal(f[2][0], st[2][2])
    np.testing.assert_array_equal(f[2][1:], x[cu[2]:cu[3]])
    # splitting a sequence and passing the final state on gives the same outputs
    a, b = x[cu[3]:cu[3] + 4], x[cu[3] + 4:cu[4]]
    ya, fa = oracle.short_conv_silu(a, w, np.array([0, 4]), state=st[3:4])
    yb, fb = oracle.short_conv_silu(b, w, np.array([0, 5]), state=fa)
    np.testing.assert_array_equal(np.concatenate([ya, yb]), y[cu[3]:cu[4]])
    np.testing.assert_array_equal(fb[0], f[3])


def test_matches_library_depthwise_conv1d():
    # one sequence from zero history is the page's own recipe: channels-first
    # layout, left pad of W - 1, grouped (depthwise) conv1d, then SiLU
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    T, H, D, W = 37, 3, 8, 4
    x = rng.standard_normal((T, H, D))
    w = rng.standard_normal((H, D, W))
    xt = torch.from_numpy(x).reshape(T, H * D).T.unsqueeze(0)            # [1, HD, T]
    ref = F.silu(F.conv1d(F.pad(xt, (W - 1, 0)), torch.from_numpy(w).reshape(H * D, 1, W),
                          groups=H * D))
    ref = ref[0].T.reshape(T, H, D).numpy()
    y, f = oracle.short_conv_silu(x, w, np.array([0, T]))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(f[0], x[T - 3:])


def test_silu_values():
    assert silu(0.0) == 0.0
    np.testing.assert_allclose(silu(40.0), 40.0, rtol=1e-15)
    assert abs(silu(-40.0)) < 1e-15
    np.testing.assert_allclose(silu(1.0), 1 / (1 + math.exp(-1)), rtol=1e-15)


@pytest.mark.parametrize("mistake", ["no_activation", "right_padded", "tap_order", "no_restart"])
def test_pins_catch_planted_mistakes(mistake):
    def bad(x, w, cu, *, state=None):
        x, w, cu = np.asarray(x, float), np.asarray(w, float), np.asarray(cu)
        T, H, D = x.shape
        W = w.shape[2]
        N = len(cu) - 1
        st = np.zeros((N, W - 1, H, D)) if state is None else np.asarray(state, float)
        y = np.zeros_like(x)
        fin = np.zeros((N, W - 1, H, D))
        for n in range(N):
            s0, s1 = cu[n], cu[n + 1]
            hist = st[n]
            if mistake == "no_restart" and s0 > 0:
                hist = x[max(0, s0 - (W - 1)):s0]
                if hist.shape[0] < W - 1:
                    hist = np.concatenate([np.zeros((W - 1 - hist.shape[0], H, D)), hist])
            seq = np.concatenate([hist, x[s0:s1]])
            if mistake == "right_padded":
                seq = np.concatenate([x[s0:s1], np.zeros((W - 1, H, D))])
            for t in range(s1 - s0):
                ww = w[:, :, ::-1] if mistake == "tap_order" else w
                pre = np.einsum("ihd,hdi->hd", seq[t:t + W], ww)
                y[s0 + t] = pre if mistake == "no_activation" else silu(pre)
            fin[n] = seq[seq.shape[0] - (W - 1):]
        return y, fin

    real = oracle.short_conv_silu
    failures = 0
    try:
        oracle.short_conv_silu = bad
        for pin in (test_worked_example_by_hand, test_degenerate_filters, test_matches_library_depthwise_conv1d,
                    test_packed_equals_separate_and_chaining):
            try:
                pin()
            except AssertionError:
                failures += 1
    finally:
        oracle.short_conv_silu = real
    assert failures >= 1, mistake
