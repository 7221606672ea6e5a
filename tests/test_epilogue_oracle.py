"""Pins of the output-epilogue oracle (per-head RMS norm + sigmoid output gate).

The definition (kimi_k3 FusedKDAChunkwise page, "Output handling"):
y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z), per row over the head
dimension. Each pin below is fixed by arithmetic, not by re-running the oracle's
formula: a hand-worked example, invariances and closed forms.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.epilogue import sigmoid


def test_worked_example_by_hand():
    # row 0: mean of squares (1 + 4 + 4 + 16) / 4 = 25/4, rms 5/2, gate ~1
    # row 1: mean of squares (9 + 16) / 4 = 25/4 again; normalised [1.2, 0, 0, 1.6],
    #        weight [2, 1, 1, 1/2] -> [2.4, 0, 0, 0.8], gates [1/2, 1/2, 3/4, 1/4]
    o = np.array([[1.0, 2.0, 2.0, 4.0], [3.0, 0.0, 0.0, 4.0]])
    z = np.array([[40.0, 40.0, 40.0, 40.0], [0.0, 0.0, math.log(3.0), -math.log(3.0)]])
    w1 = np.ones(4)
    y0 = oracle.output_norm_gate(o[:1], z[:1], w1, eps=0.0)
    np.testing.assert_allclose(y0[0], [0.4, 0.8, 0.8, 1.6], rtol=1e-15, atol=0)
    y1 = oracle.output_norm_gate(o[1:], z[1:], np.array([2.0, 1.0, 1.0, 0.5]), eps=0.0)
    np.testing.assert_allclose(y1[0], [1.2, 0.0, 0.0, 0.2], rtol=1e-15, atol=1e-300)


def test_scale_and_sign_invariance():
    rng = np.random.default_rng(11)
    o = rng.standard_normal((5, 128))
    z = rng.standard_normal((5, 128))
    w = rng.uniform(0.5, 1.5, 128)
    y = oracle.output_norm_gate(o, z, w, eps=0.0)
    for c in (1e-3, 7.0, 1e4):
        np.testing.assert_allclose(oracle.output_norm_gate(c * o, z, w, eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(oracle.output_norm_gate(-o, z, w, eps=0.0), -y, rtol=0, atol=0)


def test_rms_of_normalised_rows():
    # unit weight, gate saturated at 1: each output row has rms sqrt(ms / (ms + eps))
    rng = np.random.default_rng(12)
    o = rng.standard_normal((6, 128)) * np.array([1e-3, 0.1, 1, 3, 10, 100])[:, None]
    eps = 0.3
    y = oracle.output_norm_gate(o, np.full_like(o, 60.0), np.ones(128), eps=eps)
    ms = np.mean(o * o, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_constant_rows_and_channel_weight():
    # o = c * ones: normalised value c / sqrt(c^2 + eps) in every channel; a one-hot
    # weight keeps only its channel
    c, eps = 0.5, 0.25
    o = np.full((1, 128), c)
    w = np.zeros(128)
    w[37] = 3.0
    y = oracle.output_norm_gate(o, np.zeros_like(o), w, eps=eps)
    expect = np.zeros(128)
    expect[37] = 3.0 * c / math.sqrt(c * c + eps) * 0.5
    np.testing.assert_allclose(y[0], expect, rtol=1e-15, atol=0)


def test_sigmoid_identities_and_extremes():
    z = np.array([-1000.0, -40.0, -1.0, 0.0, 1.0, 40.0, 1000.0])
    s = sigmoid(z)
    assert np.all(np.isfinite(s))
    np.testing.assert_allclose(s + sigmoid(-z), 1.0, rtol=0, atol=1e-16)
    assert s[3] == 0.5 and s[0] == 0.0 and s[-1] == 1.0
    np.testing.assert_allclose(s[4], 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)


@pytest.mark.parametrize("mistake", ["sum_not_mean", "no_sqrt", "gate_sign", "eps_outside"])
def test_pins_catch_planted_mistakes(mistake):
    """Each plausible slip in the formula fails at least one pin above."""
    def bad(o, z, w, *, eps):
        o, z, w = np.asarray(o, float), np.asarray(z, float), np.asarray(w, float)
        ms = np.mean(o * o, axis=-1, keepdims=True)
        if mistake == "sum_not_mean":
            ms = np.sum(o * o, axis=-1, keepdims=True)
        den = np.sqrt(ms + eps)
        if mistake == "no_sqrt":
            den = ms + eps
        if mistake == "eps_outside":
            den = np.sqrt(ms) + eps
        g = sigmoid(-z if mistake == "gate_sign" else z)
        return o / den * w * g

    failures = 0
    real = oracle.output_norm_gate
    try:
        oracle.output_norm_gate = bad
        for pin in (test_worked_example_by_hand, test_rms_of_normalised_rows,
                    test_constant_rows_and_channel_weight):
            try:
                pin()
            except AssertionError:
                failures += 1
    finally:
        oracle.output_norm_gate = real
    assert failures >= 1, mistake
