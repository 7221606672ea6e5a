"""Parity of libkda's training backward (kda_backward) with the fp64 backward
oracle (GPU).

The backward runs entirely in fp32 (fp32 MFMA products and sums, no
reduced-precision operands), so every gradient is held to 1e-4 of its rms (fp32
roundoff is 6e-8; the reverse pass adds a few roundings per 16-token chunk along
state adjoints that the decay keeps bounded, a token's log-decay adjoint sums
up to 16 per-chunk terms each rounded to fp32 over 128 state rows, and the
parameter gradients sum up to T*128 terms in blocks of 16 and then in
sequence), and to bitwise repetition between runs."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_rel_rms, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-4
KEYS = ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dh0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def adjoints(p, seed, with_dht=True, do_dtype=None):
    gen = torch.Generator().manual_seed(seed)
    do = torch.randn(p.T, p.H, 128, generator=gen)
    if do_dtype is not None:
        do = do.to(do_dtype)
    dht = torch.randn(p.N, p.H, 128, 128, generator=gen) * 0.1 if with_dht else None
    return do, dht


def run_gpu(kda, p, do, dht, heads=None):
    d = {n: getattr(p, n).to(DEV) for n in ("q", "k", "v", "g", "beta_raw", "A_log", "dt_bias",
                                            "cu_seqlens")}
    r = kda.backward(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                     d["cu_seqlens"], do.to(DEV), scale=p.scale,
                     initial_state=None if p.h0 is None else p.h0.to(DEV),
                     d_final_state=None if dht is None else dht.to(DEV))
    torch.cuda.synchronize()
    return r


def run_oracle(p, do, dht, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    par = (lambda t: t) if heads is None else (lambda t: t[heads])
    return oracle.kda_backward(sel(p.q), sel(p.k), sel(p.v), sel(p.g), sel(p.beta_raw),
                               par(p.A_log), par(p.dt_bias), p.cu_seqlens, sel(do),
                               scale=p.scale, h0=None if p.h0 is None else sel(p.h0),
                               dht=None if dht is None else sel(dht))


def compare(r, ref, heads=None, label=""):
    worst = {}
    for key in KEYS:
        g = r[key]
        if heads is not None:
            g = g[heads] if key in ("dA_log", "ddt_bias") else g[:, heads]
        worst[key] = max_err_rel_rms(g, ref[key])
    print("backward %s: %s" % (label, " ".join("%s=%.2e" % kv for kv in worst.items())), flush=True)
    assert max(worst.values()) <= TOL, worst


@pytest.mark.parametrize("case", ["small", "varlen", "T1024"])
def test_backward_matches_oracle(kda, case):
    if case == "small":
        p = kda_inputs.small()
        p.h0 = torch.randn(1, 1, 128, 128, generator=torch.Generator().manual_seed(5)) * 0.1
    elif case == "varlen":
        p = kda_inputs.varlen()
    else:
        p = kda_inputs.make_prefill([1024], 4, g_std=2.0, h0_std=0.1, seed=1020)
    do, dht = adjoints(p, 100, do_dtype=p.q.dtype)
    r = run_gpu(kda, p, do, dht)
    compare(r, run_oracle(p, do, dht), label=case)


def test_backward_empty_and_short_sequences(kda):
    # empty sequences (first, middle, last) pass the final-state adjoint back;
    # lengths around the checkpoint spacing of 16
    p = kda_inputs.make_prefill([0, 5, 0, 16, 17, 1, 31, 0], 2, h0_std=0.1, seed=1021)
    do, dht = adjoints(p, 101, do_dtype=torch.bfloat16)
    r = run_gpu(kda, p, do, dht)
    ref = run_oracle(p, do, dht)
    compare(r, ref, label="empty/short")
    for n in (0, 2, 7):
        np.testing.assert_array_equal(to_np(r["dh0"][n]), to_np(dht[n]))


def test_backward_without_initial_state_or_final_adjoint(kda):
    p = kda_inputs.make_prefill([40, 9], 3, token_dtype=torch.float32, seed=1022)
    do, _ = adjoints(p, 102, with_dht=False)
    r = run_gpu(kda, p, do, None)
    compare(r, run_oracle(p, do, None), label="no h0 / dht")


def test_backward_repeats_bit_for_bit(kda):
    p = kda_inputs.varlen()
    do, dht = adjoints(p, 103, do_dtype=torch.bfloat16)
    a = run_gpu(kda, p, do, dht)
    b = run_gpu(kda, p, do, dht)
    for key in KEYS:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("lengths", [[8192], kda_inputs.LARGE_VARLEN_LENGTHS])
def test_backward_full_size_sampled_heads(kda, lengths):
    # the benchmark's prefill workload (H = 96, bf16); heads are independent,
    # so the oracle runs on three of them and those heads are compared in full
    p = kda_inputs.make_prefill(lengths, 96, g_std=2.0, h0_std=0.1, seed=1023)
    do, dht = adjoints(p, 104, do_dtype=torch.bfloat16)
    r = run_gpu(kda, p, do, dht)
    heads = [0, 41, 95]
    compare(r, run_oracle(p, do, dht, heads), heads=heads, label="full size %d seqs" % len(lengths))
