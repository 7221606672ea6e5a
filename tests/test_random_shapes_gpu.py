"""Parity over seeded random problem shapes (GPU).

Each case draws, from its own seed, a packed batch (1 to 6 sequences of 0 to
200 tokens, empty ones included), a head count with a random grouping of the
q/k heads, a chunk size, the token dtype, whether initial states are given, and
the head sizes (128 most of the time, otherwise any sizes up to 128 on the
zero-padded chunkwise path); the chunkwise prefill and the token-by-token
kernel are then both compared with the fp64 oracle at the tolerance of the
dtype (1e-4 of the rms for fp32 tokens, 2e-2 for bf16)."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_rel_rms, prefill_to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def draw(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 7))
    lengths = [int(x) if r.random() > 0.15 else 0 for x in r.integers(1, 201, size=n)]
    H = int(r.integers(1, 7))
    divs = [d for d in range(1, H + 1) if H % d == 0]
    Hqk = int(r.choice(divs))
    chunk = int(r.choice([16, 32, 64]))
    dtype = torch.float32 if r.random() < 0.4 else torch.bfloat16
    if r.random() < 0.7:
        K = V = 128
    else:
        K, V = int(r.integers(1, 129)), int(r.integers(1, 129))
    h0 = r.random() < 0.6
    g_std = float(r.choice([0.5, 1.0, 2.0, 4.0]))
    return dict(lengths=lengths, H=H, Hqk=Hqk, chunk=chunk, dtype=dtype, K=K, V=V, h0=h0,
                g_std=g_std)


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_shape_parity(kda, seed):
    c = draw(7000 + seed)
    print("case", seed, c, flush=True)
    p = kda_inputs.make_prefill(c["lengths"], c["H"], token_dtype=c["dtype"],
                                h0_std=0.1 if c["h0"] else None, chunk=c["chunk"], seed=8000 + seed,
                                K=c["K"], V=c["V"], g_std=c["g_std"])
    G = c["H"] // c["Hqk"]
    d = prefill_to_device(p, DEV)
    q, k = d["q"][:, ::G].contiguous(), d["k"][:, ::G].contiguous()
    args = (q, k, d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"], d["cu_seqlens"])
    o1, h1 = kda.chunk_fwd(*args, scale=p.scale, chunk_size=c["chunk"], initial_state=d["h0"],
                           o_dtype=torch.float32)
    o2, h2 = kda.recurrent_fwd(*args, scale=p.scale, initial_state=d["h0"],
                               o_dtype=torch.float32)
    torch.cuda.synchronize()
    qr = p.q[:, ::G].repeat_interleave(G, dim=1)
    kr = p.k[:, ::G].repeat_interleave(G, dim=1)
    ro, rht = oracle.kda_recurrent(qr, kr, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens,
                                   scale=p.scale, h0=p.h0)
    tol = 1e-4 if c["dtype"] == torch.float32 else 2e-2
    errs = [max_err_rel_rms(x, ref) for x, ref in ((o1, ro), (h1, rht), (o2, ro), (h2, rht))]
    print("errors chunked o %.2e ht %.2e, token-by-token o %.2e ht %.2e" % tuple(errs), flush=True)
    assert max(errs) <= tol, errs


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_shape_backward(kda, seed):
    """The training backward on random shapes, every gradient against the fp64
    backward oracle at 1e-4 of its rms (fp32 arithmetic throughout)."""
    c = draw(9000 + seed)
    c["lengths"] = [min(x, 90) for x in c["lengths"]]        # the oracle's reverse sweep is slow
    print("case", seed, c, flush=True)
    p = kda_inputs.make_prefill(c["lengths"], c["H"], token_dtype=c["dtype"],
                                h0_std=0.1 if c["h0"] else None, chunk=c["chunk"], seed=9500 + seed,
                                K=c["K"], V=c["V"], g_std=c["g_std"])
    gen = torch.Generator().manual_seed(9600 + seed)
    do = torch.randn(p.T, p.H, c["V"], generator=gen).to(c["dtype"])
    dht = torch.randn(p.N, p.H, c["V"], c["K"], generator=gen) * 0.1
    G = c["H"] // c["Hqk"]
    d = prefill_to_device(p, DEV)
    q, k = d["q"][:, ::G].contiguous(), d["k"][:, ::G].contiguous()
    r = kda.backward(q, k, d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                     d["cu_seqlens"], do.to(DEV), scale=p.scale, initial_state=d["h0"],
                     d_final_state=dht.to(DEV))
    torch.cuda.synchronize()
    qr = p.q[:, ::G].repeat_interleave(G, dim=1)
    kr = p.k[:, ::G].repeat_interleave(G, dim=1)
    ref = oracle.kda_backward(qr, kr, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens, do,
                              scale=p.scale, h0=p.h0, dht=dht)
    for key in ("dq", "dk"):
        ref[key] = ref[key].reshape(p.T, c["Hqk"], G, c["K"]).sum(axis=2)
    keys = ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dh0")
    worst = {key: max_err_rel_rms(r[key], ref[key]) for key in keys if ref[key].size}
    print("backward errors", " ".join("%s=%.2e" % kv for kv in worst.items()), flush=True)
    assert max(worst.values()) <= 1e-4, worst


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_shape_decode(kda, seed):
    """Decode steps on random batch sizes, head counts and head sizes (128 on the
    decode kernel, other sizes on the token-by-token kernel), several steps."""
    r = np.random.default_rng(9900 + seed)
    B, H = int(r.integers(1, 40)), int(r.integers(1, 9))
    K, V = (128, 128) if r.random() < 0.5 else (int(r.integers(1, 257)), int(r.integers(1, 257)))
    d = kda_inputs.make_decode(B, H, 3, seed=9950 + seed, K=K, V=V)
    state = d.state.to(DEV).clone()
    outs = []
    for st in d.steps:
        outs.append(kda.decode_step(st["q"].to(DEV), st["k"].to(DEV), st["v"].to(DEV),
                                    st["g"].to(DEV), st["beta_raw"].to(DEV), d.A_log.to(DEV),
                                    d.dt_bias.to(DEV), state, scale=d.scale,
                                    o_dtype=torch.float32))
    torch.cuda.synchronize()
    ref_outs, ref_state = oracle.kda_decode_steps(d.steps, d.state, d.A_log, d.dt_bias,
                                                  scale=d.scale)
    eo = max(max_err_rel_rms(a, b) for a, b in zip(outs, ref_outs))
    eh = max_err_rel_rms(state, ref_state)
    print("decode B=%d H=%d K=%d V=%d: o %.2e state %.2e" % (B, H, K, V, eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2
