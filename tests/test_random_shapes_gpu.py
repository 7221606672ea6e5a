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
