"""The chunkwise prefill at K = V = 256 on kernels sized for 256 (64-row chunks,
bf16 inputs) against the fp64 oracle. Tolerances as for the 128-wide prefill:
2e-2 of the rms for bf16 inputs, fp32 outputs under the literal metric, bf16
outputs beyond their own storage rounding."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_bf16_out, max_err_rel_rms, prefill_to_device, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-2


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def run(kda, p, o_dtype=None, **kw):
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                          initial_state=d["h0"], o_dtype=o_dtype, **kw)
    torch.cuda.synchronize()
    return o, ht


def check(p, o, ht, ref, label):
    o_ref, ht_ref = ref
    raw = max_err_rel_rms(o, o_ref)
    e_o = max_err_bf16_out(o, o_ref) if o.dtype == torch.bfloat16 else raw
    e_h = max_err_rel_rms(ht, ht_ref)
    print("%s: o err %.3e (raw %.3e)  ht err %.3e" % (label, e_o, raw, e_h), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(ht)))
    assert e_o <= TOL and e_h <= TOL


def oracle_of(p):
    return oracle.kda_recurrent(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                p.cu_seqlens, scale=p.scale, h0=p.h0)


def p256(lengths, H, seed, g_std=2.0, h0_std=0.1, name="custom"):
    return kda_inputs.make_prefill(lengths, H, g_std=g_std, h0_std=h0_std, chunk=64, seed=seed,
                                   K=256, V=256, name=name)


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_native256_ragged(kda, o_dtype):
    """Several chunks, ragged tails, an empty and a one-token sequence."""
    p = p256([1, 0, 77, 130, 64, 5, 300], 3, seed=1500)
    o, ht = run(kda, p, o_dtype)
    assert o.shape == (p.T, 3, 256) and ht.shape == (p.N, 3, 256, 256)
    check(p, o, ht, oracle_of(p), "native 256 ragged o %s" % o_dtype)
    assert torch.equal(ht[1].cpu(), p.h0[1])          # the empty sequence keeps its state


@pytest.mark.parametrize("g_std", [0.01, 0.5, 8.0])
def test_native256_gate_regimes(kda, g_std):
    p = p256([333, 211], 2, seed=1510 + int(g_std * 10), g_std=g_std)
    o, ht = run(kda, p, torch.float32)
    check(p, o, ht, oracle_of(p), "native 256 gate std %g" % g_std)


def test_native256_no_initial_state_and_large_values(kda):
    p = p256([200, 65], 2, seed=1520, h0_std=None)
    o, ht = run(kda, p, torch.float32)
    check(p, o, ht, oracle_of(p), "native 256 zero h0")
    p = p256([200], 2, seed=1521)
    p.v = (p.v.float() * 1e6).to(torch.bfloat16)
    p.h0 = p.h0 * 1e6
    o, ht = run(kda, p, torch.float32)
    check(p, o, ht, oracle_of(p), "native 256 v, h0 x 1e6")


def test_native256_grouped_heads(kda):
    """Four value heads sharing two q/k heads: the ungrouped result with q, k repeated."""
    p = p256([150, 97], 4, seed=1530)
    qg, kg = p.q[:, ::2].contiguous(), p.k[:, ::2].contiguous()
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(qg.to(DEV), kg.to(DEV), d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                          initial_state=d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    rq = qg.repeat_interleave(2, dim=1)
    rk = kg.repeat_interleave(2, dim=1)
    ref = oracle.kda_recurrent(rq, rk, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens,
                               scale=p.scale, h0=p.h0)
    check(p, o, ht, ref, "native 256 grouped")


def test_native256_split_chaining_and_determinism(kda):
    p = p256([333], 2, seed=1540)
    ref = oracle_of(p)
    d = prefill_to_device(p, DEV)
    t = 150
    cut = lambda x, a, b: x[a:b]
    o1, h1 = kda.chunk_fwd(*(cut(d[n], 0, t) for n in ("q", "k", "v", "g", "beta_raw")),
                           d["A_log"], d["dt_bias"], torch.tensor([0, t], device=DEV),
                           scale=p.scale, chunk_size=64, initial_state=d["h0"],
                           o_dtype=torch.float32)
    o2, h2 = kda.chunk_fwd(*(cut(d[n], t, 333) for n in ("q", "k", "v", "g", "beta_raw")),
                           d["A_log"], d["dt_bias"], torch.tensor([0, 333 - t], device=DEV),
                           scale=p.scale, chunk_size=64, initial_state=h1, o_dtype=torch.float32)
    torch.cuda.synchronize()
    check(p, torch.cat([o1, o2]), h2, ref, "native 256 split at %d" % t)
    a, ha = run(kda, p)
    b, hb = run(kda, p)
    assert torch.equal(a, b) and torch.equal(ha, hb)


def test_native256_gated(kda):
    """The output epilogue over 256-wide rows (a pass after the inter-chunk kernel)."""
    p = p256([77, 130], 3, seed=1550)
    z, w = kda_inputs.make_epilogue((p.T, p.H, 256), seed=1551, D=256)
    d = prefill_to_device(p, DEV)
    y, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                         d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                         initial_state=d["h0"], gate=z.to(DEV), norm_weight=w.to(DEV),
                         norm_eps=1e-5)
    torch.cuda.synchronize()
    o_ref, _ = oracle_of(p)
    y_ref = oracle.output_norm_gate(o_ref, z, w, eps=1e-5)
    e = max_err_bf16_out(y, y_ref)
    print("native 256 gated: y err %.3e" % e, flush=True)
    assert e <= TOL


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_native256_large(kda, o_dtype):
    """T = 4096 over 16 heads at K = V = 256 (the state 256 KB per head)."""
    p = p256([4096], 16, seed=1560, name="T=4096 H=16 K=V=256")
    o, ht = run(kda, p, o_dtype)
    check(p, o, ht, oracle_of(p), "native 256 T=4096 H=16 o %s" % o_dtype)
