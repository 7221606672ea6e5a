"""The chunkwise prefill at head sizes above 128 other than K = V = 256: the
256-wide kernels (64-row chunks, bf16 inputs) over copies zero-padded to 256 key
channels and value rows, against the fp64 oracle. Tolerances as for the
128-wide prefill: 2e-2 of the rms, fp32 outputs under the literal metric, bf16
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


def make(lengths, H, K, V, seed, g_std=2.0, h0_std=0.1, name="custom"):
    return kda_inputs.make_prefill(lengths, H, g_std=g_std, h0_std=h0_std, chunk=64, seed=seed,
                                   K=K, V=V, name=name)


def run(kda, p, o_dtype=None, **kw):
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                          initial_state=d["h0"], o_dtype=o_dtype, **kw)
    torch.cuda.synchronize()
    return o, ht


def oracle_of(p):
    return oracle.kda_recurrent(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                p.cu_seqlens, scale=p.scale, h0=p.h0)


def check(o, ht, ref, label):
    o_ref, ht_ref = ref
    raw = max_err_rel_rms(o, o_ref)
    e_o = max_err_bf16_out(o, o_ref) if o.dtype == torch.bfloat16 else raw
    e_h = max_err_rel_rms(ht, ht_ref)
    print("%s: o err %.3e (raw %.3e)  ht err %.3e" % (label, e_o, raw, e_h), flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(ht)))
    assert e_o <= TOL and e_h <= TOL


@pytest.mark.parametrize("K,V", [(192, 192), (129, 256), (256, 40), (200, 130), (1, 129)])
@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_padded256_ragged(kda, K, V, o_dtype):
    """Several chunks, ragged tails, an empty and a one-token sequence."""
    p = make([1, 0, 77, 130, 64, 5, 200], 2, K, V, seed=1600 + K + V)
    o, ht = run(kda, p, o_dtype)
    assert o.shape == (p.T, 2, V) and ht.shape == (p.N, 2, V, K)
    check(o, ht, oracle_of(p), "padded 256 K=%d V=%d o %s" % (K, V, o_dtype))
    assert torch.equal(ht[1].cpu(), p.h0[1])          # the empty sequence keeps its state


def test_padded256_no_initial_state(kda):
    p = make([300, 65], 3, 250, 250, seed=1620, h0_std=None)
    o, ht = run(kda, p, torch.float32)
    check(o, ht, oracle_of(p), "padded 256 K=V=250 zero h0")


def test_padded256_grouped_heads(kda):
    """Four value heads sharing two q/k heads: the ungrouped result with q, k repeated."""
    p = make([150, 97], 4, 192, 160, seed=1630)
    qg, kg = p.q[:, ::2].contiguous(), p.k[:, ::2].contiguous()
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(qg.to(DEV), kg.to(DEV), d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                          initial_state=d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.kda_recurrent(qg.repeat_interleave(2, dim=1), kg.repeat_interleave(2, dim=1),
                               p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens,
                               scale=p.scale, h0=p.h0)
    check(o, ht, ref, "padded 256 grouped K=192 V=160")


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_padded256_gated(kda, o_dtype):
    """The output epilogue over V-wide rows after the padded prefill."""
    K, V = 160, 200
    p = make([77, 130], 3, K, V, seed=1640)
    z, w = kda_inputs.make_epilogue((p.T, p.H, V), seed=1641, D=V)
    d = prefill_to_device(p, DEV)
    y, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                         d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                         initial_state=d["h0"], o_dtype=o_dtype, gate=z.to(DEV),
                         norm_weight=w.to(DEV), norm_eps=1e-5)
    torch.cuda.synchronize()
    o_ref, _ = oracle_of(p)
    y_ref = oracle.output_norm_gate(o_ref, z, w, eps=1e-5)
    e = max_err_bf16_out(y, y_ref) if y.dtype == torch.bfloat16 else max_err_rel_rms(y, y_ref)
    print("padded 256 gated K=%d V=%d y %s: err %.3e" % (K, V, o_dtype, e), flush=True)
    assert e <= TOL


def test_padded256_matches_native_on_zero_padded_inputs(kda):
    """K = V = 192 gives the K = V = 256 result of the same inputs padded with zeros
    (the same kernels, bit for bit)."""
    p = make([150, 97], 2, 192, 192, seed=1650)
    o, ht = run(kda, p, torch.float32)
    pad = lambda x, n: torch.nn.functional.pad(x, (0, n - x.shape[-1]))
    q, k, v, g = pad(p.q, 256), pad(p.k, 256), pad(p.v, 256), pad(p.g, 256)
    dtb = pad(p.dt_bias, 256)
    h0 = torch.nn.functional.pad(p.h0, (0, 64, 0, 64))
    o2, ht2 = kda.chunk_fwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), p.beta_raw.to(DEV),
                            p.A_log.to(DEV), dtb.to(DEV), p.cu_seqlens.to(DEV), scale=p.scale,
                            chunk_size=64, initial_state=h0.to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2[..., :192]) and torch.equal(ht, ht2[:, :, :192, :192])
    assert torch.count_nonzero(o2[..., 192:]) == 0


def test_padded256_large(kda):
    """T = 2048 over 8 heads at K = V = 192."""
    p = make([2048], 8, 192, 192, seed=1660, name="T=2048 H=8 K=V=192")
    o, ht = run(kda, p, torch.float32)
    check(o, ht, oracle_of(p), "padded 256 T=2048 H=8 K=V=192")


def test_padded256_stages_split(kda):
    """The two stage entry points (intra, then inter on the same workspace) give the
    one-call result bit for bit at K = 200, V = 144."""
    p = make([150, 97, 1], 2, 200, 144, seed=1670)
    d = prefill_to_device(p, DEV)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
            d["cu_seqlens"])
    o, ht = kda.chunk_fwd(*args, scale=p.scale, chunk_size=64, initial_state=d["h0"])
    ws = kda.Workspace(DEV)
    o2 = torch.empty_like(o)
    h2 = torch.empty_like(ht)
    for stage in ("intra", "inter"):
        kda.chunk_fwd(*args, scale=p.scale, chunk_size=64, initial_state=d["h0"], out=o2,
                      final_state=h2, workspace=ws, stage=stage)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ht, h2)


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
@pytest.mark.parametrize("Kd", [192, 256])
def test_full_size_sampled_heads(kda, Kd, o_dtype):
    """The head-size leg bench.py times beside the step, at its size (T = 8192,
    H = 96, K = V = 192 over padded copies and 256 natively; bf16 outputs as timed,
    and fp32 outputs for the literal metric), checked on three sampled heads: heads
    are independent, so the oracle runs on those heads' inputs alone."""
    p = kda_inputs.make_prefill([8192], 96, token_dtype=torch.bfloat16, g_std=2.0, h0_std=0.1,
                                seed=2300 + Kd, K=Kd, V=Kd)
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=64,
                          initial_state=d["h0"], o_dtype=o_dtype)
    torch.cuda.synchronize()
    heads = [0, 37, 95]
    o_s, ht_s = o[:, heads].cpu(), ht[:, heads].cpu()
    del o, ht, d
    ref = oracle.kda_recurrent(p.q[:, heads], p.k[:, heads], p.v[:, heads], p.g[:, heads],
                               p.beta_raw[:, heads], p.A_log[heads], p.dt_bias[heads],
                               p.cu_seqlens, scale=p.scale, h0=p.h0[:, heads])
    check(o_s, ht_s, ref, "T=8192 H=96 K=V=%d o %s, heads %s" % (Kd, o_dtype, heads))
