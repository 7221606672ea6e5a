"""The chunkwise prefill with the output epilogue (kda_chunk_fwd_gated)
against the fp64 oracle: the recurrence's outputs, then the per-head RMS norm
with channel weight and the sigmoid gate, all in fp64.

Tolerances as for the prefill (1e-4 of the rms for fp32 inputs, 2e-2 for bf16;
fp32 outputs under the literal metric, bf16 outputs beyond their own storage
rounding). The gated call is also held against the prefill to fp32 o followed
by the standalone epilogue call at 1e-5 (with bf16 gate logits the gated call
reads them as stored, the standalone call a fp32 copy)."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_bf16_out, max_err_rel_rms, prefill_to_device, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
EPS = 1e-5


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def run(kda, p, z, w, o_dtype=None, chunk=None, gated=True):
    d = prefill_to_device(p, DEV)
    kw = dict(gate=z.to(DEV), norm_weight=w.to(DEV), norm_eps=EPS) if gated else {}
    y, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale,
                          chunk_size=chunk or p.chunk, initial_state=d["h0"], o_dtype=o_dtype,
                          **kw)
    torch.cuda.synchronize()
    return y, ht


def check(kda, p, o_dtype, label, seed, chunk=None):
    V = p.v.shape[2]
    z, w = kda_inputs.make_epilogue((p.T, p.H, V), token_dtype=p.q.dtype, seed=seed, D=V)
    o_ref, ht_ref = oracle.kda_recurrent(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                         p.cu_seqlens, scale=p.scale, h0=p.h0)
    y_ref = oracle.output_norm_gate(o_ref, z, w, eps=EPS)
    y, ht = run(kda, p, z, w, o_dtype=o_dtype, chunk=chunk)
    tol = 1e-4 if p.q.dtype == torch.float32 else 2e-2
    raw = max_err_rel_rms(y, y_ref)
    e_y = max_err_bf16_out(y, y_ref) if y.dtype == torch.bfloat16 else raw
    e_h = max_err_rel_rms(ht, ht_ref)
    print("%s: y err %.3e (raw %.3e)  ht err %.3e  tol %.0e" % (label, e_y, raw, e_h, tol),
          flush=True)
    assert np.all(np.isfinite(to_np(y)))
    assert e_y <= tol and e_h <= tol
    if p.T > 0 and y.dtype == torch.float32 and V == 128:
        # against the two calls: prefill to fp32 o, then the standalone epilogue
        o32, _ = run(kda, p, z, w, o_dtype=torch.float32, chunk=chunk, gated=False)
        y2 = kda.output_norm_gate(o32, z.to(DEV).to(torch.float32) if z.dtype != torch.float32
                                  else z.to(DEV), w.to(DEV), eps=EPS)
        torch.cuda.synchronize()
        e2 = max_err_rel_rms(y, to_np(y2))
        print("  gated call vs prefill + epilogue calls: %.3e" % e2, flush=True)
        assert e2 <= 1e-5


@pytest.mark.parametrize("dtype,chunk", [(torch.float32, 16), (torch.float32, 64),
                                         (torch.bfloat16, 32), (torch.bfloat16, 64)])
@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_gated_ragged(kda, dtype, chunk, o_dtype):
    """Several chunks, ragged tails, an empty and a one-token sequence."""
    p = kda_inputs.make_prefill([1, 0, 77, 130, 64, 5], 3, token_dtype=dtype, g_std=2.0,
                                h0_std=0.1, chunk=chunk, seed=1300 + chunk)
    check(kda, p, o_dtype, "gated ragged %s C=%d o %s" % (dtype, chunk, o_dtype), seed=1301)


def test_gated_other_head_sizes(kda):
    """K=48, V=80: the prefill on zero-padded copies, then the epilogue as a pass."""
    p = kda_inputs.make_prefill([33, 0, 70], 2, g_std=1.0, h0_std=0.1, chunk=32, seed=1310,
                                K=48, V=80)
    check(kda, p, torch.float32, "gated K=48 V=80", seed=1311)


def test_gated_empty_batch(kda):
    p = kda_inputs.make_prefill([0, 0], 2, h0_std=1.0, chunk=64, seed=1312)
    z, w = kda_inputs.make_epilogue((0, 2, 128), seed=1313)
    y, ht = run(kda, p, z, w)
    assert y.shape == (0, 2, 128) and torch.equal(ht.cpu(), p.h0)


def test_gated_rejects(kda):
    p = kda_inputs.make_prefill([10], 1, chunk=16, seed=1314)
    z, w = kda_inputs.make_epilogue((10, 1, 128), seed=1315)
    d = prefill_to_device(p, DEV)
    with pytest.raises(ValueError):
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                      d["cu_seqlens"], chunk_size=16, gate=z.to(DEV), norm_weight=None)
    with pytest.raises(kda.KDAError):
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                      d["cu_seqlens"], chunk_size=16, gate=z.to(DEV), norm_weight=w.to(DEV),
                      norm_eps=0.0)


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_gated_large(kda, o_dtype):
    """The T=8192, H=96 prefill with the epilogue."""
    p = kda_inputs.large()
    check(kda, p, o_dtype, "gated T=8192 H=96 o %s" % o_dtype, seed=1320)


# 50 sequences of 3 heads: 150 chains, 304 workgroups of the inter-chunk kernel,
# more than the 256 CUs hold at once, so the epilogue is not fused in it but runs
# as a pass over staged outputs
MANY = [1, 0, 77, 130, 64, 5] + [9, 70, 0, 33] * 11


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_gated_unfused(kda, o_dtype):
    """A batch with too many sequences for the fused epilogue."""
    p = kda_inputs.make_prefill(MANY, 3, g_std=2.0, h0_std=0.1, chunk=64, seed=1325)
    check(kda, p, o_dtype, "gated unfused 50 sequences o %s" % o_dtype, seed=1326)


def test_gated_fp16_staging(kda):
    """bf16 outputs of the natively sized K = V = 128 kernels (64-row chunks,
    bf16 tokens) when the epilogue is not fused (too many sequences): the
    chunkwise forward stages o in fp16, each 16-feature block
    of a row divided by a power of two, and the epilogue multiplies the scale
    back. Against the prefill's fp32 o followed by the standalone fp32
    epilogue, element by element within the staging bound: a staged value is
    off by at most 2^-11 of its block's largest magnitude b, which moves
    y = x r w sigmoid(z) by at most |w sigmoid(z)| r 2^-11 (b + |x| r m)
    (m: the row's largest magnitude; the second term is the change of the
    row's inverse rms r), plus y's own bf16 rounding. Heads scaled by 2^20
    and 2^-20, one head's first block by 2^12 (a block scale, not a row scale,
    keeps the other blocks exact to their own magnitude) and a sequence of
    zeros (outputs exactly 0)."""
    from helpers import bf16_half_ulp
    p = kda_inputs.make_prefill(MANY, 3, g_std=2.0, h0_std=0.1, chunk=64, seed=1330)
    v, h0 = p.v.to(torch.float32), p.h0.clone()
    for h, f in ((0, 2.0 ** 20), (2, 2.0 ** -20)):
        v[:, h] *= f
        h0[:, h] *= f
    v[:, 1, :16] *= 2.0 ** 12
    h0[:, 1, :16] *= 2.0 ** 12
    z0, z1 = int(p.cu_seqlens[4]), int(p.cu_seqlens[5])
    v[z0:z1] = 0.0
    h0[4] = 0.0
    p.v, p.h0 = v.to(torch.bfloat16), h0           # power-of-two scalings: exact in bf16
    z, w = kda_inputs.make_epilogue((p.T, p.H, 128), token_dtype=torch.bfloat16, seed=1331, D=128)
    y, _ = run(kda, p, z, w)
    assert y.dtype == torch.bfloat16
    o32, _ = run(kda, p, z, w, o_dtype=torch.float32, gated=False)
    y2 = kda.output_norm_gate(o32, z.to(DEV).to(torch.float32), w.to(DEV), eps=EPS)
    torch.cuda.synchronize()
    x = to_np(o32).astype(np.float64)
    T, H = x.shape[:2]
    ax = np.abs(x)
    b = np.repeat(ax.reshape(T, H, 8, 16).max(-1), 16, axis=-1)
    m = ax.max(-1, keepdims=True)
    r = 1.0 / np.sqrt((x * x).mean(-1, keepdims=True) + EPS)
    zs = to_np(z).astype(np.float64)
    ws = np.abs(to_np(w).astype(np.float64)) / (1.0 + np.exp(-zs))
    bound = ws * r * 2.0 ** -11 * (b + ax * r * m)
    yg, yr = to_np(y).astype(np.float64), to_np(y2).astype(np.float64)
    ex = np.abs(yg - yr) - bf16_half_ulp(yg) - 1e-6 * np.abs(yr)
    ratio = float(np.max(ex / np.maximum(bound, 1e-300)))
    print("fp16 staging: max excess over the bound's share %.3f" % ratio, flush=True)
    assert np.all(ex <= 1.5 * bound)
    assert np.all(yg[z0:z1] == 0.0)


@pytest.mark.parametrize("N,H", [(32, 4), (17, 8)])
def test_gated_fusion_boundary(kda, N, H):
    """Either side of the fused epilogue's residency limit (128 chains: 32 x 4 is
    fused, 17 x 8 = 136 is not): both paths against the oracle, with fp32 results
    also against the prefill to fp32 o followed by the standalone epilogue."""
    lengths = [(37 * i) % 150 for i in range(N)]
    p = kda_inputs.make_prefill(lengths, H, g_std=2.0, h0_std=0.1, chunk=64, seed=1340 + N)
    for o_dtype in (None, torch.float32):
        check(kda, p, o_dtype, "gated N=%d H=%d o %s" % (N, H, o_dtype), seed=1341)
