"""Parity of libkda's output epilogue (per-head RMS norm, channel weight, sigmoid
gate) with the fp64 oracle, standalone and fused into the decode step (GPU).

The epilogue itself is fp32 arithmetic: judged at 1e-5 of the rms for fp32
rows and, for bf16 rows, beyond the output's own storage rounding at the same
1e-5. End-to-end results (prefill or decode followed by the epilogue) are held
to the path's bf16 bound, 2e-2 of the rms."""
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


def err(y, ref, dtype):
    return max_err_bf16_out(y, ref) if dtype == torch.bfloat16 else max_err_rel_rms(y, ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows", [1, 15, 16, 17, 1000, 4099])
def test_norm_gate_matches_oracle(kda, dtype, rows):
    gen = torch.Generator().manual_seed(900 + rows)
    # rows of very different magnitudes (the norm removes the scale)
    o = (torch.randn(rows, 128, generator=gen) *
         torch.exp(3 * torch.randn(rows, 1, generator=gen))).to(dtype)
    z, w = kda_inputs.make_epilogue((rows, 128), token_dtype=dtype, seed=rows)
    y = kda.output_norm_gate(o.to(DEV), z.to(DEV), w.to(DEV), eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.output_norm_gate(o, z, w, eps=EPS)
    e = err(y, ref, dtype)
    print("norm_gate %s rows=%d: err %.3e" % (dtype, rows, e), flush=True)
    assert y.dtype == dtype and y.shape == o.shape
    assert e <= 1e-5


def test_norm_gate_in_place_and_3d(kda):
    o = torch.randn(37, 5, 128, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    z, w = kda_inputs.make_epilogue((37, 5, 128), seed=8)
    ref = oracle.output_norm_gate(o, z, w, eps=EPS)
    od = o.to(DEV)
    y = kda.output_norm_gate(od, z.to(DEV), w.to(DEV), eps=EPS, out=od)
    torch.cuda.synchronize()
    assert y.data_ptr() == od.data_ptr()
    assert max_err_bf16_out(od, ref) <= 1e-5


def test_norm_gate_zero_rows_and_zero_vectors(kda):
    e = torch.empty(0, 128, device=DEV, dtype=torch.bfloat16)
    w = torch.ones(128, device=DEV)
    assert kda.output_norm_gate(e, e, w).shape == (0, 128)
    # an all-zero row maps to zeros (eps keeps the norm finite)
    o = torch.zeros(3, 128, device=DEV)
    z = torch.randn(3, 128, device=DEV)
    y = kda.output_norm_gate(o, z, w)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_prefill_then_epilogue(kda):
    """The epilogue on the T=4096, H=32 prefill output: against the oracle applied
    to the GPU's own o (the epilogue alone) and to the oracle's o (end to end)."""
    p = kda_inputs.prefill_4k()
    d = prefill_to_device(p, DEV)
    o, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                         d["cu_seqlens"], scale=p.scale, chunk_size=64, output_final_state=False,
                         o_dtype=torch.float32)
    z, w = kda_inputs.make_epilogue(tuple(o.shape), token_dtype=torch.float32, seed=41)
    y = kda.output_norm_gate(o, z.to(DEV), w.to(DEV), eps=EPS)
    torch.cuda.synchronize()
    e_alone = max_err_rel_rms(y, oracle.output_norm_gate(o.cpu(), z, w, eps=EPS))
    ref_o, _ = oracle.kda_recurrent(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                    p.cu_seqlens, scale=p.scale)
    e_path = max_err_rel_rms(y, oracle.output_norm_gate(ref_o, z, w, eps=EPS))
    print("prefill+epilogue: epilogue %.3e, end to end %.3e" % (e_alone, e_path), flush=True)
    assert e_alone <= 1e-5 and e_path <= 2e-2


@pytest.mark.parametrize("in_dtype,o_dtype", [(torch.float32, torch.float32),
                                              (torch.bfloat16, torch.bfloat16),
                                              (torch.bfloat16, torch.float32)])
def test_decode_gated(kda, in_dtype, o_dtype):
    """kda_decode_step_gated: the state update is bitwise that of kda_decode_step,
    the output the epilogue of the ungated output (same bound as standalone), and
    against the oracle end to end."""
    d = kda_inputs.make_decode(24, 6, 3, seed=45)
    A_log, dt_bias = d.A_log.to(DEV), d.dt_bias.to(DEV)
    s_plain = d.state.to(DEV).clone()
    s_gated = d.state.to(DEV).clone()
    ref_state = d.state
    for i, st in enumerate(d.steps):
        cv = lambda x: x.to(in_dtype).to(DEV)
        z, w = kda_inputs.make_epilogue((24, 6, 128), token_dtype=in_dtype, seed=60 + i)
        args = (cv(st["q"]), cv(st["k"]), cv(st["v"]), st["g"].to(DEV), st["beta_raw"].to(DEV),
                A_log, dt_bias)
        o_plain = kda.decode_step(*args, s_plain, scale=d.scale, o_dtype=torch.float32)
        y = kda.decode_step(*args, s_gated, scale=d.scale, o_dtype=o_dtype,
                            gate=z.to(DEV), norm_weight=w.to(DEV), norm_eps=EPS)
        torch.cuda.synchronize()
        assert torch.equal(s_plain, s_gated)
        e_ep = err(y, oracle.output_norm_gate(o_plain.cpu(), z, w, eps=EPS), o_dtype)
        step = [{k: (v.to(in_dtype) if k in ("q", "k", "v") else v) for k, v in st.items()}]
        ref_outs, ref_state = oracle.kda_decode_steps(step, ref_state, d.A_log, d.dt_bias,
                                                      scale=d.scale)
        e_path = err(y, oracle.output_norm_gate(ref_outs[0], z, w, eps=EPS), o_dtype)
        print("decode gated %s->%s step %d: epilogue %.3e, end to end %.3e"
              % (in_dtype, o_dtype, i, e_ep, e_path), flush=True)
        assert e_ep <= 1e-5
        assert e_path <= (1e-4 if in_dtype == torch.float32 else 2e-2)


def test_norm_gate_bench_size_sampled(kda):
    """At the prefill benchmark's output size (T=8192, H=96 rows of 128, bf16),
    checked on sampled rows against the oracle."""
    rows = 8192 * 96
    gen = torch.Generator().manual_seed(77)
    o = torch.randn(rows, 128, generator=gen).to(torch.bfloat16)
    z, w = kda_inputs.make_epilogue((rows, 128), seed=78)
    y = kda.output_norm_gate(o.to(DEV), z.to(DEV), w.to(DEV), eps=EPS).cpu()
    idx = torch.randint(0, rows, (4096,), generator=gen)
    idx = torch.cat([idx, torch.tensor([0, rows - 1])])
    ref = oracle.output_norm_gate(o[idx], z[idx], w, eps=EPS)
    assert max_err_bf16_out(y[idx], ref) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D,rows", [(64, 1001), (17, 5), (256, 63), (1, 9), (96, 4)])
def test_norm_gate_other_widths(kda, dtype, D, rows):
    """Rows of widths other than 128 (the outputs of other head sizes): the
    one-wave-per-row kernel, same bar as the 128-wide kernel."""
    gen = torch.Generator().manual_seed(950 + D + rows)
    o = (torch.randn(rows, D, generator=gen) *
         torch.exp(3 * torch.randn(rows, 1, generator=gen))).to(dtype)
    z = (torch.randn(rows, D, generator=gen) * 2.0).to(dtype)
    w = torch.rand(D, generator=gen) + 0.5
    y = kda.output_norm_gate(o.to(DEV), z.to(DEV), w.to(DEV), eps=EPS)
    torch.cuda.synchronize()
    e = err(y, oracle.output_norm_gate(o, z, w, eps=EPS), dtype)
    print("norm_gate D=%d rows=%d %s: %.3e" % (D, rows, dtype, e), flush=True)
    assert y.shape == (rows, D) and e <= 1e-5
