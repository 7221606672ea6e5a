"""Parity of libkda's batched decode step with the fp64 CPU oracle (GPU).

A decode step is the recurrence with every request a sequence of length one;
the oracle carries its state in fp64 across steps. Tolerances as for prefill
(2e-2 of the rms for bf16 inputs; bf16 outputs are judged beyond their own
storage rounding, fp32 results directly)."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_bf16_out, max_err_rel_rms

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def run_steps(kda, d, o_dtype=None, in_dtype=None):
    state = d.state.to(DEV).clone()
    A_log, dt_bias = d.A_log.to(DEV), d.dt_bias.to(DEV)
    outs = []
    for st in d.steps:
        cv = (lambda x: x.to(DEV)) if in_dtype is None else (lambda x: x.to(in_dtype).to(DEV))
        outs.append(kda.decode_step(cv(st["q"]), cv(st["k"]), cv(st["v"]), st["g"].to(DEV),
                                    st["beta_raw"].to(DEV), A_log, dt_bias, state,
                                    scale=d.scale, o_dtype=o_dtype))
    torch.cuda.synchronize()
    return outs, state


@pytest.mark.parametrize("in_dtype", [torch.float32, torch.bfloat16])
def test_decode_small_fp32_out(kda, in_dtype):
    d = kda_inputs.make_decode(5, 3, 6, seed=42)
    outs, state = run_steps(kda, d, o_dtype=torch.float32, in_dtype=in_dtype)
    steps = [{k: (v.to(in_dtype) if k in ("q", "k", "v") else v) for k, v in st.items()}
             for st in d.steps]
    ref_outs, ref_state = oracle.kda_decode_steps(steps, d.state, d.A_log, d.dt_bias,
                                                  scale=d.scale)
    e_o = max_err_rel_rms(torch.stack(outs).cpu(), np.stack(ref_outs))
    e_s = max_err_rel_rms(state, ref_state)
    print("decode small %s: o %.3e state %.3e" % (in_dtype, e_o, e_s), flush=True)
    assert e_o <= 1e-5 and e_s <= 1e-5          # fp32 arithmetic throughout


def test_decode_equals_prefill_of_length_one(kda):
    """One decode step equals a prefill where every request is a 1-token sequence
    (fp32 inputs, so both sides compute to fp32 accuracy)."""
    d = kda_inputs.make_decode(16, 4, 1, seed=43)
    outs, state = run_steps(kda, d, o_dtype=torch.float32, in_dtype=torch.float32)
    st = d.steps[0]
    f = lambda x: x.float().to(DEV)
    o, ht = kda.chunk_fwd(f(st["q"]), f(st["k"]), f(st["v"]), st["g"].to(DEV),
                          st["beta_raw"].to(DEV), d.A_log.to(DEV), d.dt_bias.to(DEV),
                          torch.arange(17, device=DEV), scale=d.scale, chunk_size=16,
                          initial_state=d.state.to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert max_err_rel_rms(outs[0], o.cpu().double().numpy()) < 1e-5
    assert max_err_rel_rms(state, ht.cpu().double().numpy()) < 1e-5


def test_decode_deterministic(kda):
    d = kda_inputs.make_decode(32, 8, 2, seed=44)
    a, sa = run_steps(kda, d)
    b, sb = run_steps(kda, d)
    assert all(torch.equal(x, y) for x, y in zip(a, b)) and torch.equal(sa, sb)


@pytest.mark.parametrize("o_dtype", [None, torch.float32])
def test_decode_256x32_64_steps(kda, o_dtype):
    """The decode workload: 256 requests, H=32, 64 consecutive steps, state in
    place. bf16 output is judged beyond its own storage rounding (raw error
    printed); fp32 output under the literal metric, over all 64 steps' outputs
    and the final state."""
    d = kda_inputs.decode(64)
    outs, state = run_steps(kda, d, o_dtype=o_dtype)
    ref_outs, ref_state = oracle.kda_decode_steps(d.steps, d.state, d.A_log, d.dt_bias,
                                                  scale=d.scale)
    o_all = torch.stack(outs).cpu()
    ref_all = np.stack(ref_outs)
    raw = max_err_rel_rms(o_all, ref_all)
    e_o = max_err_bf16_out(o_all, ref_all) if o_all.dtype == torch.bfloat16 else raw
    e_s = max_err_rel_rms(state, ref_state)
    print("decode 256x32x64 o %s: o err %.3e (raw %.3e) state err %.3e"
          % (o_all.dtype, e_o, raw, e_s), flush=True)
    assert np.all(np.isfinite(o_all.double().numpy()))
    assert e_o <= 2e-2 and e_s <= 2e-2
