"""kda_chunk_fwd_noalloc (the prefill with the library's fixed device scratch
instead of a caller workspace) against kda_chunk_fwd on the same inputs, both
called through the C ABI: two calls in a row, the second on a smaller
problem, each bit for bit equal to the workspace entry point (the same
kernels) and within the parity tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_bf16_out, max_err_rel_rms, prefill_to_device

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def _noalloc(kda, p, d, o_dtype):
    T, H = p.T, p.H
    o = torch.full((T, H, 128), float("nan"), dtype=o_dtype, device=DEV)
    ht = torch.full((p.N, H, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    lib = kda.kda.lib
    dt = kda.kda._dt
    st = lib.kda_chunk_fwd_noalloc(
        d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["g"].data_ptr(),
        d["beta_raw"].data_ptr(), d["A_log"].data_ptr(), d["dt_bias"].data_ptr(),
        float(p.scale), -5.0, d["cu_seqlens"].data_ptr(), p.N, T, H, 128, 128, p.chunk,
        dt(d["q"]), None if d["h0"] is None else d["h0"].data_ptr(), ht.data_ptr(),
        o.data_ptr(), dt(o), torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0, lib.kda_last_error()
    return o, ht


def _check(kda, p, o_dtype):
    need = kda.workspace_size(p.T, p.N, p.H, p.chunk, p.q.dtype)
    assert need <= kda.kda.NOALLOC_SCRATCH_BYTES
    print("case %s (H=%d, T=%d, C=%d, o %s): scratch %d bytes"
          % (p.name, p.H, p.T, p.chunk, o_dtype, need), flush=True)
    d = prefill_to_device(p, DEV)
    o_ws, ht_ws = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                                d["dt_bias"], d["cu_seqlens"], scale=p.scale,
                                chunk_size=p.chunk, initial_state=d["h0"], o_dtype=o_dtype)
    o_na, ht_na = _noalloc(kda, p, d, o_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws) and torch.equal(ht_na, ht_ws)
    o_ref, ht_ref = oracle.kda_recurrent(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                         p.cu_seqlens, scale=p.scale, h0=p.h0)
    tol = 1e-4 if p.q.dtype == torch.float32 else 2e-2
    e_o = (max_err_bf16_out(o_na, o_ref) if o_dtype == torch.bfloat16
           else max_err_rel_rms(o_na, o_ref))
    e_h = max_err_rel_rms(ht_na, ht_ref)
    print("  noalloc vs oracle: o %.3e  ht %.3e  (tol %.0e)" % (e_o, e_h, tol), flush=True)
    assert e_o <= tol and e_h <= tol


def test_noalloc_two_calls_second_smaller(kda):
    # one GPU's tensor-parallel share of the T=8192, H=96 prefill (12 heads),
    # close to the fixed scratch's size ...
    big = kda_inputs.make_prefill([8192], 12, g_std=2.0, h0_std=0.1, chunk=64, seed=1201,
                                  name="T=8192 H=12 bf16")
    _check(kda, big, torch.float32)
    # ... then a smaller ragged batch with an empty sequence, other chunk size and dtype,
    # on the same scratch (the previous call's contents are left in it)
    small = kda_inputs.make_prefill([77, 0, 130, 5], 3, token_dtype=torch.float32,
                                    g_std=1.0, h0_std=0.1, chunk=32, seed=1202,
                                    name="ragged [77,0,130,5] H=3 fp32")
    _check(kda, small, torch.float32)


def test_noalloc_bf16_out_after_other_calls(kda):
    p = kda_inputs.make_prefill([333, 64, 1], 4, g_std=2.0, h0_std=0.1, chunk=64, seed=1203,
                                name="[333,64,1] H=4 bf16")
    _check(kda, p, torch.bfloat16)
