"""Grouped value heads (H value heads sharing H_qk q/k heads) on the GPU.

The grouped computation is, by definition, the ungrouped one with q and k
repeated H / H_qk times along the head axis. Checked three ways: the grouped
call equals the ungrouped GPU call on repeated q and k bit for bit (forward:
the same arithmetic, only the q/k addresses differ), and both the forward and
the backward agree with the fp64 oracle run on repeated q and k (the backward's
dq and dk summed over each group), to the tolerances of the ungrouped tests."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_rel_rms, prefill_to_device, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def grouped_problem(lengths, H, Hqk, dtype=torch.bfloat16, seed=0, chunk=32):
    p = kda_inputs.make_prefill(lengths, H, token_dtype=dtype, h0_std=0.1, chunk=chunk, seed=seed)
    G = H // Hqk
    # one q/k head per group: keep the group's first head
    p.q = p.q[:, ::G].contiguous()
    p.k = p.k[:, ::G].contiguous()
    return p, G


def rep(x, G):
    return x.repeat_interleave(G, dim=1).contiguous()


@pytest.mark.parametrize("H,Hqk,chunk", [(8, 2, 32), (8, 1, 64), (6, 3, 16)])
def test_prefill_grouped_matches_repeated(kda, H, Hqk, chunk):
    p, G = grouped_problem([17, 64, 5, 90], H, Hqk, seed=H * 10 + Hqk, chunk=chunk)
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                          d["cu_seqlens"], scale=p.scale, chunk_size=chunk, initial_state=d["h0"],
                          o_dtype=torch.float32)
    o2, ht2 = kda.chunk_fwd(rep(d["q"], G), rep(d["k"], G), d["v"], d["g"], d["beta_raw"],
                            d["A_log"], d["dt_bias"], d["cu_seqlens"], scale=p.scale,
                            chunk_size=chunk, initial_state=d["h0"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    ro, rht = oracle.kda_recurrent(rep(p.q, G), rep(p.k, G), p.v, p.g, p.beta_raw, p.A_log,
                                   p.dt_bias, p.cu_seqlens, scale=p.scale, h0=p.h0)
    e = max(max_err_rel_rms(o, ro), max_err_rel_rms(ht, rht))
    print("prefill grouped H=%d Hqk=%d: %.3e" % (H, Hqk, e), flush=True)
    assert e <= 2e-2


@pytest.mark.parametrize("with_slots,gated", [(False, False), (True, False), (True, True)])
def test_decode_grouped_matches_repeated(kda, with_slots, gated):
    B, H, Hqk = 16, 8, 2
    G = H // Hqk
    d = kda_inputs.make_decode(B, H, 1, seed=77)
    st = {kk: vv.to(DEV) for kk, vv in d.steps[0].items()}
    q, k = st["q"][:, ::G].contiguous(), st["k"][:, ::G].contiguous()
    S = d.state.to(DEV)
    kw, slot = {}, None
    if gated:
        z, w = kda_inputs.make_epilogue((B, H, 128), seed=78)
        kw = dict(gate=z.to(DEV), norm_weight=w.to(DEV))
    if with_slots:
        pool = torch.zeros(B + 3, H, 128, 128, device=DEV)
        perm = torch.randperm(B + 3, generator=torch.Generator().manual_seed(79))[:B]
        pool[perm.to(DEV)] = S
        slot = perm.to(torch.int32).to(DEV)
        pool2 = pool.clone()
        o = kda.decode_step(q, k, st["v"], st["g"], st["beta_raw"], d.A_log.to(DEV),
                            d.dt_bias.to(DEV), pool, scale=d.scale, slot_idx=slot, **kw)
        o2 = kda.decode_step(rep(q, G), rep(k, G), st["v"], st["g"], st["beta_raw"],
                             d.A_log.to(DEV), d.dt_bias.to(DEV), pool2, scale=d.scale,
                             slot_idx=slot, **kw)
        torch.cuda.synchronize()
        assert torch.equal(pool, pool2)
    else:
        S2 = S.clone()
        o = kda.decode_step(q, k, st["v"], st["g"], st["beta_raw"], d.A_log.to(DEV),
                            d.dt_bias.to(DEV), S, scale=d.scale, **kw)
        o2 = kda.decode_step(rep(q, G), rep(k, G), st["v"], st["g"], st["beta_raw"],
                             d.A_log.to(DEV), d.dt_bias.to(DEV), S2, scale=d.scale, **kw)
        torch.cuda.synchronize()
        assert torch.equal(S, S2)
    assert torch.equal(o, o2)
    if not gated:
        ro, _ = oracle.kda_recurrent(rep(q.cpu(), G), rep(k.cpu(), G), st["v"].cpu(),
                                     st["g"].cpu(), st["beta_raw"].cpu(), d.A_log, d.dt_bias,
                                     torch.arange(B + 1), scale=d.scale, h0=d.state)
        assert max_err_rel_rms(o, ro) <= 2e-2


@pytest.mark.parametrize("H,Hqk", [(8, 2), (4, 1)])
def test_backward_grouped_matches_oracle(kda, H, Hqk):
    p, G = grouped_problem([17, 40, 0, 33], H, Hqk, seed=90 + H)
    gen = torch.Generator().manual_seed(91)
    do = torch.randn(p.T, H, 128, generator=gen).to(torch.bfloat16)
    dht = torch.randn(p.N, H, 128, 128, generator=gen) * 0.1
    d = prefill_to_device(p, DEV)
    r = kda.backward(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                     d["cu_seqlens"], do.to(DEV), scale=p.scale, initial_state=d["h0"],
                     d_final_state=dht.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.kda_backward(rep(p.q, G), rep(p.k, G), p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                              p.cu_seqlens, do, scale=p.scale, h0=p.h0, dht=dht)
    T = p.T
    for key in ("dq", "dk"):
        ref[key] = ref[key].reshape(T, H // G, G, 128).sum(axis=2)
    worst = {key: max_err_rel_rms(r[key], ref[key]) for key in
             ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dh0")}
    print("backward grouped H=%d Hqk=%d: %s" % (H, Hqk, worst), flush=True)
    assert tuple(r["dq"].shape) == (T, Hqk, 128)
    assert max(worst.values()) <= 1e-4, worst
