"""KDA forward for head sizes other than 128 (kda_recurrent_fwd) on the GPU.

The FlashKDA issue page ("Proposed scope") asks for arbitrary key/value
dimensions; the chunkwise path and the decode kernels are built for K = V = 128,
so these sizes run on the token-by-token kernel. Parity: against the fp64
oracle (which takes any K, V), element by element, at 1e-4 of the rms for fp32
tokens and 2e-2 for bf16 tokens (fp32 outputs, the literal metric), over
packed ragged sequences with initial states, sizes that are and are not
multiples of 16 (both the key lanes and the 16-row blocks end ragged), grouped
value heads, empty sequences, in-place state update as a batched decode, and
K = V = 128 against the chunkwise prefill. Sizes up to 128 also run on the
chunkwise prefill (kda_chunk_fwd over zero-padded copies in its workspace):
the same parity bar over chunk sizes 16/32/64, both dtypes, grouped heads, the
two stages called separately and the final state written over the initial one."""
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


def run(kda, p, *, o_dtype=torch.float32, h0=True, Hqk=None):
    d = prefill_to_device(p, DEV)
    q, k = d["q"], d["k"]
    if Hqk is not None:
        G = p.H // Hqk
        q, k = q[:, ::G].contiguous(), k[:, ::G].contiguous()
    o, ht = kda.recurrent_fwd(q, k, d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                              d["cu_seqlens"], scale=p.scale,
                              initial_state=d["h0"] if h0 else None, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, ht


def ref(p, h0=True, Hqk=None):
    q, k = p.q, p.k
    if Hqk is not None:
        G = p.H // Hqk
        q = q[:, ::G].repeat_interleave(G, dim=1)
        k = k[:, ::G].repeat_interleave(G, dim=1)
    return oracle.kda_recurrent(q, k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens,
                                scale=p.scale, h0=p.h0 if h0 else None)


@pytest.mark.parametrize("K,V", [(64, 64), (32, 96), (256, 48), (7, 5), (100, 130), (16, 256),
                                 (1, 1), (96, 40), (150, 200), (192, 72)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_general_parity(kda, K, V, dtype):
    p = kda_inputs.make_prefill([17, 33, 5, 40], 3, token_dtype=dtype, h0_std=0.1, seed=K * 7 + V,
                                K=K, V=V, g_std=2.0)
    o, ht = run(kda, p)
    ro, rht = ref(p)
    eo, eh = max_err_rel_rms(o, ro), max_err_rel_rms(ht, rht)
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    print("general K=%d V=%d %s: o %.3e ht %.3e" % (K, V, dtype, eo, eh), flush=True)
    assert eo <= tol and eh <= tol


def test_general_bf16_output(kda):
    p = kda_inputs.make_prefill([50, 31], 2, token_dtype=torch.bfloat16, h0_std=0.1, seed=3,
                                K=64, V=64)
    o, ht = run(kda, p, o_dtype=torch.bfloat16)
    ro, rht = ref(p)
    e = max_err_bf16_out(o, ro)
    print("general bf16 out: %.3e" % e, flush=True)
    assert o.dtype == torch.bfloat16 and e <= 2e-2 and max_err_rel_rms(ht, rht) <= 2e-2


def test_general_grouped_no_h0_empty(kda):
    p = kda_inputs.make_prefill([0, 21, 0, 16, 3], 4, token_dtype=torch.float32, h0_std=0.1,
                                seed=11, K=48, V=80)
    o, ht = run(kda, p, h0=False, Hqk=2)
    ro, rht = ref(p, h0=False, Hqk=2)
    assert max_err_rel_rms(o, ro) <= 1e-4 and max_err_rel_rms(ht, rht) <= 1e-4
    assert torch.count_nonzero(ht[0]) == 0 and torch.count_nonzero(ht[2]) == 0


def test_general_empty_sequence_copies_state(kda):
    p = kda_inputs.make_prefill([0, 9], 2, token_dtype=torch.float32, h0_std=0.1, seed=5,
                                K=24, V=40)
    o, ht = run(kda, p)
    assert torch.equal(ht[0].cpu(), p.h0[0])


def test_general_decode_in_place(kda):
    """A batched decode step: every sequence one token long, state updated in place,
    repeated over a few steps; equals the oracle's decode steps."""
    d = kda_inputs.make_decode(6, 3, 4, seed=21, K=64, V=96)
    state = d.state.to(DEV).clone()
    cu = torch.arange(7, dtype=torch.int64, device=DEV)
    outs = []
    for st in d.steps:
        o, ht = kda.recurrent_fwd(st["q"].to(DEV), st["k"].to(DEV), st["v"].to(DEV),
                                  st["g"].to(DEV), st["beta_raw"].to(DEV), d.A_log.to(DEV),
                                  d.dt_bias.to(DEV), cu, scale=d.scale, initial_state=state,
                                  final_state=state, o_dtype=torch.float32)
        assert ht is state
        outs.append(o)
    torch.cuda.synchronize()
    ref_outs, ref_state = oracle.kda_decode_steps(d.steps, d.state, d.A_log, d.dt_bias,
                                                  scale=d.scale)
    eo = max(max_err_rel_rms(a, b) for a, b in zip(outs, ref_outs))
    eh = max_err_rel_rms(state, ref_state)
    print("general decode in place: o %.3e state %.3e" % (eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2


def test_general_matches_chunked_at_128(kda):
    """At K = V = 128 the token-by-token kernel and the chunkwise prefill compute
    the same function; with fp32 tokens both are within 1e-4 of each other."""
    p = kda_inputs.make_prefill([70, 33], 2, token_dtype=torch.float32, h0_std=0.1, seed=8, chunk=32)
    d = prefill_to_device(p, DEV)
    o1, h1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                           d["cu_seqlens"], scale=p.scale, chunk_size=32, initial_state=d["h0"])
    o2, h2 = run(kda, p)
    ro, rht = ref(p)
    assert max_err_rel_rms(o2, ro) <= 1e-4 and max_err_rel_rms(h2, rht) <= 1e-4
    assert max_err_rel_rms(o1, o2.cpu().double().numpy()) <= 2e-4


def test_general_repeats_bitwise(kda):
    p = kda_inputs.make_prefill([40, 7], 2, token_dtype=torch.bfloat16, h0_std=0.1, seed=9,
                                K=96, V=32)
    o1, h1 = run(kda, p)
    o2, h2 = run(kda, p)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def run_chunked(kda, p, chunk, *, Hqk=None, h0=True, o_dtype=torch.float32, stages=False,
                in_place=False):
    d = prefill_to_device(p, DEV)
    q, k = d["q"], d["k"]
    if Hqk is not None:
        G = p.H // Hqk
        q, k = q[:, ::G].contiguous(), k[:, ::G].contiguous()
    st0 = d["h0"] if h0 else None
    kw = dict(scale=p.scale, chunk_size=chunk, initial_state=st0, o_dtype=o_dtype)
    if in_place:
        kw["final_state"] = st0
    args = (q, k, d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"], d["cu_seqlens"])
    if stages:
        ws = kda.Workspace(DEV)
        o, ht = kda.chunk_fwd(*args, workspace=ws, stage="intra", **kw)
        o, ht = kda.chunk_fwd(*args, workspace=ws, stage="inter", out=o, final_state=ht,
                              **{x: y for x, y in kw.items() if x != "final_state"})
    else:
        o, ht = kda.chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    return o, ht


@pytest.mark.parametrize("K,V,dtype,chunk", [
    (64, 64, torch.bfloat16, 64), (64, 64, torch.float32, 32), (32, 96, torch.bfloat16, 64),
    (100, 128, torch.float32, 16), (128, 48, torch.bfloat16, 64), (7, 5, torch.float32, 16),
    (1, 1, torch.bfloat16, 32), (96, 17, torch.bfloat16, 16)])
def test_chunked_below_128(kda, K, V, dtype, chunk):
    p = kda_inputs.make_prefill([17, 33, 5, 70, 0, 64], 3, token_dtype=dtype, h0_std=0.1,
                                seed=K * 3 + V + chunk, K=K, V=V, g_std=2.0, chunk=chunk)
    o, ht = run_chunked(kda, p, chunk)
    ro, rht = ref(p)
    eo, eh = max_err_rel_rms(o, ro), max_err_rel_rms(ht, rht)
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    print("chunked K=%d V=%d %s C=%d: o %.3e ht %.3e" % (K, V, dtype, chunk, eo, eh), flush=True)
    assert o.shape == (p.T, 3, V) and ht.shape == (6, 3, V, K)
    assert eo <= tol and eh <= tol


def test_chunked_below_128_variants(kda):
    """Grouped heads without initial states; the two stages called separately;
    the final state written over the initial one; bf16 output."""
    p = kda_inputs.make_prefill([40, 3, 90], 4, token_dtype=torch.bfloat16, h0_std=0.1, seed=31,
                                K=64, V=80)
    o, ht = run_chunked(kda, p, 64, Hqk=2, h0=False)
    ro, rht = ref(p, h0=False, Hqk=2)
    assert max_err_rel_rms(o, ro) <= 2e-2 and max_err_rel_rms(ht, rht) <= 2e-2
    ro, rht = ref(p)
    o1, h1 = run_chunked(kda, p, 32)
    o2, h2 = run_chunked(kda, p, 32, stages=True)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o3, h3 = run_chunked(kda, p, 32, in_place=True)
    assert torch.equal(o1, o3) and torch.equal(h1, h3)
    o4, _ = run_chunked(kda, p, 32, o_dtype=torch.bfloat16)
    assert max_err_bf16_out(o4, ro) <= 2e-2 and max_err_rel_rms(h1, rht) <= 2e-2


def test_chunked_below_128_matches_recurrent(kda):
    """Both paths compute the same function for K, V below 128 (fp32 tokens)."""
    p = kda_inputs.make_prefill([130, 61], 2, token_dtype=torch.float32, h0_std=0.1, seed=33,
                                K=64, V=64, chunk=64)
    o1, h1 = run_chunked(kda, p, 64)
    o2, h2 = run(kda, p)
    assert max_err_rel_rms(o1, o2.cpu().double().numpy()) <= 2e-4
    assert max_err_rel_rms(h1, h2.cpu().double().numpy()) <= 2e-4


@pytest.mark.parametrize("K,V,Hqk", [(64, 96, None), (48, 48, 1), (200, 16, None)])
def test_decode_step_other_sizes(kda, K, V, Hqk):
    """kda_decode_step (and its grouped form) at head sizes other than 128: the
    state updated in place over several steps, against the oracle's steps."""
    d = kda_inputs.make_decode(5, 3, 4, seed=K + V, K=K, V=V)
    G = 3 if Hqk is None else 3 // Hqk
    state = d.state.to(DEV).clone()
    outs = []
    for st in d.steps:
        q, k = st["q"].to(DEV), st["k"].to(DEV)
        if Hqk is not None:
            q, k = q[:, ::G].contiguous(), k[:, ::G].contiguous()
        outs.append(kda.decode_step(q, k, st["v"].to(DEV), st["g"].to(DEV),
                                    st["beta_raw"].to(DEV), d.A_log.to(DEV), d.dt_bias.to(DEV),
                                    state, scale=d.scale, o_dtype=torch.float32))
    torch.cuda.synchronize()
    steps = d.steps
    if Hqk is not None:
        steps = [dict(st, q=st["q"][:, ::G].repeat_interleave(G, dim=1),
                      k=st["k"][:, ::G].repeat_interleave(G, dim=1)) for st in d.steps]
    ref_outs, ref_state = oracle.kda_decode_steps(steps, d.state, d.A_log, d.dt_bias,
                                                  scale=d.scale)
    eo = max(max_err_rel_rms(a, b) for a, b in zip(outs, ref_outs))
    eh = max_err_rel_rms(state, ref_state)
    print("decode K=%d V=%d: o %.3e state %.3e" % (K, V, eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2


@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_decode_other_sizes_with_epilogue(kda, o_dtype):
    """The decode step with the output epilogue at K = 64, V = 96 (the epilogue as a
    second pass over o): against the oracle's decode steps followed by the
    oracle's norm and gate, over a state pool with a padding request."""
    B, H, K, V = 4, 3, 64, 96
    d = kda_inputs.make_decode(B, H, 3, seed=61, K=K, V=V)
    gen = torch.Generator().manual_seed(62)
    slots = torch.tensor([2, -1, 0, 5], dtype=torch.int32)
    pool = (torch.randn(6, H, V, K, generator=gen) * 0.1)
    w = torch.rand(V, generator=gen) + 0.5
    pool_d = pool.to(DEV)
    live = [0, 2, 3]
    ref_state = pool[slots[live].long()].double().numpy()
    for i, st in enumerate(d.steps):
        z = (torch.randn(B, H, V, generator=gen) * 2.0).to(st["q"].dtype)
        y = kda.decode_step(*(st[n].to(DEV) for n in ("q", "k", "v", "g", "beta_raw")),
                            d.A_log.to(DEV), d.dt_bias.to(DEV), pool_d, scale=d.scale,
                            o_dtype=o_dtype, gate=z.to(DEV), norm_weight=w.to(DEV),
                            slot_idx=slots.to(DEV))
        torch.cuda.synchronize()
        sub = {n: st[n][live] for n in st}
        ro, ref_state = oracle.kda_decode_steps([sub], ref_state, d.A_log, d.dt_bias,
                                                scale=d.scale)
        ry = oracle.output_norm_gate(ro[0], z[live], w, eps=kda.NORM_EPS)
        e = (max_err_bf16_out(y[live], ry) if o_dtype == torch.bfloat16
             else max_err_rel_rms(y[live], ry))
        print("gated decode K=%d V=%d step %d: %.3e" % (K, V, i, e), flush=True)
        assert e <= 2e-2 and torch.count_nonzero(y[1]) == 0
    assert max_err_rel_rms(pool_d[[2, 0, 5]], ref_state) <= 2e-2


def test_decode_other_sizes_state_pool(kda):
    """The serving decode over a state pool at K = 48, V = 80: request b uses pool
    entry slot_idx[b]; the result equals the plain step on the gathered states,
    bit for bit, the other pool entries are untouched and a padding request
    (slot -1) gets zero outputs."""
    B, H, S, K, V = 5, 3, 9, 48, 80
    d = kda_inputs.make_decode(B, H, 2, seed=77, K=K, V=V)
    gen = torch.Generator().manual_seed(78)
    pool = (torch.randn(S, H, V, K, generator=gen) * 0.1).to(DEV)
    slots = torch.tensor([4, 0, -1, 7, 2], dtype=torch.int32, device=DEV)
    ref_state = pool[slots.clamp(min=0).long()].clone()
    pool0 = pool.clone()
    for st in d.steps:
        args = [st[n].to(DEV) for n in ("q", "k", "v", "g", "beta_raw")]
        o = kda.decode_step(*args, d.A_log.to(DEV), d.dt_bias.to(DEV), pool, scale=d.scale,
                            o_dtype=torch.float32, slot_idx=slots)
        o_ref = kda.decode_step(*args, d.A_log.to(DEV), d.dt_bias.to(DEV), ref_state,
                                scale=d.scale, o_dtype=torch.float32)
        torch.cuda.synchronize()
        live = [0, 1, 3, 4]
        assert torch.equal(o[live], o_ref[live])
        assert torch.count_nonzero(o[2]) == 0
    for b, sl in ((0, 4), (1, 0), (3, 7), (4, 2)):
        assert torch.equal(pool[sl], ref_state[b])
    for sl in (1, 3, 5, 6, 8):
        assert torch.equal(pool[sl], pool0[sl])


@pytest.mark.parametrize("K,V,dtype,Hqk", [(64, 64, torch.bfloat16, None),
                                           (32, 96, torch.float32, None),
                                           (100, 20, torch.bfloat16, 1)])
def test_backward_below_128(kda, K, V, dtype, Hqk):
    """kda_backward at head sizes below 128 (zero-padded inside the library)
    against the fp64 backward oracle, every gradient to 1e-4 of its rms."""
    p = kda_inputs.make_prefill([20, 0, 45], 3, token_dtype=dtype, h0_std=0.1, seed=K + 2 * V,
                                K=K, V=V)
    gen = torch.Generator().manual_seed(K * V)
    do = torch.randn(p.T, p.H, V, generator=gen).to(dtype)
    dht = torch.randn(p.N, p.H, V, K, generator=gen) * 0.1
    d = prefill_to_device(p, DEV)
    q, k = d["q"], d["k"]
    qr, kr = p.q, p.k
    if Hqk is not None:
        G = p.H // Hqk
        q, k = q[:, ::G].contiguous(), k[:, ::G].contiguous()
        qr = p.q[:, ::G].repeat_interleave(G, dim=1)
        kr = p.k[:, ::G].repeat_interleave(G, dim=1)
    r = kda.backward(q, k, d["v"], d["g"], d["beta_raw"], d["A_log"], d["dt_bias"],
                     d["cu_seqlens"], do.to(DEV), scale=p.scale, initial_state=d["h0"],
                     d_final_state=dht.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.kda_backward(qr, kr, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens, do,
                              scale=p.scale, h0=p.h0, dht=dht)
    if Hqk is not None:
        G = p.H // Hqk
        for key in ("dq", "dk"):
            ref[key] = ref[key].reshape(p.T, Hqk, G, K).sum(axis=2)
    worst = {key: max_err_rel_rms(r[key], ref[key]) for key in
             ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dh0")}
    print("backward K=%d V=%d: %s" % (K, V, " ".join("%s=%.2e" % kv for kv in worst.items())),
          flush=True)
    assert r["dv"].shape == (p.T, p.H, V) and r["dh0"].shape == (p.N, p.H, V, K)
    assert max(worst.values()) <= 1e-4, worst
