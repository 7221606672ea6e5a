"""Serving forms (GPU): the decode step over a state pool with per-request slot
indices, and HIP-graph capture and replay of the decode and prefill calls.

Slot indexing only changes where each request's state lives, so its results
must equal, bit for bit, the plain decode step on the gathered states; graph
replays must equal eager calls bit for bit (the kernels are deterministic).
Both forms are also checked directly against the fp64 oracle: the slot-indexed
step's outputs and updated pool entries over consecutive steps, and every graph
replay of the prefill and of the slot-indexed decode."""
import pytest
import torch

import kda_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def decode_inputs(B, H, seed, dtype=torch.bfloat16):
    d = kda_inputs.make_decode(B, H, 1, seed=seed)
    st = d.steps[0]
    cv = lambda x: x.to(dtype).to(DEV)
    return d, (cv(st["q"]), cv(st["k"]), cv(st["v"]), st["g"].to(DEV), st["beta_raw"].to(DEV),
               d.A_log.to(DEV), d.dt_bias.to(DEV))


@pytest.mark.parametrize("gated", [False, True])
def test_decode_slots_equal_gathered_states(kda, gated):
    H, S = 3, 10
    slots = [7, 2, -1, 9, 0, 15]                        # -1 and 15 (>= S) are padding
    B = len(slots)
    d, args = decode_inputs(B, H, seed=51)
    gen = torch.Generator().manual_seed(52)
    pool = (torch.randn(S, H, 128, 128, generator=gen) * 0.1).to(DEV)
    pool0 = pool.clone()
    kw = {}
    if gated:
        z, w = kda_inputs.make_epilogue((B, H, 128), seed=53)
        kw = dict(gate=z.to(DEV), norm_weight=w.to(DEV))
    idx = torch.tensor(slots, dtype=torch.int32, device=DEV)
    y = kda.decode_step(*args, pool, scale=d.scale, slot_idx=idx, **kw)
    # reference: the plain step on the gathered states (padding rows gather slot 0)
    gather = torch.tensor([s if 0 <= s < S else 0 for s in slots], device=DEV)
    states = pool0[gather].clone()
    ref = kda.decode_step(*args, states, scale=d.scale, **kw)
    torch.cuda.synchronize()
    valid = [i for i, s in enumerate(slots) if 0 <= s < S]
    pad = [i for i, s in enumerate(slots) if not 0 <= s < S]
    assert torch.equal(y[valid], ref[valid])
    assert torch.all(y[pad] == 0)
    for i in valid:
        assert torch.equal(pool[slots[i]], states[i])
    untouched = [s for s in range(S) if s not in slots]
    assert torch.equal(pool[untouched], pool0[untouched])


def test_graph_capture_decode_slots(kda):
    """Capture the gated slot-indexed step once, replay it on new inputs copied
    into the captured buffers; every replay equals an eager call."""
    H, S, B = 4, 12, 8
    d, args = decode_inputs(B, H, seed=54)
    static = [a.clone() for a in args]
    gen = torch.Generator().manual_seed(55)
    pool = (torch.randn(S, H, 128, 128, generator=gen) * 0.1).to(DEV)
    idx = torch.randperm(S, generator=gen)[:B].to(torch.int32).to(DEV)
    z, w = (t.to(DEV) for t in kda_inputs.make_epilogue((B, H, 128), seed=56))
    out = torch.empty(B, H, 128, dtype=torch.bfloat16, device=DEV)

    def call(a, p, i, zz):
        return kda.decode_step(*a, p, scale=d.scale, slot_idx=i, gate=zz, norm_weight=w, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(static, pool.clone(), idx, z)              # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    gpool = pool.clone()
    with torch.cuda.graph(graph):
        call(static, gpool, idx, z)
    torch.cuda.synchronize()
    ref_pool = pool.clone()                             # the eager twin of gpool
    gpool.copy_(pool)
    for rep in range(4):
        _, fresh = decode_inputs(B, H, seed=60 + rep)
        for dst, src in zip(static, fresh):
            dst.copy_(src)
        idx.copy_(torch.randperm(S, generator=gen)[:B].to(torch.int32).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_graph = out.clone()
        eager = call(fresh, ref_pool, idx, z).clone()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_graph, eager), rep
        assert torch.equal(gpool, ref_pool), rep


@pytest.mark.parametrize("chunk,K,V", [(32, 128, 128), (64, 128, 128), (64, 64, 48)])
def test_graph_capture_prefill(kda, chunk, K, V):
    """Capture chunk_fwd (intra + inter, caller workspace; below 128 also the
    zero-fill copies) and replay it on new token values; every replay equals an
    eager call bit for bit."""
    lengths = [300, 0, 211, 64]
    p = kda_inputs.make_prefill(lengths, 4, h0_std=0.1, chunk=chunk, seed=70, K=K, V=V)
    names = ("q", "k", "v", "g", "beta_raw", "A_log", "dt_bias", "cu_seqlens", "h0")
    static = {n: getattr(p, n).to(DEV).clone() for n in names}
    ws = kda.Workspace(DEV)
    o = torch.empty(p.T, 4, V, dtype=torch.bfloat16, device=DEV)
    ht = torch.empty(len(lengths), 4, V, K, dtype=torch.float32, device=DEV)

    def call(t, out_o, out_h, w):
        return kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta_raw"], t["A_log"],
                             t["dt_bias"], t["cu_seqlens"], scale=p.scale, chunk_size=chunk,
                             initial_state=t["h0"], out=out_o, final_state=out_h, workspace=w)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(static, o, ht, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, o, ht, ws)
    torch.cuda.synchronize()
    ws2 = kda.Workspace(DEV)
    for rep in range(3):
        q = kda_inputs.make_prefill(lengths, 4, h0_std=0.1, chunk=chunk, seed=80 + rep, K=K, V=V)
        fresh = {n: getattr(q, n).to(DEV) for n in names}
        for n in names:
            static[n].copy_(fresh[n])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_g, h_g = o.clone(), ht.clone()
        o_e, h_e = call(fresh, None, None, ws2)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(h_g, h_e), rep


@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_graph_capture_prefill_gated(kda, o_dtype):
    """Capture the gated prefill with the epilogue fused into the inter kernel
    (the exchange words' fill, intra, inter with the fifth wave) and replay it on
    new tokens and gate logits; every replay equals an eager call bit for bit
    (the exchange words are cleared on every replay, so a replay never reads an
    earlier one's row sums)."""
    lengths = [300, 0, 211, 64]
    H = 4
    p = kda_inputs.make_prefill(lengths, H, h0_std=0.1, chunk=64, seed=71)
    names = ("q", "k", "v", "g", "beta_raw", "A_log", "dt_bias", "cu_seqlens", "h0")
    static = {n: getattr(p, n).to(DEV).clone() for n in names}
    z, w = kda_inputs.make_epilogue((p.T, H, 128), seed=72)
    static["z"], static["w"] = z.to(DEV), w.to(DEV)
    ws = kda.Workspace(DEV)
    y = torch.empty(p.T, H, 128, dtype=o_dtype, device=DEV)
    ht = torch.empty(len(lengths), H, 128, 128, dtype=torch.float32, device=DEV)

    def call(t, out_y, out_h, wsp):
        return kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta_raw"], t["A_log"],
                             t["dt_bias"], t["cu_seqlens"], scale=p.scale, chunk_size=64,
                             initial_state=t["h0"], out=out_y, final_state=out_h, workspace=wsp,
                             o_dtype=o_dtype, gate=t["z"], norm_weight=t["w"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(static, y, ht, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, y, ht, ws)
    torch.cuda.synchronize()
    ws2 = kda.Workspace(DEV)
    for rep in range(3):
        q = kda_inputs.make_prefill(lengths, H, h0_std=0.1, chunk=64, seed=90 + rep)
        fresh = {n: getattr(q, n).to(DEV) for n in names}
        z2, w2 = kda_inputs.make_epilogue((p.T, H, 128), seed=95 + rep)
        fresh["z"], fresh["w"] = z2.to(DEV), w2.to(DEV)
        for n in fresh:
            static[n].copy_(fresh[n])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_g, h_g = y.clone(), ht.clone()
        y_e, h_e = call(fresh, None, None, ws2)
        torch.cuda.synchronize()
        assert torch.isfinite(y_g.float()).all()
        assert torch.equal(y_g, y_e) and torch.equal(h_g, h_e), rep


# ---- the same serving forms anchored to the fp64 oracle -----------------------

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from helpers import max_err_bf16_out, max_err_rel_rms  # noqa: E402


@pytest.mark.parametrize("in_dtype,gated", [(torch.float32, False), (torch.bfloat16, False),
                                            (torch.bfloat16, True)])
def test_decode_slots_against_oracle(kda, in_dtype, gated):
    """Three consecutive slot-indexed steps over a pool (padding requests included,
    different slot lists per step): every valid request's output and the pool's
    updated entries against the oracle run on the gathered states; entries no
    request names stay untouched. fp32 outputs (the step computes in fp32):
    1e-5 of the rms; with the epilogue, y against the oracle's epilogue of its o."""
    H, S = 3, 10
    gen = torch.Generator().manual_seed(90)
    pool0 = torch.randn(S, H, 128, 128, generator=gen) * 0.1
    pool = pool0.to(DEV)
    ref_pool = pool0.double().numpy().copy()
    steps = [[7, 2, -1, 9, 0, 15], [2, 9, 4, 10, 7, -3], [0, 1, 2, 3, 4, 5]]
    for i, slots in enumerate(steps):
        B = len(slots)
        d = kda_inputs.make_decode(B, H, 1, seed=91 + i)
        st = d.steps[0]
        cv = lambda x: x.to(in_dtype)
        q, k, v = cv(st["q"]), cv(st["k"]), cv(st["v"])
        kw = {}
        if gated:
            z, w = kda_inputs.make_epilogue((B, H, 128), token_dtype=in_dtype, seed=95 + i)
            kw = dict(gate=z.to(DEV), norm_weight=w.to(DEV))
        idx = torch.tensor(slots, dtype=torch.int32, device=DEV)
        y = kda.decode_step(q.to(DEV), k.to(DEV), v.to(DEV), st["g"].to(DEV),
                            st["beta_raw"].to(DEV), d.A_log.to(DEV), d.dt_bias.to(DEV), pool,
                            scale=d.scale, slot_idx=idx, o_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        valid = [j for j, s in enumerate(slots) if 0 <= s < S]
        vs = [slots[j] for j in valid]
        sel = lambda x: x[valid]
        o_ref, h_ref = oracle.kda_recurrent(sel(q), sel(k), sel(v), sel(st["g"]),
                                            sel(st["beta_raw"]), d.A_log, d.dt_bias,
                                            torch.arange(len(valid) + 1), scale=d.scale,
                                            h0=ref_pool[vs])
        if gated:
            o_ref = oracle.output_norm_gate(o_ref, sel(z), w, eps=kda.NORM_EPS)
        ref_pool[vs] = h_ref
        e_o = max_err_rel_rms(y[valid], o_ref)
        e_s = max_err_rel_rms(pool, ref_pool)
        print("slots step %d %s gated=%s: o %.3e pool %.3e" % (i, in_dtype, gated, e_o, e_s),
              flush=True)
        assert e_o <= 1e-5 and e_s <= 1e-5
        pad = [j for j, s in enumerate(slots) if not 0 <= s < S]
        assert torch.all(y[pad] == 0)
    never = [s for s in range(S) if all(s not in sl for sl in steps)]
    assert torch.equal(pool[never].cpu(), pool0[never])


def test_graph_replays_against_oracle(kda):
    """Prefill and slot-indexed decode captured once and replayed on fresh inputs:
    every replay against the oracle (the prefill's bf16 output beyond its storage
    rounding at 2e-2, final states and the decode at the literal metric)."""
    lengths = [300, 0, 211, 64]
    p = kda_inputs.make_prefill(lengths, 4, h0_std=0.1, chunk=64, seed=100)
    names = ("q", "k", "v", "g", "beta_raw", "A_log", "dt_bias", "cu_seqlens", "h0")
    static = {n: getattr(p, n).to(DEV).clone() for n in names}
    ws = kda.Workspace(DEV)
    o = torch.empty(p.T, 4, 128, dtype=torch.bfloat16, device=DEV)
    ht = torch.empty(len(lengths), 4, 128, 128, dtype=torch.float32, device=DEV)

    def call(t):
        kda.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta_raw"], t["A_log"], t["dt_bias"],
                      t["cu_seqlens"], scale=p.scale, chunk_size=64, initial_state=t["h0"],
                      out=o, final_state=ht, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static)
    torch.cuda.synchronize()
    for rep in range(3):
        q = kda_inputs.make_prefill(lengths, 4, g_std=2.0, h0_std=0.1, chunk=64, seed=101 + rep)
        for n in names:
            static[n].copy_(getattr(q, n).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ref, h_ref = oracle.kda_recurrent(q.q, q.k, q.v, q.g, q.beta_raw, q.A_log, q.dt_bias,
                                            q.cu_seqlens, scale=q.scale, h0=q.h0)
        e_o, e_h = max_err_bf16_out(o, o_ref), max_err_rel_rms(ht, h_ref)
        print("prefill replay %d: o %.3e ht %.3e" % (rep, e_o, e_h), flush=True)
        assert e_o <= 2e-2 and e_h <= 2e-2
        _ = torch.zeros(1, device=DEV) + 1              # eager work between replays

    # decode over a pool, captured with its slot indices as a device tensor
    H, S, B = 4, 12, 8
    gen = torch.Generator().manual_seed(110)
    pool0 = torch.randn(S, H, 128, 128, generator=gen) * 0.1
    d0 = kda_inputs.make_decode(B, H, 1, seed=111)
    st0 = d0.steps[0]
    sd = [st0[n].to(DEV).clone() for n in ("q", "k", "v", "g", "beta_raw")]
    A_log, dt_bias = d0.A_log.to(DEV), d0.dt_bias.to(DEV)
    idx = torch.randperm(S, generator=gen)[:B].to(torch.int32).to(DEV)
    pool = pool0.to(DEV)
    out = torch.empty(B, H, 128, dtype=torch.float32, device=DEV)

    def dec():
        kda.decode_step(*sd, A_log, dt_bias, pool, scale=d0.scale, slot_idx=idx, out=out,
                        o_dtype=torch.float32)

    with torch.cuda.stream(s):
        dec()                                           # eager warm-up (updates the pool)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        dec()
    torch.cuda.synchronize()
    pool.copy_(pool0.to(DEV))
    ref_pool = pool0.double().numpy().copy()
    for rep in range(3):
        dr = kda_inputs.make_decode(B, H, 1, seed=112 + rep)
        for t, n in zip(sd, ("q", "k", "v", "g", "beta_raw")):
            t.copy_(dr.steps[0][n].to(DEV))
        sl = torch.randperm(S, generator=gen)[:B].to(torch.int32)
        idx.copy_(sl.to(DEV))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        st = dr.steps[0]
        o_ref, h_ref = oracle.kda_recurrent(st["q"], st["k"], st["v"], st["g"], st["beta_raw"],
                                            d0.A_log, d0.dt_bias, torch.arange(B + 1),
                                            scale=d0.scale, h0=ref_pool[sl.numpy()])
        ref_pool[sl.numpy()] = h_ref
        e_o, e_s = max_err_rel_rms(out, o_ref), max_err_rel_rms(pool, ref_pool)
        print("decode replay %d: o %.3e pool %.3e" % (rep, e_o, e_s), flush=True)
        assert e_o <= 1e-5 and e_s <= 1e-5
