"""Serving forms (GPU): the decode step over a state pool with per-request slot
indices, and HIP-graph capture and replay of the decode and prefill calls.

Slot indexing only changes where each request's state lives, so its results
must equal, bit for bit, the plain decode step on the gathered states; graph
replays must equal eager calls bit for bit (the kernels are deterministic)."""
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
