"""Parity of libkda's q/k/v front end (causal depthwise short conv + SiLU over
packed sequences, carried-in and final conv states) with the fp64 oracle (GPU).

Tolerance, per element, from the arithmetic: the kernel sums W products in
fp32 and evaluates SiLU with the hardware exp2 and reciprocal, so its fp32
result lies within 6e-7 * A + 5e-7 * |y| of the exact value, where
A = sum_i |w_i| * max|x| bounds the pre-activation's terms (a few fp32 roundings
of A, a few ulp of the sigmoid); bf16 results may add half a bf16 spacing of
the stored value (the output's own rounding). Final conv states are copies of
inputs and must match bit for bit."""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import bf16_half_ulp, max_err_bf16_out, prefill_to_device, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


def check_y(y, ref, x, w, state):
    """Elementwise bound above; returns the worst excess ratio (<= 1 passes)."""
    yg = to_np(y)
    xmax = float(np.max(np.abs(to_np(x)))) if x.numel() else 0.0
    if state is not None and state.numel():
        xmax = max(xmax, float(np.max(np.abs(to_np(state)))))
    A = np.sum(np.abs(to_np(w)), axis=-1) * xmax                  # [H, D]
    tol = 6e-7 * A[None] + 5e-7 * np.abs(ref) + 1e-30
    if y.dtype == torch.bfloat16:
        tol = tol + bf16_half_ulp(yg)
    return float(np.max(np.abs(yg - ref) / tol)) if ref.size else 0.0


def run(kda, x, w, cu, state, *, final=True, in_place=False, x_dev=None):
    xd = x.to(DEV) if x_dev is None else x_dev
    sd = None if state is None else state.to(DEV)
    y, f = kda.short_conv(xd, w.to(DEV), cu.to(DEV), initial_state=sd,
                          output_final_state=final and not in_place,
                          final_state=sd if in_place else None)
    torch.cuda.synchronize()
    return y, f


LENGTHS = [1, 2, 3, 0, 5, 40, 33, 100, 0]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("with_state", [False, True])
def test_short_conv_ragged_matches_oracle(kda, dtype, W, with_state):
    # sequences shorter than W - 1, empty ones (also last), one spanning strips
    x, w, cu, st = kda_inputs.make_short_conv(LENGTHS, 3, W, token_dtype=dtype,
                                              with_state=with_state, seed=40 + W)
    y, f = run(kda, x, w, cu, st)
    ref, fref = oracle.short_conv_silu(x, w, cu, state=st)
    r = check_y(y, ref, x, w, st)
    print("short_conv %s W=%d state=%s: worst/tol %.3f" % (dtype, W, with_state, r), flush=True)
    assert y.dtype == dtype and tuple(y.shape) == tuple(x.shape)
    assert r <= 1.0
    assert tuple(f.shape) == (len(LENGTHS), W - 1, 3, 128)
    np.testing.assert_array_equal(to_np(f), fref)


@pytest.mark.parametrize("lengths", [
    [0, 0, 16, 0, 16, 0, 5, 0],     # empty sequences before the first token, at strip starts, last
    [48, 20],                       # a sequence ending exactly at a strip end (not the last strip)
    [48],                           # ... and at the end of the input
    [16, 16, 16, 3],                # every sequence start on a strip start
    [2, 1, 1, 2, 1, 40],            # starts closer together than the kernel size
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W", [2, 4])
def test_short_conv_sequence_edges(kda, lengths, dtype, W):
    for with_state in (False, True):
        x, w, cu, st = kda_inputs.make_short_conv(lengths, 2, W, token_dtype=dtype,
                                                  with_state=with_state, seed=60 + len(lengths))
        y, f = run(kda, x, w, cu, st)
        ref, fref = oracle.short_conv_silu(x, w, cu, state=st)
        assert check_y(y, ref, x, w, st) <= 1.0, (lengths, with_state)
        np.testing.assert_array_equal(to_np(f), fref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_short_conv_several_channel_blocks(kda, dtype):
    # 20 heads = 2560 channels: one full block of 2048 channels and a partial one
    x, w, cu, st = kda_inputs.make_short_conv([70, 1, 129, 0, 57], 20, 4, token_dtype=dtype, seed=7)
    y, f = run(kda, x, w, cu, st)
    ref, fref = oracle.short_conv_silu(x, w, cu, state=st)
    assert check_y(y, ref, x, w, st) <= 1.0
    np.testing.assert_array_equal(to_np(f), fref)


def test_short_conv_strided_rows_of_a_fused_projection(kda):
    # x is the k slice of a [T, 3 * H * 128] projection output (row stride 3 H 128)
    H, W = 4, 4
    x, w, cu, st = kda_inputs.make_short_conv([31, 64, 9], H, W, seed=11)
    T = x.shape[0]
    fused = torch.randn(T, 3, H, 128, generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    fused[:, 1] = x
    fd = fused.to(DEV)
    xs = fd[:, 1]                                     # [T, H, 128], stride(0) = 3 H 128
    assert xs.stride(0) == 3 * H * 128
    y, f = run(kda, x, w, cu, st, x_dev=xs)
    ref, fref = oracle.short_conv_silu(x, w, cu, state=st)
    assert check_y(y, ref, x, w, st) <= 1.0
    np.testing.assert_array_equal(to_np(f), fref)


def test_short_conv_state_updated_in_place_and_chained(kda):
    # split every sequence in two; the second call continues from the first
    # call's final state, held in the same buffer (updated in place)
    H, W = 2, 4
    lens = [50, 2, 0, 17]
    x, w, cu, st = kda_inputs.make_short_conv(lens, H, W, seed=13)
    ref, fref = oracle.short_conv_silu(x, w, cu, state=st)
    cut = [n // 2 + (n % 3) if n else 0 for n in lens]
    cut = [min(c, n) for c, n in zip(cut, lens)]
    pa = [x[cu[i]:cu[i] + cut[i]] for i in range(len(lens))]
    pb = [x[cu[i] + cut[i]:cu[i + 1]] for i in range(len(lens))]
    cua = torch.tensor([0] + list(np.cumsum(cut)), dtype=torch.int64)
    cub = torch.tensor([0] + list(np.cumsum([n - c for n, c in zip(lens, cut)])), dtype=torch.int64)
    sd = st.to(DEV)
    ya, _ = kda.short_conv(torch.cat(pa).to(DEV), w.to(DEV), cua.to(DEV), initial_state=sd,
                           final_state=sd)
    yb, _ = kda.short_conv(torch.cat(pb).to(DEV), w.to(DEV), cub.to(DEV), initial_state=sd,
                           final_state=sd)
    torch.cuda.synchronize()
    ya, yb = to_np(ya), to_np(yb)
    got = np.concatenate([np.concatenate([ya[cua[i]:cua[i + 1]], yb[cub[i]:cub[i + 1]]])
                          for i in range(len(lens))])
    assert max_err_bf16_out(torch.from_numpy(got).to(torch.bfloat16), ref) < 1e-5
    np.testing.assert_array_equal(to_np(sd), fref)


def test_short_conv_no_tokens_passes_states_on(kda):
    x, w, cu, st = kda_inputs.make_short_conv([0, 0, 0], 2, 3, seed=14)
    y, f = run(kda, x, w, cu, st)
    assert y.shape[0] == 0
    np.testing.assert_array_equal(to_np(f), to_np(st))
    y, f = run(kda, x, w, cu, None)
    assert not np.any(to_np(f))


@pytest.mark.parametrize("lengths", [[8192], kda_inputs.LARGE_VARLEN_LENGTHS])
def test_short_conv_full_size(kda, lengths):
    # the prefill workload's q at full size (T = 8192, H = 96, bf16, W = 4),
    # checked against the oracle on every element
    x, w, cu, st = kda_inputs.make_short_conv(lengths, 96, 4, seed=15)
    y, f = run(kda, x, w, cu, st)
    ref, fref = oracle.short_conv_silu(x, w, cu, state=st)
    r = check_y(y, ref, x, w, st)
    print("short_conv full size %d seqs: worst/tol %.3f" % (len(lengths), r), flush=True)
    assert r <= 1.0
    np.testing.assert_array_equal(to_np(f), fref)


def test_front_end_then_prefill_then_epilogue(kda):
    # the block's path on a small packed batch: short conv + SiLU on q, k, v,
    # chunkwise recurrence, output norm and gate; the oracle chain rounds its
    # conv outputs to bf16 (the storage type between the stages) and runs the
    # fp64 recurrence; held to the prefill's bf16 bound
    lens, H, W = [17, 33, 65], 4, 4
    p = kda_inputs.make_prefill(lens, H, h0_std=0.1, chunk=32, seed=16)
    qkv_w = [kda_inputs.make_short_conv(lens, H, W, seed=17 + i)[1] for i in range(3)]
    d = prefill_to_device(p, DEV)
    conv = [kda.short_conv(d[n], qkv_w[i].to(DEV), d["cu_seqlens"])[0]
            for i, n in enumerate(("q", "k", "v"))]
    o, ht = kda.chunk_fwd(conv[0], conv[1], conv[2], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=p.chunk,
                          initial_state=d["h0"], o_dtype=torch.float32)
    z, nw = kda_inputs.make_epilogue(tuple(o.shape), token_dtype=torch.float32, seed=18)
    y = kda.output_norm_gate(o, z.to(DEV), nw.to(DEV), eps=kda.NORM_EPS)
    torch.cuda.synchronize()
    rc = [torch.from_numpy(oracle.short_conv_silu(t, qkv_w[i], p.cu_seqlens)[0]).to(torch.bfloat16)
          for i, t in enumerate((p.q, p.k, p.v))]
    ro, rht = oracle.kda_recurrent(rc[0], rc[1], rc[2], p.g, p.beta_raw, p.A_log, p.dt_bias,
                                   p.cu_seqlens, scale=p.scale, h0=p.h0)
    ry = oracle.output_norm_gate(ro, z, nw, eps=kda.NORM_EPS)
    from helpers import max_err_rel_rms
    e_o, e_y = max_err_rel_rms(o, ro), max_err_rel_rms(y, ry)
    print("front end + prefill + epilogue: o %.3e y %.3e" % (e_o, e_y), flush=True)
    assert e_o <= 2e-2 and e_y <= 2e-2
    assert max_err_rel_rms(ht, rht) <= 2e-2


def test_short_conv_state_pool_serving(kda):
    # a pool of conv states addressed per sequence: a prefill chunk of three
    # requests, then four decode steps of one token each over a shuffled subset
    # with a padding entry; against the oracle run per request with the pool
    # entry as its carried-in state
    H, W, S = 2, 4, 6
    C = H * 128
    gen = torch.Generator().manual_seed(21)
    pool = torch.randn(S, W - 1, H, 128, generator=gen).to(torch.bfloat16)
    w = kda_inputs.make_short_conv([1], H, W, seed=22)[1]
    ref_pool = pool.clone()
    pool_d = pool.to(DEV)
    calls = [([5, 1, 12], [4, 0, 2]), ([1, 1, 1], [2, 4, 0]), ([1, 1, 1, 1], [0, 9, 4, 2]),
             ([1, 1], [-1, 2]), ([1, 1, 1], [4, 0, 2])]
    for step, (lens, slots) in enumerate(calls):
        x = torch.randn(sum(lens), H, 128, generator=gen).to(torch.bfloat16)
        cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int64)
        idx = torch.tensor(slots, dtype=torch.int32)
        y, _ = kda.short_conv(x.to(DEV), w.to(DEV), cu.to(DEV), state_pool=pool_d,
                              slot_idx=idx.to(DEV))
        torch.cuda.synchronize()
        yg = to_np(y)
        for n, sl in enumerate(slots):
            s0, s1 = int(cu[n]), int(cu[n + 1])
            if not 0 <= sl < S:
                assert not np.any(yg[s0:s1]), (step, n)          # padding: zero outputs
                continue
            ry, rf = oracle.short_conv_silu(x[s0:s1], w, np.array([0, s1 - s0]),
                                            state=ref_pool[sl:sl + 1])
            assert check_y(y[s0:s1], ry, x[s0:s1], w, ref_pool[sl:sl + 1]) <= 1.0, (step, n)
            ref_pool[sl] = torch.from_numpy(rf[0]).to(torch.bfloat16)
        np.testing.assert_array_equal(to_np(pool_d), to_np(ref_pool))
