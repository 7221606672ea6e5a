"""Parity of libkda's chunkwise prefill with the fp64 CPU oracle (GPU).

Tolerance (the spec bar, max-abs error relative to the oracle's RMS):
1e-4 for fp32 inputs, 2e-2 for bf16 inputs, separately for o and the final
states. fp32 results are compared directly. A bf16-stored output is compared
after allowing its own storage rounding (half a bf16 ulp of each element, see
helpers.max_err_bf16_out); the raw error is reported too. The reason: the
outputs are heavy-tailed (max|o| ~ 16 rms), so rounding the exact result to
bf16 alone exceeds 2e-2 of the rms on the large workloads.
"""
import math

import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from helpers import max_err_bf16_out, max_err_rel_rms, prefill_to_device, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd as m
    return m


_ORACLE_CACHE = {}


def oracle_of(p, key=None):
    key = key or p.name
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = oracle.kda_recurrent(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log,
                                                  p.dt_bias, p.cu_seqlens, scale=p.scale,
                                                  h0=p.h0)
    return _ORACLE_CACHE[key]


def run_gpu(kda, p, chunk=None, o_dtype=None, **kw):
    d = prefill_to_device(p, DEV)
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale,
                          chunk_size=chunk or p.chunk, initial_state=d["h0"], o_dtype=o_dtype,
                          **kw)
    torch.cuda.synchronize()
    return o, ht


def check(p, o, ht, ref, label):
    o_ref, ht_ref = ref
    tol = TOL[p.q.dtype]
    e_ht = max_err_rel_rms(ht, ht_ref)
    if o.dtype == torch.bfloat16:
        e_o = max_err_bf16_out(o, o_ref)
        raw = max_err_rel_rms(o, o_ref)
    else:
        e_o = raw = max_err_rel_rms(o, o_ref)
    print("%s: o err %.3e (raw %.3e)  ht err %.3e  tol %.0e" % (label, e_o, raw, e_ht, tol),
          flush=True)
    assert np.all(np.isfinite(to_np(o))) and np.all(np.isfinite(to_np(ht)))
    assert e_o <= tol, (label, "o", e_o)
    assert e_ht <= tol, (label, "ht", e_ht)


# ---- the standard workloads ----------------------------------------------------

def test_small_fp32(kda):
    p = kda_inputs.small()
    o, ht = run_gpu(kda, p)
    check(p, o, ht, oracle_of(p), p.name)


def test_varlen_bf16(kda):
    p = kda_inputs.varlen()
    ref = oracle_of(p)
    o, ht = run_gpu(kda, p)
    check(p, o, ht, ref, p.name)
    o32, ht32 = run_gpu(kda, p, o_dtype=torch.float32)
    check(p, o32, ht32, ref, p.name + " fp32-out")


# ---- chunk size, edge cases, invariants ---------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_sizes_ragged(kda, dtype, chunk):
    """Several tiles, ragged tails, a zero-length and a one-token sequence."""
    p = kda_inputs.make_prefill([1, 0, 77, 130, 64, 5], 3, token_dtype=dtype, g_std=2.0,
                                h0_std=0.1, chunk=chunk, seed=500 + chunk)
    ref = oracle_of(p, ("ragged", dtype, chunk))
    o, ht = run_gpu(kda, p, o_dtype=torch.float32)
    check(p, o, ht, ref, "ragged %s C=%d" % (dtype, chunk))
    # the zero-length sequence returns its initial state
    assert torch.equal(ht[1].cpu(), p.h0[1])


@pytest.mark.parametrize("g_std", [0.01, 0.5, 2.0, 8.0])
def test_gate_regimes(kda, g_std):
    """Weak to very strong decay (the page sweeps gate regimes 0.01 .. 2.0)."""
    p = kda_inputs.make_prefill([300, 211], 4, g_std=g_std, h0_std=0.1, chunk=64,
                                seed=600 + int(g_std * 100))
    ref = oracle_of(p, ("gate", g_std))
    o, ht = run_gpu(kda, p)
    check(p, o, ht, ref, "gate std %g" % g_std)


def test_no_initial_no_final(kda):
    p = kda_inputs.make_prefill([40, 90], 2, chunk=32, seed=700)
    ref = oracle_of(p, "nofinal")
    o, ht = run_gpu(kda, p, output_final_state=False)
    assert ht is None
    e = max_err_bf16_out(o, ref[0])
    assert e <= 2e-2


def test_empty_batch(kda):
    """T = 0: no output rows; final = initial."""
    p = kda_inputs.make_prefill([0, 0], 2, h0_std=1.0, chunk=64, seed=701)
    o, ht = run_gpu(kda, p)
    assert o.shape == (0, 2, 128)
    assert torch.equal(ht.cpu(), p.h0)


def test_final_state_aliases_initial(kda):
    p = kda_inputs.make_prefill([100, 37], 2, h0_std=0.1, chunk=32, seed=702)
    ref = oracle_of(p, "alias")
    d = prefill_to_device(p, DEV)
    state = d["h0"].clone()
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta_raw"], d["A_log"],
                          d["dt_bias"], d["cu_seqlens"], scale=p.scale, chunk_size=32,
                          initial_state=state, final_state=state)
    torch.cuda.synchronize()
    assert ht.data_ptr() == state.data_ptr()
    check(p, o, ht, ref, "aliased state")


def test_split_chaining(kda):
    """Two calls chained through the final state equal one call (checkpoint/resume)."""
    p = kda_inputs.make_prefill([333], 2, h0_std=0.1, chunk=64, seed=703)
    ref = oracle_of(p, "split")
    d = prefill_to_device(p, DEV)
    t = 150
    first = {k: (v[:t] if k not in ("A_log", "dt_bias", "cu_seqlens", "h0") else v)
             for k, v in d.items()}
    second = {k: (v[t:] if k not in ("A_log", "dt_bias", "cu_seqlens", "h0") else v)
              for k, v in d.items()}
    o1, h1 = kda.chunk_fwd(first["q"], first["k"], first["v"], first["g"], first["beta_raw"],
                           d["A_log"], d["dt_bias"], torch.tensor([0, t], device=DEV),
                           scale=p.scale, chunk_size=64, initial_state=d["h0"])
    o2, h2 = kda.chunk_fwd(second["q"], second["k"], second["v"], second["g"],
                           second["beta_raw"], d["A_log"], d["dt_bias"],
                           torch.tensor([0, 333 - t], device=DEV), scale=p.scale,
                           chunk_size=64, initial_state=h1)
    torch.cuda.synchronize()
    check(p, torch.cat([o1, o2]), h2, ref, "split at %d" % t)


def test_varlen_equals_separate_runs(kda):
    p = kda_inputs.make_prefill([65, 1, 129], 2, h0_std=0.1, chunk=64, seed=704)
    o, ht = run_gpu(kda, p, o_dtype=torch.float32)
    cu = p.cu_seqlens.tolist()
    for n in range(3):
        sub = kda_inputs.PrefillInputs("sub", p.q[cu[n]:cu[n + 1]], p.k[cu[n]:cu[n + 1]],
                                       p.v[cu[n]:cu[n + 1]], p.g[cu[n]:cu[n + 1]],
                                       p.beta_raw[cu[n]:cu[n + 1]], p.A_log, p.dt_bias,
                                       torch.tensor([0, cu[n + 1] - cu[n]]), p.h0[n:n + 1],
                                       64, p.scale)
        o1, ht1 = run_gpu(kda, sub, o_dtype=torch.float32)
        # same kernels, same per-sequence work: bitwise equal
        assert torch.equal(o1, o[cu[n]:cu[n + 1]])
        assert torch.equal(ht1, ht[n:n + 1])


def test_deterministic(kda):
    p = kda_inputs.make_prefill([500, 300], 4, h0_std=0.1, chunk=64, seed=705)
    o1, h1 = run_gpu(kda, p)
    o2, h2 = run_gpu(kda, p)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_large_values_fp16_scaling(kda):
    """v and h0 far outside fp16 range still work: power-of-two scaling of the
    unbounded operands keeps the fp16 products finite."""
    p = kda_inputs.make_prefill([200], 2, h0_std=0.1, chunk=64, seed=706)
    p.v = (p.v.float() * 1e6).to(torch.bfloat16)
    p.h0 = p.h0 * 1e6
    ref = oracle_of(p, "large values")
    o, ht = run_gpu(kda, p)
    check(p, o, ht, ref, "v, h0 x 1e6")


# ---- white-box: the intra-chunk stage against the oracle's chunk form ---------

def _kperm(g, e):
    return 4 * g + e if e < 4 else 16 + 4 * g + (e - 4)


def _tile_chan(kb, r):
    """Key channel of row r of a kg^T tile kb (record layout)."""
    return 32 * (kb // 2) + 8 * (r // 4) + 4 * (kb % 2) + r % 4


def unpack_record(raw: np.ndarray, C: int, precise: bool):
    """Decode one workspace record (layout documented in csrc/kda_internal.h)."""
    NB, CP = C // 16, max(C, 32)
    CS = CP // 32
    elt = np.float32 if precise else np.float16
    esz = 4 if precise else 2
    frag = 64 * 8 * esz
    off = 0

    def take(nfr):
        nonlocal off
        a = raw[off:off + nfr * frag].view(elt).astype(np.float64).reshape(nfr, 64, 8)
        off += nfr * frag
        return a

    Wf, Qf, Kf, Mf = take(NB * 4), take(NB * 4), take(8 * CS), take(NB * CS)
    gam = raw[off:off + 512].view(np.float32).astype(np.float64)
    off += 512
    ub_scale = float(raw[off:off + 4].view(np.float32)[0])
    off += 16
    ub = (raw[off:off + 8 * NB * 64 * 4 * esz].view(elt).astype(np.float64).reshape(8, NB, 64, 4)
          * ub_scale)
    W = np.zeros((C, 128)); QG = np.zeros((C, 128)); KG = np.zeros((CP, 128)); M = np.zeros((C, CP))
    UB = np.zeros((C, 128))
    for lane in range(64):
        r, g = lane % 16, lane // 16
        for e in range(8):
            kk = _kperm(g, e)                # k over t
            kc = 8 * g + e                   # k over key channels
            for tb in range(NB):
                for s in range(4):
                    W[16 * tb + r, 32 * s + kc] = -Wf[tb * 4 + s, lane, e]   # stored negated
                    QG[16 * tb + r, 32 * s + kc] = Qf[tb * 4 + s, lane, e]
                for s in range(CS):
                    if 2 * s <= tb:          # fragments above the diagonal are not stored
                        M[16 * tb + r, 32 * s + kk] = Mf[tb * CS + s, lane, e]
            for kb in range(8):
                for s in range(CS):
                    KG[32 * s + kk, _tile_chan(kb, r)] = Kf[kb * CS + s, lane, e]
        for vb in range(8):
            for tb in range(NB):
                for i in range(4):
                    UB[16 * tb + 4 * g + i, 16 * vb + r] = ub[vb, tb, lane, i]
    return dict(W=W, qg=QG, kg=KG[:C], M=M[:, :C], Gamma_C=gam, U_base=UB)


@pytest.mark.parametrize("dtype,chunk", [(torch.float32, 16), (torch.bfloat16, 32),
                                         (torch.bfloat16, 64), (torch.float32, 64)])
def test_intra_stage_matches_chunk_form(kda, dtype, chunk):
    p = kda_inputs.make_prefill([chunk + 9, 2 * chunk], 2, token_dtype=dtype, g_std=2.0,
                                chunk=chunk, seed=800 + chunk)
    ws = kda.Workspace(DEV)
    run_gpu(kda, p, workspace=ws)
    _, _, saved = oracle.kda_chunked(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                     p.cu_seqlens, scale=p.scale, chunk=chunk, keep=True)
    precise = dtype == torch.float32
    rec_bytes = (kda.workspace_size(chunk, 1, 1, chunk, dtype) -
                 kda.workspace_size(0, 1, 1, chunk, dtype))
    raw = ws.buf.cpu().numpy()
    H = p.H
    cu = p.cu_seqlens.tolist()
    tol = 1e-5 if precise else 3e-3
    for (n, j, h), it in saved.items():
        slot = cu[n] // chunk + n + j
        rec = unpack_record(raw[(slot * H + h) * rec_bytes:(slot * H + h + 1) * rec_bytes],
                            chunk, precise)
        L = it["W"].shape[0]
        for name in ("W", "qg", "kg", "M", "U_base"):
            got, want = rec[name][:L], it[name]
            if name == "M":
                got = got[:, :L]
            scale = max(np.max(np.abs(want)), 1e-30)
            err = np.max(np.abs(got - want)) / scale
            assert err < tol, (n, j, h, name, err)
            if name in ("W", "kg", "U_base"):
                # padding rows must not reach U or the state; those of qg and M only
                # feed output rows that are never stored, and are left unspecified
                assert np.all(rec[name][L:] == 0.0), (n, j, h, name, "padding rows not zero")
        err = np.max(np.abs(rec["Gamma_C"] - it["Gamma_C"])) / max(np.max(it["Gamma_C"]), 1e-30)
        assert err < tol, (n, j, h, "Gamma_C", err)


# ---- the large workloads (last: slowest) -------------------------------------
# Every workload runs twice: with bf16 output (judged beyond its own storage
# rounding, raw error printed) and with fp32 output, where the literal metric
# max|o - o_ref| / rms(o_ref) <= 2e-2 applies unchanged.

def _both_outputs(kda, p, ref):
    o, ht = run_gpu(kda, p)
    check(p, o, ht, ref, p.name)
    del o, ht
    o32, ht32 = run_gpu(kda, p, o_dtype=torch.float32)
    check(p, o32, ht32, ref, p.name + " fp32-out")


def test_prefill_4k(kda):
    p = kda_inputs.prefill_4k()
    _both_outputs(kda, p, oracle_of(p))


@pytest.mark.parametrize("T,H", [(17, 16), (1024, 4)])
def test_contract_fixed_shapes(kda, golden_contract, T, H):
    """The fixed shapes the FlashInfer kda_backward contract admits besides the
    standard workloads (B=1, T=17, H=16 and B=1, T=1024, H=4), bf16 tokens,
    random initial states, chunk 64."""
    assert [1, T, H] in golden_contract["admitted_shapes"]["fixed"]
    p = kda_inputs.make_prefill([T], H, g_std=2.0, h0_std=0.1, chunk=64, seed=1100 + H,
                                name="contract T=%d H=%d bf16 C=64" % (T, H))
    _both_outputs(kda, p, oracle_of(p))


def test_contract_fixed_t17_h16_fp32(kda):
    p = kda_inputs.make_prefill([17], 16, token_dtype=torch.float32, h0_std=0.1, chunk=16,
                                seed=1116, name="contract T=17 H=16 fp32 C=16")
    o, ht = run_gpu(kda, p)
    check(p, o, ht, oracle_of(p), p.name)


def test_large(kda):
    p = kda_inputs.large()
    _both_outputs(kda, p, oracle_of(p))


def test_large_varlen(kda):
    p = kda_inputs.large_varlen()
    _both_outputs(kda, p, oracle_of(p))


def test_contract_packed_8x1024_h96(kda, golden_contract):
    """The contract's third packed shape: eight sequences of 1024 tokens at H=96
    (768 chains of the inter-chunk kernel)."""
    lengths = [1024] * 8
    assert {"lengths": lengths, "H": 96} in golden_contract["admitted_shapes"]["packed"]
    p = kda_inputs.packed_8x1024()
    _both_outputs(kda, p, oracle_of(p))


# ---- batch-size and length extremes ----------------------------------------------

def _many_lengths():
    rng = np.random.default_rng(5)
    return [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, 300, size=150)]


@pytest.mark.parametrize("dtype,chunk", [(torch.bfloat16, 64), (torch.float32, 32)])
def test_many_sequences(kda, dtype, chunk):
    """150 packed sequences of 0 to 299 tokens (more sequences than the inter
    kernel ranks by length), random initial states; fp32 output under the
    literal metric."""
    p = kda_inputs.make_prefill(_many_lengths(), 2, token_dtype=dtype, h0_std=0.1, chunk=chunk,
                                seed=1501 if dtype == torch.bfloat16 else 1502,
                                name="150 sequences %s C=%d" % (dtype, chunk))
    o, ht = run_gpu(kda, p, o_dtype=torch.float32)
    check(p, o, ht, oracle_of(p), p.name)


@pytest.mark.parametrize("T,dtype,gshift", [(65536, torch.bfloat16, 0.0), (65536, torch.bfloat16, -10.0),
                                            (32768, torch.float32, -10.0)])
def test_long_sequence(kda, T, dtype, gshift):
    """One sequence of 32768 or 65536 tokens (512 or 1024 chunk steps of the
    state), H=2, with the gates as drawn or shifted by -10 so that the state
    barely decays (lambda of about -2e-4 per token): the state's power-of-two
    scaling over long chains. fp32 output under the literal metric."""
    p = kda_inputs.make_prefill([T], 2, token_dtype=dtype, h0_std=0.1, chunk=64,
                                seed=1503 + int(-gshift) + (T >> 14),
                                name="T=%d %s gate shift %g" % (T, dtype, gshift))
    if gshift:
        p.g = p.g + gshift
    o, ht = run_gpu(kda, p, o_dtype=torch.float32)
    check(p, o, ht, oracle_of(p), p.name)
