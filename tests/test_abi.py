"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments with the documented status before any
HIP call (validation is host-only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def kda():
    import kimi_delta_attention_05_amd.kda as m
    return m


def test_library_exports_every_declared_symbol(kda):
    syms = declared_symbols()
    assert set(syms) == set(kda.EXPORTS)
    for s in syms:
        assert hasattr(kda.lib, s), s
    assert kda.version() == 106


def test_status_strings(kda):
    for code in range(5):
        assert kda.lib.kda_status_string(code)
    assert kda.lib.kda_status_string(99) == b"unknown status"


FAKE = 0x10000     # never dereferenced: every call below fails validation first


def chunk_call(kda, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.088,
                lb=-5.0, cu=FAKE, N=1, T=17, H=1, K=128, V=128, C=16, dt=kda.KDA_F32, h0=None,
                ht=None, o=FAKE, odt=kda.KDA_F32, ws=0x100000, wsb=1 << 40, stream=None)
    args.update(kw)
    return kda.lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                 args["A_log"], args["dt_bias"], args["scale"], args["lb"],
                                 args["cu"], args["N"], args["T"], args["H"], args["K"], args["V"],
                                 args["C"], args["dt"], args["h0"], args["ht"], args["o"],
                                 args["odt"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(K=129), 2), (dict(V=256), 2), (dict(K=0), 2), (dict(V=0), 2), (dict(C=48), 2),
    (dict(K=256, V=256), 2), (dict(K=256, V=256, C=64), 2), (dict(K=257, V=128, C=64, dt=1), 2),
    (dict(K=200, V=64, C=32, dt=1), 2), (dict(K=64, V=129, C=64), 2),
    (dict(C=128), 2), (dict(dt=7), 2),
    (dict(odt=3), 2),
    (dict(N=0), 1), (dict(T=-1), 1), (dict(H=0), 1), (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1), (dict(lb=0.0), 1), (dict(lb=-5.5), 1), (dict(lb=0.5), 1),
    (dict(cu=None), 1), (dict(A_log=None), 1), (dict(q=None), 1), (dict(o=None), 1),
    (dict(ws=None), 3), (dict(wsb=1024), 3), (dict(ws=0x100010), 3),
    # 16-byte alignment of tensor pointers, 4-byte for beta / A_log; head count cap
    (dict(q=FAKE + 8), 1), (dict(k=FAKE + 2), 1), (dict(v=FAKE + 4), 1), (dict(g=FAKE + 4), 1),
    (dict(dt_bias=FAKE + 4), 1), (dict(o=FAKE + 8), 1), (dict(h0=FAKE + 4), 1),
    (dict(ht=FAKE + 12), 1), (dict(beta=FAKE + 2), 1), (dict(A_log=FAKE + 1), 1),
    (dict(H=65537), 1),
])
def test_chunk_fwd_rejects(kda, kw, status):
    assert chunk_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def decode_call(kda, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.088,
             lb=-5.0, state=FAKE, o=FAKE, odt=kda.KDA_BF16, B=4, H=2, K=128, V=128,
             dt=kda.KDA_BF16, stream=None)
    a.update(kw)
    return kda.lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                                   a["dt_bias"], a["scale"], a["lb"], a["state"], a["o"],
                                   a["odt"], a["B"], a["H"], a["K"], a["V"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(K=257), 2), (dict(V=0), 2), (dict(dt=5), 2), (dict(B=0), 1), (dict(H=-1), 1),
    (dict(state=None), 1), (dict(q=None), 1), (dict(lb=-6.0), 1), (dict(scale=-1.0), 1),
    (dict(state=FAKE + 4), 1), (dict(q=FAKE + 8), 1), (dict(o=FAKE + 4), 1),
    (dict(beta=FAKE + 2), 1), (dict(H=70000), 1),
])
def test_decode_rejects(kda, kw, status):
    assert decode_call(kda, **kw) == status


def gated_call(kda, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.088,
             lb=-5.0, state=FAKE, o=FAKE, odt=kda.KDA_BF16, B=4, H=2, K=128, V=128,
             dt=kda.KDA_BF16, z=FAKE, w=FAKE, eps=1e-5, stream=None)
    a.update(kw)
    return kda.lib.kda_decode_step_gated(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                                         a["dt_bias"], a["scale"], a["lb"], a["state"], a["o"],
                                         a["odt"], a["B"], a["H"], a["K"], a["V"], a["dt"],
                                         a["z"], a["w"], a["eps"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), 1), (dict(w=None), 1), (dict(eps=0.0), 1), (dict(eps=-1e-5), 1),
    (dict(eps=float("inf")), 1), (dict(z=FAKE + 8), 1), (dict(w=FAKE + 4), 1),
    (dict(K=257), 2), (dict(B=0), 1), (dict(state=None), 1), (dict(o=FAKE + 4), 1),
])
def test_decode_gated_rejects(kda, kw, status):
    assert gated_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def slots_call(kda, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.088,
             lb=-5.0, pool=FAKE, S=8, idx=FAKE, o=FAKE, odt=kda.KDA_BF16, B=4, H=2, K=128, V=128,
             dt=kda.KDA_BF16, z=None, w=None, eps=1e-5, stream=None)
    a.update(kw)
    return kda.lib.kda_decode_step_slots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                                         a["dt_bias"], a["scale"], a["lb"], a["pool"], a["S"],
                                         a["idx"], a["o"], a["odt"], a["B"], a["H"], a["K"],
                                         a["V"], a["dt"], a["z"], a["w"], a["eps"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=0), 1), (dict(idx=None), 1), (dict(idx=FAKE + 2), 1), (dict(pool=None), 1),
    (dict(pool=FAKE + 4), 1), (dict(S=1 << 30, H=4), 1), (dict(z=FAKE), 1),
    (dict(z=FAKE, w=FAKE, eps=0.0), 1), (dict(K=257), 2), (dict(B=0), 1),
])
def test_decode_slots_rejects(kda, kw, status):
    assert slots_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def norm_gate_call(kda, **kw):
    a = dict(o=FAKE, z=FAKE, w=FAKE, eps=1e-5, rows=10, D=128, dt=kda.KDA_BF16, y=FAKE, stream=None)
    a.update(kw)
    return kda.lib.kda_output_norm_gate(a["o"], a["z"], a["w"], a["eps"], a["rows"], a["D"],
                                        a["dt"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), 1), (dict(D=257), 2), (dict(D=0), 2), (dict(dt=9), 2), (dict(eps=0.0), 1),
    (dict(eps=float("nan")), 1), (dict(o=None), 1), (dict(z=None), 1), (dict(w=None), 1),
    (dict(y=None), 1), (dict(o=FAKE + 2), 1), (dict(z=FAKE + 8), 1), (dict(w=FAKE + 4), 1),
    (dict(y=FAKE + 4), 1), (dict(rows=1 << 40), 1),
])
def test_output_norm_gate_rejects(kda, kw, status):
    assert norm_gate_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def test_output_norm_gate_zero_rows_enqueues_nothing(kda):
    # rows = 0 returns OK without touching memory or launching, NULL pointers included
    assert norm_gate_call(kda, rows=0) == 0
    assert norm_gate_call(kda, rows=0, o=None, z=None, w=None, y=None) == 0
    assert norm_gate_call(kda, rows=0, D=300) == 2


def short_conv_call(kda, **kw):
    a = dict(x=FAKE, xs=256, w=FAKE, W=4, cu=FAKE, N=2, T=100, C=256, dt=kda.KDA_BF16,
             si=None, so=None, y=1 << 30, stream=None)
    a.update(kw)
    return kda.lib.kda_short_conv(a["x"], a["xs"], a["w"], a["W"], a["cu"], a["N"], a["T"],
                                  a["C"], a["dt"], a["si"], a["so"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(T=-1), 1), (dict(W=0), 2), (dict(W=5), 2), (dict(C=0), 1),
    (dict(C=12), 1), (dict(xs=128), 1), (dict(xs=260), 1), (dict(dt=5), 2), (dict(cu=None), 1),
    (dict(w=None), 1), (dict(x=None), 1), (dict(y=None), 1), (dict(x=FAKE + 8), 1),
    (dict(y=FAKE * 4 + 2), 1), (dict(si=FAKE + 4), 1), (dict(w=FAKE + 2), 1), (dict(cu=FAKE + 4), 1),
    # y overlapping x (bf16 rows of 256 elements: x spans 99 * 512 + 512 bytes)
    (dict(y=FAKE), 1), (dict(y=FAKE + 99 * 512), 1),
    # y overlapping a state; the final state overlapping x or part of the initial state
    (dict(si=1 << 29, y=(1 << 29) + 512), 1), (dict(so=FAKE + 256 * 2 * 3), 1),
    (dict(si=1 << 29, so=(1 << 29) + 512), 1),
    (dict(C=1 << 40, xs=1 << 40), 1),
])
def test_short_conv_rejects(kda, kw, status):
    assert short_conv_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def short_conv_slots_call(kda, **kw):
    a = dict(x=FAKE, xs=256, w=FAKE, W=4, cu=FAKE, N=2, T=100, C=256, dt=kda.KDA_BF16,
             pool=1 << 29, S=4, idx=1 << 28, y=1 << 30, stream=None)
    a.update(kw)
    return kda.lib.kda_short_conv_slots(a["x"], a["xs"], a["w"], a["W"], a["cu"], a["N"], a["T"],
                                        a["C"], a["dt"], a["pool"], a["S"], a["idx"], a["y"],
                                        a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(W=5), 2), (dict(C=12), 1), (dict(S=0), 1), (dict(idx=None), 1),
    (dict(idx=(1 << 28) + 2), 1), (dict(pool=None), 1), (dict(pool=(1 << 29) + 8), 1),
    (dict(y=(1 << 29) + 64), 1), (dict(pool=FAKE + 512), 1), (dict(dt=3), 2),
])
def test_short_conv_slots_rejects(kda, kw, status):
    assert short_conv_slots_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def test_short_conv_nothing_to_do(kda):
    # no tokens and W = 1 (no state to pass on): OK with no launch, NULL x and y accepted
    assert short_conv_call(kda, T=0, W=1, x=None, y=None, so=FAKE) == 0


def backward_call(kda, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.088,
             lb=-5.0, cu=FAKE, N=1, T=17, H=1, K=128, V=128, dt=kda.KDA_BF16, h0=None, do=FAKE,
             dodt=kda.KDA_BF16, dht=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE,
             dA=FAKE, ddt=FAKE, dh0=None, ws=0x100000, wsb=1 << 40, stream=None)
    a.update(kw)
    return kda.lib.kda_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                                a["dt_bias"], a["scale"], a["lb"], a["cu"], a["N"], a["T"], a["H"],
                                a["K"], a["V"], a["dt"], a["h0"], a["do"], a["dodt"], a["dht"],
                                a["dq"], a["dk"], a["dv"], a["dg"], a["dbeta"], a["dA"], a["ddt"],
                                a["dh0"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), 1), (dict(T=-1), 1), (dict(H=0), 1), (dict(H=65536), 1), (dict(K=129), 2),
    (dict(dt=4), 2), (dict(dodt=4), 2), (dict(scale=0.0), 1), (dict(lb=1.0), 1),
    (dict(cu=None), 1), (dict(dA=None), 1), (dict(ddt=None), 1), (dict(q=None), 1),
    (dict(do=None), 1), (dict(dq=None), 1), (dict(dbeta=None), 1), (dict(ws=None), 3),
    (dict(wsb=1024), 3), (dict(ws=0x100040), 3), (dict(dq=FAKE + 8), 1), (dict(dh0=FAKE + 4), 1),
    (dict(dbeta=FAKE + 2), 1), (dict(N=1 << 20, H=1024), 1),
])
def test_backward_rejects(kda, kw, status):
    assert backward_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def test_backward_workspace_size(kda):
    # per (16-token chunk slot, head): a 64 KiB state checkpoint (whose rows
    # then hold the reverse pass's partial sums), the chunk's operand record
    # (7168 floats, then X and P: 2 x 320), R of the chunk (8 KiB), 129
    # parameter sums
    slots = 8192 // 16 + 1
    per = 65536 + (7168 + 640) * 4 + 8192 + 129 * 4
    a = kda.backward_workspace_size(8192, 1, 96)
    assert slots * 96 * per <= a < slots * 96 * per + 1024
    assert a % 256 == 0
    with pytest.raises(ValueError):
        kda.backward_workspace_size(16, 0, 1)


def test_grouped_entry_points_reject_bad_groups(kda):
    # H_qk must divide H (validation runs before any HIP call)
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE)
    for hqk in (0, 3, 5, 9, -1):
        st = kda.lib.kda_chunk_fwd_grouped(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.088, -5.0,
                                           FAKE, 1, 17, 8, 128, 128, 16, kda.KDA_F32, None, None,
                                           FAKE, kda.KDA_F32, 0x100000, 1 << 40, None, hqk)
        assert st == 1 and b"H_qk" in kda.lib.kda_last_error()
        st = kda.lib.kda_decode_step_grouped(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.088, -5.0,
                                             FAKE, 0, None, FAKE, kda.KDA_F32, 4, 8, hqk, 128, 128,
                                             kda.KDA_BF16, None, None, 1e-5, None)
        assert st == 1
        st = backward_call_grouped(kda, hqk)
        assert st == 1


def backward_call_grouped(kda, hqk):
    return kda.lib.kda_backward_grouped(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.088, -5.0, FAKE,
                                        1, 17, 8, hqk, 128, 128, kda.KDA_BF16, None, FAKE,
                                        kda.KDA_BF16, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        None, 0x100000, 1 << 40, None)


def recurrent_call(kda, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.125,
             lb=-5.0, cu=FAKE, N=2, T=17, H=4, Hqk=4, K=64, V=48, dt=kda.KDA_F32, h0=FAKE,
             ht=FAKE + (1 << 24), o=FAKE, odt=kda.KDA_F32, stream=None)
    a.update(kw)
    return kda.lib.kda_recurrent_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                                     a["dt_bias"], a["scale"], a["lb"], a["cu"], a["N"], a["T"],
                                     a["H"], a["Hqk"], a["K"], a["V"], a["dt"], a["h0"], a["ht"],
                                     a["o"], a["odt"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), 2), (dict(K=257), 2), (dict(V=0), 2), (dict(V=300), 2), (dict(dt=4), 2),
    (dict(odt=9), 2),
    (dict(N=0), 1), (dict(T=-1), 1), (dict(H=0), 1), (dict(H=65537), 1), (dict(Hqk=3), 1),
    (dict(Hqk=0), 1), (dict(scale=0.0), 1), (dict(scale=float("inf")), 1), (dict(lb=0.0), 1),
    (dict(lb=-7.0), 1), (dict(cu=None), 1), (dict(A_log=None), 1), (dict(dt_bias=None), 1),
    (dict(q=None), 1), (dict(o=None), 1), (dict(beta=None), 1),
    # element alignment (bf16 tokens 2 bytes, fp32 arrays 4, offsets 8)
    (dict(q=FAKE + 2), 1), (dict(dt=1, v=FAKE + 1), 1), (dict(g=FAKE + 2), 1),
    (dict(cu=FAKE + 4), 1), (dict(h0=FAKE + 2), 1), (dict(odt=1, o=FAKE + 1), 1),
    # final state overlapping the initial state without being it
    (dict(ht=FAKE + 64), 1),
])
def test_recurrent_fwd_rejects(kda, kw, status):
    assert recurrent_call(kda, **kw) == status
    assert kda.lib.kda_last_error()


def test_workspace_size_below_128(kda):
    # head sizes below 128 add zero-padded copies (q, k, v, g, dt_bias, states, o)
    # after the records; 0 and 257 are rejected, and 129 where the 256-wide kernels
    # do not run (chunk_size 32)
    import torch
    T, N, H, C = 1000, 3, 4, 64
    base = kda.workspace_size(T, N, H, C, torch.bfloat16)
    padded = kda.workspace_size(T, N, H, C, torch.bfloat16, K=64, V=48)
    assert padded >= base + T * H * 128 * (3 * 2 + 4 + 4) + N * H * 128 * 128 * 4 + H * 128 * 4
    assert padded == kda.workspace_size(T, N, H, C, torch.bfloat16, K=1, V=1)
    for K, V, Cx in ((129, 64, 32), (64, 0, C), (257, 64, C)):
        with pytest.raises(ValueError):
            kda.workspace_size(T, N, H, Cx, torch.bfloat16, K=K, V=V)


def test_backward_workspace_size_below_128(kda):
    # head sizes below 128 add the padded inputs, adjoints and gradients after the
    # backward's own layout; 0 and 129 are rejected
    T, N, H = 1000, 2, 3
    base = kda.backward_workspace_size(T, N, H)
    padded = kda.backward_workspace_size(T, N, H, K=64, V=32)
    assert padded >= base + T * H * 128 * 4 * 9 + 3 * N * H * 128 * 128 * 4
    for K, V in ((0, 64), (64, 129)):
        with pytest.raises(ValueError):
            kda.backward_workspace_size(T, N, H, K=K, V=V)


def test_workspace_size_arithmetic(kda):
    # one record per (slot, head); slots = floor(T / C) + N
    for T, N, H, C in [(8192, 1, 96, 64), (8192, 6, 96, 64), (17, 1, 1, 16), (115, 3, 4, 32), (0, 2, 3, 64)]:
        a = kda.workspace_size(T, N, H, C, in_dtype=__import__("torch").bfloat16)
        b = kda.workspace_size(T + C, N, H, C, in_dtype=__import__("torch").bfloat16)
        per = (b - a) // H
        assert (b - a) % H == 0 and per > 0
        assert a == (T // C + N) * H * per + 256
    import torch
    assert kda.workspace_size(64, 1, 1, 64, torch.float32) > kda.workspace_size(64, 1, 1, 64, torch.bfloat16)
    with pytest.raises(ValueError):
        kda.workspace_size(64, 1, 1, 48)
    with pytest.raises(ValueError):
        kda.workspace_size(64, 0, 1, 64)


def test_check_cu_seqlens_rejects_null(kda):
    assert kda.lib.kda_check_cu_seqlens(None, 1, 10, None) == 1


def test_binding_requires_gpu_tensors(kda):
    import torch
    import kda_inputs
    p = kda_inputs.small()
    with pytest.raises(RuntimeError):
        kda.chunk_fwd(p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias, p.cu_seqlens,
                      scale=p.scale, chunk_size=16)


def test_no_cpu_fallback_in_product():
    """The product package never imports the oracle and has no CPU compute path."""
    pkg = os.path.join(ROOT, "kimi_delta_attention_05_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert "oracle" not in src, name
            assert "kda_inputs" not in src, name


def noalloc_call(kda, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, scale=0.088,
                lb=-5.0, cu=FAKE, N=1, T=17, H=1, K=128, V=128, C=16, dt=kda.KDA_F32, h0=None,
                ht=None, o=FAKE, odt=kda.KDA_F32, stream=None)
    args.update(kw)
    return kda.lib.kda_chunk_fwd_noalloc(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                         args["A_log"], args["dt_bias"], args["scale"], args["lb"],
                                         args["cu"], args["N"], args["T"], args["H"], args["K"],
                                         args["V"], args["C"], args["dt"], args["h0"], args["ht"],
                                         args["o"], args["odt"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    # beyond the fixed scratch: the T=8192, H=96 prefill needs ~0.92 GB
    (dict(T=8192, H=96, C=64, dt=1, odt=1), 3),
    (dict(T=1 << 20, H=4, C=64), 3),
    (dict(K=129), 2), (dict(C=48), 2), (dict(N=0), 1), (dict(q=None), 1), (dict(lb=0.0), 1),
    (dict(q=FAKE + 8), 1),
])
def test_chunk_fwd_noalloc_rejects(kda, kw, status):
    """Checked on the host before any HIP call, like every entry point."""
    assert noalloc_call(kda, **kw) == status
    msg = kda.lib.kda_last_error().decode()
    assert msg
    if status == 3:
        assert "fixed 134217728 bytes" in msg, msg


def test_noalloc_scratch_limit_covers_stated_shapes(kda):
    """The header's examples: T = 8192 at H = 12 fits the fixed scratch, H = 96 does not."""
    assert kda.workspace_size(8192, 1, 12, 64) <= kda.NOALLOC_SCRATCH_BYTES
    assert kda.workspace_size(8192, 1, 96, 64) > kda.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), 1), (dict(dst=None), 1), (dict(n=17), 1), (dict(src=FAKE + 4), 1),
    (dict(dst=FAKE + 8 + (1 << 20)), 1), (dict(dst=FAKE + 512), 1),   # misaligned; overlapping
])
def test_stream_copy_rejects(kda, kw, status):
    a = dict(src=FAKE, dst=FAKE + (1 << 20), n=1024)
    a.update(kw)
    assert kda.lib.kda_stream_copy(a["src"], a["dst"], a["n"], None) == status
    assert kda.lib.kda_last_error()


def test_stream_copy_zero_bytes_enqueues_nothing(kda):
    assert kda.lib.kda_stream_copy(None, None, 0, None) == 0


def test_chunk_fwd_gated_rejects_before_any_hip_call(kda):
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.088, -5.0, FAKE, 1, 17, 1, 128, 128, 16,
            kda.KDA_F32, None, None, FAKE, kda.KDA_F32, 0x100000, 1 << 40, None]
    f = kda.lib.kda_chunk_fwd_gated
    assert f(*base, None, FAKE, 1e-5) == 1                  # no z (T > 0)
    assert f(*base, FAKE + (1 << 20), None, 1e-5) == 1      # no norm weight
    assert f(*base, FAKE + (1 << 20), FAKE, 0.0) == 1       # eps must be > 0
    assert f(*base, FAKE + (1 << 20) + 4, FAKE, 1e-5) == 1  # z misaligned
    assert f(*base, FAKE, FAKE, 1e-5) == 1                  # z overlaps o


def test_gated_workspace_size(kda):
    f = kda.lib.kda_chunk_fwd_gated_workspace_size
    base = kda.lib.kda_chunk_fwd_workspace_size(8192, 1, 96, 128, 128, 64, kda.KDA_BF16)
    up = (base + 255) // 256 * 256
    # fused epilogue: the halves' row-sum exchange, one 8-byte word per row of each
    # chunk slot, head and half; bf16 results of the unfused pass staged in fp16
    # with a 4-byte scale per 16 features, whichever is larger
    xchg = (8192 // 64 + 1) * 96 * 128 * 8
    assert f(8192, 1, 96, 128, 128, 64, kda.KDA_BF16, kda.KDA_F32) == up + xchg
    assert f(8192, 1, 96, 128, 128, 64, kda.KDA_BF16, kda.KDA_BF16) == \
        up + 8192 * 96 * (128 * 2 + 8 * 4)
    b1 = kda.lib.kda_chunk_fwd_workspace_size(64, 64, 2, 128, 128, 64, kda.KDA_BF16)
    assert f(64, 64, 2, 128, 128, 64, kda.KDA_BF16, kda.KDA_BF16) == \
        (b1 + 255) // 256 * 256 + (64 // 64 + 64) * 2 * 128 * 8
    b32 = kda.lib.kda_chunk_fwd_workspace_size(8192, 1, 96, 128, 128, 32, kda.KDA_BF16)
    assert f(8192, 1, 96, 128, 128, 32, kda.KDA_BF16, kda.KDA_F32) == b32
    assert f(8192, 1, 96, 128, 128, 32, kda.KDA_BF16, kda.KDA_BF16) == \
        (b32 + 255) // 256 * 256 + 8192 * 96 * 128 * 4
    assert f(100, 2, 3, 48, 80, 32, kda.KDA_F32, kda.KDA_BF16) > \
        kda.lib.kda_chunk_fwd_workspace_size(100, 2, 3, 48, 80, 32, kda.KDA_F32)
    assert f(8192, 1, 96, 128, 128, 64, kda.KDA_BF16, 7) == 0
    assert f(8192, 1, 96, 257, 128, 64, kda.KDA_BF16, kda.KDA_BF16) == 0
    assert f(8192, 1, 96, 129, 128, 32, kda.KDA_BF16, kda.KDA_BF16) == 0


def test_workspace_size_native_64(kda):
    """K = V = 64 with 64-row chunks of bf16 inputs runs on kernels sized for 64:
    records only (no padded copies), each smaller than a 128-wide record; other
    dtypes and chunk sizes at 64 keep the padded layout."""
    import torch
    T, N, H = 1000, 3, 4
    slots = T // 64 + N
    n64 = kda.workspace_size(T, N, H, 64, torch.bfloat16, K=64, V=64)
    n128 = kda.workspace_size(T, N, H, 64, torch.bfloat16)
    assert (n64 - 256) % (slots * H) == 0
    rec64 = (n64 - 256) // (slots * H)
    assert rec64 < (n128 - 256) // (slots * H)
    # W, qg, kg (64 x 64 fp16 each), M (8 fragments), decay (64 fp32), scale, Ub (64 x 64)
    assert rec64 == 3 * 64 * 64 * 2 + 8 * 1024 + 64 * 4 + 16 + 64 * 64 * 2
    assert kda.workspace_size(T, N, H, 32, torch.bfloat16, K=64, V=64) > n128
    assert kda.workspace_size(T, N, H, 64, torch.float32, K=64, V=64) > n128


def test_workspace_size_native_256(kda):
    """K = V = 256 with 64-row chunks of bf16 inputs runs on kernels sized for 256:
    one record per chunk slot and head, no padded copies; other dtypes and chunk
    sizes are rejected (the token-by-token forward takes them)."""
    import torch
    T, N, H = 1000, 3, 4
    slots = T // 64 + N
    n = kda.workspace_size(T, N, H, 64, torch.bfloat16, K=256, V=256)
    assert (n - 256) % (slots * H) == 0
    # W, qg, kg (64 x 256 fp16 each), M (8 fragments), decay (256 fp32), scale, Ub (64 x 256)
    assert (n - 256) // (slots * H) == 3 * 64 * 256 * 2 + 8 * 1024 + 256 * 4 + 16 + 64 * 256 * 2
    for C, dt in ((32, torch.bfloat16), (64, torch.float32)):
        with pytest.raises(ValueError):
            kda.workspace_size(T, N, H, C, dt, K=256, V=256)


@pytest.mark.parametrize("K,V", [(192, 192), (129, 256), (256, 40), (1, 200)])
def test_workspace_size_padded_256(kda, K, V):
    """K or V above 128 (up to 256; 64-row chunks of bf16 inputs): the 256-wide
    kernels' records, then the copies padded to 256 (q, k, v in bf16, g fp32,
    dt_bias, states and the fp32 output staging), each 256-byte aligned."""
    import torch
    T, N, H = 1000, 3, 4
    up = lambda x: (x + 255) // 256 * 256
    rec = kda.workspace_size(T, N, H, 64, torch.bfloat16, K=256, V=256)
    tok = T * H * 256
    want = up(rec)
    for nbytes in (tok * 2, tok * 2, tok * 2, tok * 4, H * 256 * 4, N * H * 256 * 256 * 4, tok * 4):
        want = up(want + nbytes)
    assert kda.workspace_size(T, N, H, 64, torch.bfloat16, K=K, V=V) == want
    for C, dt in ((32, torch.bfloat16), (64, torch.float32)):
        with pytest.raises(ValueError):
            kda.workspace_size(T, N, H, C, dt, K=K, V=V)
