#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X.

One step = the whole path once: a chunkwise prefill of T=8192 tokens x H=96
heads (bf16 q/k/v, chunk 64, random fp32 initial states; intra-chunk kernel
then inter-chunk kernel) followed by one batched decode step of 256 requests x
32 heads (fp32 state updated in place). Decode inputs cycle through 64
pre-generated token sets (64 consecutive steps). Inputs are seeded synthetic
tensors already resident in HBM when timing starts.

Prints one JSON line: value = tokens processed per second over the timed steps
(8192 prefill + 256 decode tokens per step), per-kernel HIP-event timings, the
roofline of the dominant kernel and of each kernel, and the fp64 CPU oracle
timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
D = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kimi_delta_attention_05_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "intra_kernel": ("kda_prefill.hip", "kda_common.h", "kda_internal.h"),
    "inter_kernel": ("kda_prefill.hip", "kda_common.h", "kda_internal.h"),
    "inter_kernel_gated": ("kda_prefill.hip", "kda_common.h", "kda_internal.h"),
    "decode_step_kernel": ("kda_decode.hip", "kda_common.h", "kda_internal.h"),
    "short_conv_kernel": ("kda_shortconv.hip", "kda_common.h", "kda_internal.h"),
    "norm_gate_kernel": ("kda_epilogue.hip", "kda_common.h", "kda_internal.h"),
    "bwd_prep_kernel": ("kda_backward.hip", "kda_common.h", "kda_internal.h"),
    "bwd_ckpt_kernel": ("kda_backward.hip", "kda_common.h", "kda_internal.h"),
    "bwd_chunk_kernel": ("kda_backward.hip", "kda_common.h", "kda_internal.h"),
    "bwd_chunk_final_kernel": ("kda_backward.hip", "kda_common.h", "kda_internal.h"),
    "bwd_param_kernel": ("kda_backward.hip", "kda_common.h", "kda_internal.h"),
}

# fp32 MFMA arithmetic of the chunked backward per 16-token chunk and head
# (K = V = 128), as its kernels execute it: the operand record (KE KI^T,
# QG KI^T), the checkpoint pass (KE S^T, T R, KG^T U), the reverse pass (KG dS^T,
# QG^T dO, KE^T dR, the partials dO S, U dS, dR S, and six 16x16x128 products),
# the finalize (dP KI, dM KI, dP^T KE, dM^T QG)
BWD_FLOPS_PER_CHUNK_HEAD = (2 * 16 * 16 * D * 2          # prep
                            + 2 * 16 * D * D * 2 + 16 * 16 * D * 2   # checkpoint
                            + 6 * 16 * D * D * 2 + 6 * 16 * 16 * D * 2   # reverse
                            + 4 * 16 * 16 * D * 2)       # finalize


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha") != source_sha(*KERNEL_SOURCES[kernel]):
        return None
    return t.get("bytes_per_launch")


def prefill_flops_per_token_head(C):
    # W S^T, qg S^T, state update (2 d^2 each); A; M; T v; T (k e^G); M U; inverse
    return 6 * D * D + (C - 1) * D + 4 * (C + 1) * D + C * C / 3.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps first bring the GPU to its steady clocks: after 3 the timed
    # steps still run about 5% slower than after 50 (about 45 ms)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (--gpus 1); multi-GPU runs are "
              "not part of it", file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_inputs
    import kimi_delta_attention_05_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs ...")
    p = kda_inputs.large()
    dd = kda_inputs.decode(64)
    T, H, N, C = p.T, p.H, p.N, p.chunk
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    g, beta_raw = p.g.to(dev), p.beta_raw.to(dev)
    A_log, dt_bias, cu = p.A_log.to(dev), p.dt_bias.to(dev), p.cu_seqlens.to(dev)
    h0 = p.h0.to(dev)
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    ws = kda.Workspace(dev)
    B, HD = 256, 32
    dstate = dd.state.to(dev)
    dA, ddt = dd.A_log.to(dev), dd.dt_bias.to(dev)
    dsteps = [{kk: vv.to(dev) for kk, vv in st.items()} for st in dd.steps]
    dout = torch.empty((B, HD, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def prefill(stage):
        kda.chunk_fwd(q, k, v, g, beta_raw, A_log, dt_bias, cu, scale=p.scale, chunk_size=C,
                      initial_state=h0, out=o, final_state=ht, workspace=ws, stage=stage)

    def decode(i):
        st = dsteps[i % len(dsteps)]
        kda.decode_step(st["q"], st["k"], st["v"], st["g"], st["beta_raw"], dA, ddt, dstate,
                        scale=dd.scale, out=dout)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        prefill("intra")
        if ev is not None:
            ev[1].record()
        prefill("inter")
        if ev is not None:
            ev[2].record()
        decode(i)
        if ev is not None:
            ev[3].record()

    log("warmup %d steps ..." % args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed %d steps in %.3f s" % (K, wall))

    intra_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    inter_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / K
    decode_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / K
    prefill_ms = intra_ms + inter_ms

    th = T * H
    kernels = {
        # algorithmic bytes each kernel must move: inputs it reads, outputs it writes
        "intra_kernel": dict(ms=intra_ms, bytes=th * (3 * 2 * D + 4 * D + 4)),
        "inter_kernel": dict(ms=inter_ms, bytes=th * 2 * D + 2 * N * H * D * D * 4),
        "decode_step_kernel": dict(ms=decode_ms, bytes=B * HD * (2 * D * D * 4 + 3 * 2 * D + 4 * D + 4
                                                                 + 2 * D)),
    }
    for name, kd in kernels.items():
        kd["achieved_GBs"] = kd["bytes"] / (kd["ms"] * 1e-3) / 1e9
        kd["frac"] = kd["achieved_GBs"] / HBM_PEAK_GBS
        kd["traffic"] = measured_traffic(name)
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    kd = kernels[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(kd["achieved_GBs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kd["frac"], 4),
                "traffic": kd["traffic"]}

    prefill_bytes = th * (4 * 2 * D + 4 * D + 4) + 2 * N * H * D * D * 4
    prefill_flops = th * prefill_flops_per_token_head(C)
    tokens_per_step = T + B
    value = tokens_per_step * K / wall

    line = {
        "metric": "KDA fwd tokens/s (T=8192,H=96 prefill; decode bs=256) + % MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; fp16 MFMA operands, fp32 accumulate/state",
        "data": "synthetic (seeded N(0,1) tokens, N(0,2^2) gates, U(0,ln16) A_log, U(-1,1) dt_bias)",
        "config": {"workload": "prefill T=8192 H=96 K=V=128 chunk 64 bf16 + decode B=256 H=32 "
                               "T=1, one of each per step",
                   "prefill_tokens_per_step": T, "decode_tokens_per_step": B,
                   "heads_prefill": H, "heads_decode": HD, "chunk": C},
        "prefill": {"ms": round(prefill_ms, 4), "tokens_per_s": round(T / (prefill_ms * 1e-3), 1),
                    "hbm_frac_path": round(prefill_bytes / (prefill_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "mfma_frac_path": round(prefill_flops / (prefill_ms * 1e-3) / 1e12
                                            / MFMA_BF16_PEAK_TFLOPS, 4)},
        "decode": {"us": round(decode_ms * 1e3, 2), "tokens_per_s": round(B / (decode_ms * 1e-3), 1),
                   "hbm_frac": round(kernels["decode_step_kernel"]["frac"], 4)},
        "kernels": {n: {"us": round(x["ms"] * 1e3, 2), "alg_bytes": int(x["bytes"]),
                        "achieved_GBs": round(x["achieved_GBs"], 1), "frac": round(x["frac"], 4),
                        "traffic": x["traffic"]} for n, x in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": None,
    }

    line["decode_64_consecutive"] = decode_consecutive_timing(kda, dd, dsteps, dA, ddt, dstate, dout)
    line["epilogue"] = epilogue_timing(kda, o, dsteps, dA, ddt, dstate, dd.scale, dout)
    line["epilogue"].update(gated_prefill_timing(kda, p, (q, k, v, g, beta_raw, A_log, dt_bias, cu),
                                                 h0, o, ht, ws))
    line["front_end"] = front_end_timing(kda, (q, k, v), cu)
    line["backward"] = backward_timing(kda, p, (q, k, v, g, beta_raw, A_log, dt_bias, cu, h0))
    line["other_prefill_configs"] = other_prefill_timing(kda, dev)
    line["any_head_size"] = general_timing(kda, dev)
    line["achievable"] = achievable_hbm(kda, kernels)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p, dd)
    print(json.dumps(line), flush=True)


def decode_consecutive_timing(kda, dd, dsteps, dA, ddt, dstate, dout, reps=5):
    """The decode workload as stated: 64 consecutive T=1 steps of the B=256, H=32
    batch, back to back on one stream (state carried in place), timed with
    events around the 64 launches; the median of `reps` such sequences, the state
    restored from a pristine copy outside the timed region."""
    import torch
    pristine = dstate.clone()
    B, HD, Dv = dout.shape
    n = len(dsteps)

    def run():
        for st in dsteps:
            kda.decode_step(st["q"], st["k"], st["v"], st["g"], st["beta_raw"], dA, ddt, dstate,
                            scale=dd.scale, out=dout)

    dstate.copy_(pristine)
    run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        dstate.copy_(pristine)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2] / n
    nbytes = B * HD * (2 * Dv * Dv * 4 + 3 * 2 * Dv + 4 * Dv + 4 + 2 * Dv)
    gb = nbytes / (ms * 1e-3) / 1e9
    return {"steps": n, "us_per_step": round(ms * 1e3, 2),
            "tokens_per_s": round(B / (ms * 1e-3), 1), "alg_bytes_per_step": nbytes,
            "achieved_GBs": round(gb, 1), "hbm_frac": round(gb / HBM_PEAK_GBS, 4)}


def epilogue_timing(kda, o, dsteps, dA, ddt, dstate, dscale, dout, reps=20):
    """The output epilogue (per-head RMS norm + sigmoid gate), measured beside the
    step and not part of it: the standalone kernel over the prefill output
    (T*H rows of 128 bf16, y written in place of a copy of o) and the decode step
    with the epilogue fused, against the plain decode step."""
    import torch
    import kda_inputs
    T, H, Dv = o.shape
    z, w = kda_inputs.make_epilogue((T, H, Dv), seed=2001)
    z, w = z.to(o.device), w.to(o.device)
    y = torch.empty_like(o)
    B, HD = dout.shape[0], dout.shape[1]
    zd, wd = kda_inputs.make_epilogue((B, HD, Dv), seed=2002)
    zd, wd = zd.to(o.device), wd.to(o.device)

    def timed(fn):
        for _ in range(3):
            fn(0)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record()
            fn(i)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        return sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) / reps

    ms_ng = timed(lambda i: kda.output_norm_gate(o, z, w, out=y))
    rows = T * H
    ng_bytes = rows * 3 * Dv * 2 + Dv * 4                 # o, z read, y written (bf16)

    def dec(i, gated):
        st = dsteps[i % len(dsteps)]
        kw = dict(gate=zd, norm_weight=wd) if gated else {}
        kda.decode_step(st["q"], st["k"], st["v"], st["g"], st["beta_raw"], dA, ddt, dstate,
                        scale=dscale, out=dout, **kw)

    ms_plain = timed(lambda i: dec(i, False))
    ms_gated = timed(lambda i: dec(i, True))
    gb = ng_bytes / (ms_ng * 1e-3) / 1e9
    return {"norm_gate_kernel": {"rows": rows, "us": round(ms_ng * 1e3, 2), "alg_bytes": ng_bytes,
                                 "achieved_GBs": round(gb, 1), "frac": round(gb / HBM_PEAK_GBS, 4),
                                 "traffic": measured_traffic("norm_gate_kernel")},
            "decode_step_gated_us": round(ms_gated * 1e3, 2),
            "decode_step_plain_us": round(ms_plain * 1e3, 2)}


def gated_prefill_timing(kda, p, args, h0, o, ht, ws, reps=20):
    """The prefill with the output epilogue (per-head RMS norm + sigmoid gate,
    kda_chunk_fwd_gated: at this size applied by the inter-chunk kernel itself),
    beside the plain prefill and the plain prefill followed by a separate
    epilogue call (which reads o back from the memory-side cache): the median
    of `reps` calls each."""
    import torch
    import kda_inputs
    T, H, Dv = o.shape
    z, w = kda_inputs.make_epilogue((T, H, Dv), seed=2003)
    z, w = z.to(o.device), w.to(o.device)
    y = torch.empty_like(o)

    def plain():
        kda.chunk_fwd(*args, scale=p.scale, chunk_size=p.chunk, initial_state=h0, out=o,
                      final_state=ht, workspace=ws)

    def gated():
        kda.chunk_fwd(*args, scale=p.scale, chunk_size=p.chunk, initial_state=h0, out=y,
                      final_state=ht, workspace=ws, gate=z, norm_weight=w)

    def separate():
        plain()
        kda.output_norm_gate(o, z, w, out=y)

    # the three calls alternate, so that clock drift over the run affects each alike
    fns = (plain, gated, separate)
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    ts = [[], [], []]
    for _ in range(reps):
        for i, fn in enumerate(fns):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts[i].append(e0.elapsed_time(e1))
    mp, mg, ms = (sorted(t)[len(t) // 2] for t in ts)
    return {"prefill_plain_ms": round(mp, 4), "prefill_gated_ms": round(mg, 4),
            "prefill_then_epilogue_call_ms": round(ms, 4),
            "gated_over_plain": round(mg / mp, 4),
            "inter_kernel_gated_traffic": measured_traffic("inter_kernel_gated")}


def front_end_timing(kda, qkv, cu, W=4, reps=20):
    """The q/k/v front end (causal depthwise short conv of W taps + SiLU),
    measured beside the step and not part of it: one launch each for q, k and v
    of the prefill workload (T*H*128 bf16 channels in and out, conv states
    carried in and out), as a model runs it before the recurrence."""
    import torch
    import kda_inputs
    T, H, Dk = qkv[0].shape
    N = cu.numel() - 1
    ws, sts, outs, fins = [], [], [], []
    for i in range(3):
        _, w, _, st = kda_inputs.make_short_conv([0] * N, H, W, seed=2100 + i)
        ws.append(w.to(qkv[0].device))
        sts.append(st.to(qkv[0].device))
        outs.append(torch.empty_like(qkv[i]))
        fins.append(torch.empty_like(sts[-1]))

    def run(i):
        kda.short_conv(qkv[i], ws[i], cu, initial_state=sts[i], final_state=fins[i], out=outs[i])

    for _ in range(3):
        for i in range(3):
            run(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * reps + 1)]
    ev[0].record()
    for r in range(reps):
        for i in range(3):
            run(i)
            ev[3 * r + i + 1].record()
    torch.cuda.synchronize()
    ms = sum(ev[j].elapsed_time(ev[j + 1]) for j in range(3 * reps)) / (3 * reps)
    C = H * Dk
    nbytes = 2 * T * C * 2 + C * W * 4 + 2 * N * (W - 1) * C * 2    # x in, y out, weights, states
    gb = nbytes / (ms * 1e-3) / 1e9
    return {"short_conv_kernel": {"tokens": T, "channels": C, "W": W, "launches_per_layer": 3,
                                  "us": round(ms * 1e3, 2), "alg_bytes": nbytes,
                                  "achieved_GBs": round(gb, 1), "frac": round(gb / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic("short_conv_kernel")}}


FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA


def backward_timing(kda, p, dev_inputs, reps=3):
    """The training backward of the recurrence (kda_backward) on the prefill
    workload, measured beside the step and not part of it: output adjoint bf16
    [T, H, 128], final-state adjoint fp32, every gradient fp32."""
    import torch
    q, k, v, g, beta_raw, A_log, dt_bias, cu, h0 = dev_inputs
    T, H, Dk = q.shape
    N = cu.numel() - 1
    gen = torch.Generator().manual_seed(2200)
    d_o = torch.randn(T, H, Dk, generator=gen).to(torch.bfloat16).to(q.device)
    dht = (torch.randn(N, H, Dk, Dk, generator=gen) * 0.1).to(q.device)
    ws = kda.Workspace(q.device)

    def run():
        return kda.backward(q, k, v, g, beta_raw, A_log, dt_bias, cu, d_o, scale=p.scale,
                            initial_state=h0, d_final_state=dht, workspace=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    cu_h = cu.cpu().tolist()
    chunks = sum((cu_h[i + 1] - cu_h[i] + 15) // 16 for i in range(N))
    flops = chunks * H * BWD_FLOPS_PER_CHUNK_HEAD
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "workspace_bytes": kda.backward_workspace_size(T, N, H),
            "traffic": {kn: measured_traffic(kn) for kn in
                        ("bwd_prep_kernel", "bwd_ckpt_kernel", "bwd_chunk_kernel",
                         "bwd_chunk_final_kernel")},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4),
                         "alg_flops": flops, "dtype": "f32"}}


def other_prefill_timing(kda, dev, reps=10):
    """The prefill on the three other large workloads, beside the step and not
    part of it: T=4096, H=32 (its ~0.2 GB of inputs fit in the 256 MB MALL, so it
    is timed both back to back and with a 512 MB buffer written between runs),
    the packed six-sequence mix at H=96 (lengths 1300, 547, 2048, 963, 271,
    3063) and eight packed sequences of 1024 tokens at H=96. Each with its path HBM and MFMA fractions and its roofline fraction,
    max(flops / MFMA peak, bytes / HBM peak) / time."""
    import torch
    import kda_inputs
    out = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for name, p, cold in (("prefill T=4096 H=32", kda_inputs.prefill_4k(), True),
                          ("prefill varlen six sequences H=96", kda_inputs.large_varlen(), False),
                          ("prefill packed 8x1024 H=96", kda_inputs.packed_8x1024(), False)):
        args = [x.to(dev) for x in (p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                    p.cu_seqlens)]
        h0 = None if p.h0 is None else p.h0.to(dev)
        o = torch.empty((p.T, p.H, D), dtype=torch.bfloat16, device=dev)
        ht = torch.empty((p.N, p.H, D, D), dtype=torch.float32, device=dev)
        ws = kda.Workspace(dev)

        def run():
            kda.chunk_fwd(*args, scale=p.scale, chunk_size=p.chunk, initial_state=h0, out=o,
                          final_state=ht, workspace=ws)

        def timed(between=None):
            ts = []
            for _ in range(reps):
                if between is not None:
                    between()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return sorted(ts)[len(ts) // 2]

        run()
        torch.cuda.synchronize()
        th = p.T * p.H
        nbytes = th * (4 * 2 * D + 4 * D + 4) + (2 if h0 is not None else 1) * p.N * p.H * D * D * 4
        flops = th * prefill_flops_per_token_head(p.chunk)

        def stats(ms):
            t = ms * 1e-3
            return {"ms": round(ms, 4), "tokens_per_s": round(p.T / t, 1),
                    "hbm_frac_path": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                    "mfma_frac_path": round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "roofline_frac": round(max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                                               nbytes / (HBM_PEAK_GBS * 1e9)) / t, 4)}

        r = {"tokens": p.T, "heads": p.H, "sequences": p.N, "alg_bytes": nbytes, "alg_flops": flops}
        r["warm"] = stats(timed())
        if cold:
            r["mall_flushed"] = stats(timed(lambda: flush.fill_(1)))
        out[name] = r
    del flush
    return out


def general_timing(kda, dev, T=8192, H=96, reps=3):
    """The forward for head sizes other than 128 (kda_recurrent_fwd, token by
    token in fp32), measured beside the step and not part of it: the prefill
    workload's tokens and heads (one sequence, bf16 tokens, fp32 initial states)
    at K = V = 64, 192 and 256, and at K = V = 128 for comparison with the
    chunkwise path. Arithmetic: 7 flops per state element and token (decay, the
    two dot products, the update) against the fp32 vector peak. At K = V = 64,
    192 and 256 the chunkwise prefill is timed too (kernels sized for 64 and 256;
    192 on the 256-wide kernels over copies padded with zeros)."""
    import torch
    import kda_inputs
    out = {}
    for Kd in (64, 128, 192, 256):
        p = kda_inputs.make_prefill([T], H, token_dtype=torch.bfloat16, g_std=2.0, h0_std=0.1,
                                    seed=2300 + Kd, K=Kd, V=Kd)
        args = [x.to(dev) for x in (p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias,
                                    p.cu_seqlens)]
        h0 = p.h0.to(dev)
        o = torch.empty((T, H, Kd), dtype=torch.bfloat16, device=dev)
        ht = torch.empty_like(h0)

        def run():
            kda.recurrent_fwd(*args, scale=p.scale, initial_state=h0, final_state=ht, out=o)

        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = T * H * 7 * Kd * Kd
        tf = flops / (ms * 1e-3) / 1e12
        out["K=V=%d" % Kd] = {"ms": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
                              "roofline": {"bound": "alu", "achieved": round(tf, 2),
                                           "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                                           "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4)}}
        if Kd != D:
            # the same problem on the chunkwise prefill
            ws = kda.Workspace(dev)

            def run_c():
                kda.chunk_fwd(*args, scale=p.scale, chunk_size=64, initial_state=h0,
                              final_state=ht, out=o, workspace=ws)

            run_c()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                run_c()
            e1.record()
            torch.cuda.synchronize()
            mc = e0.elapsed_time(e1) / reps
            out["K=V=%d" % Kd]["chunked"] = {"ms": round(mc, 3),
                                             "tokens_per_s": round(T / (mc * 1e-3), 1)}
    return out


def achievable_hbm(kda, kernels, nbytes=1 << 30, reps=5):
    """Measured streaming rates beside the published 8 TB/s: this library's own
    streaming copy kernel (kda_stream_copy: 16-byte non-temporal loads and
    stores) and the runtime's device-to-device copy, each the best of a few
    1 GiB copies (bytes read + written per second), with each hot-path
    kernel's algorithmic rate as a fraction of the own copy's. The fastest of
    the hot-path kernels in the run is named too."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return min(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))

    ms_rt = best(lambda: dst.copy_(src))
    ms_own = best(lambda: kda.stream_copy(src, dst))
    gbs_rt = 2 * nbytes / (ms_rt * 1e-3) / 1e9
    gbs = 2 * nbytes / (ms_own * 1e-3) / 1e9
    del src, dst
    fastest = max(kernels, key=lambda n: kernels[n]["achieved_GBs"])
    return {"own_copy_kernel": "stream_copy_kernel", "own_copy_GBs": round(gbs, 1),
            "own_copy_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "runtime_copy_GBs": round(gbs_rt, 1), "copy_bytes": 2 * nbytes,
            "kernel_frac_of_own_copy": {n: round(x["achieved_GBs"] / gbs, 4)
                                        for n, x in kernels.items()},
            "fastest_hot_path_kernel": {"kernel": fastest,
                                        "GBs": round(kernels[fastest]["achieved_GBs"], 1)}}


def copy_calibration(nbytes=1 << 30, reps=3):
    """The library's streaming copy (stream_copy_kernel) over a buffer of known
    size: its FETCH_SIZE / WRITE_SIZE counter readings give the factor that
    converts those counters to bytes on this GPU."""
    import torch
    import kimi_delta_attention_05_amd as kda
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        kda.stream_copy(src, dst)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = min(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    print(json.dumps({"kernel": "stream_copy_kernel", "copy_bytes_read": nbytes,
                      "copy_bytes_written": nbytes, "reps": reps, "best_ms": round(ms, 4),
                      "GBs_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, dd, heads_1t=8):
    """The fp64 oracle as it stands, on the host cores: the same prefill
    (T=8192, H=96) once and two decode steps of the same batch, on all the
    threads OpenMP gives it; and on one thread, over the first `heads_1t` of the
    96 heads of the prefill (a bounded sample, scaled to the whole prefill: the
    heads are independent chains of equal length)."""
    import numpy as np
    import torch
    import oracle
    f32 = lambda x: np.ascontiguousarray(x.float().numpy())
    args = [f32(x) for x in (p.q, p.k, p.v, p.g, p.beta_raw, p.A_log, p.dt_bias)]
    h0 = p.h0.double().numpy()
    cu = p.cu_seqlens.numpy()
    threads = oracle.max_threads()
    log("cpu baseline: oracle prefill on %d threads ..." % threads)
    t0 = time.perf_counter()
    oracle.kda_recurrent(*args, cu, scale=p.scale, h0=h0)
    t_prefill = time.perf_counter() - t0
    state = dd.state.double().numpy()
    B = state.shape[0]
    cud = np.arange(B + 1, dtype=np.int64)
    dsteps = [[f32(st[n]) for n in ("q", "k", "v", "g", "beta_raw")] for st in dd.steps[:2]]
    dA, ddt = f32(dd.A_log), f32(dd.dt_bias)
    log("cpu baseline: oracle decode ...")
    t0 = time.perf_counter()
    for st in dsteps:
        _, state = oracle.kda_recurrent(*st, dA, ddt, cud, scale=dd.scale, h0=state)
    t_decode = (time.perf_counter() - t0) / len(dsteps)
    tokens = p.T + B
    # one thread, a head sample of the prefill
    hs = slice(0, heads_1t)
    sub = [np.ascontiguousarray(a[:, hs]) for a in args[:5]] + \
          [np.ascontiguousarray(args[5][hs]), np.ascontiguousarray(args[6][hs])]
    log("cpu baseline: oracle prefill on 1 thread, %d of %d heads ..." % (heads_1t, p.H))
    t0 = time.perf_counter()
    oracle.kda_recurrent(*sub, cu, scale=p.scale, h0=np.ascontiguousarray(h0[:, hs]), nthreads=1)
    t_1 = (time.perf_counter() - t0) * p.H / heads_1t
    return {"value": round(tokens / (t_prefill + t_decode), 1), "unit": "tokens/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "one full prefill T=8192 H=96 (%.2f s) + mean of 2 decode steps "
                      "B=256 H=32 (%.2f s/step), fp64, OpenMP over (sequence, head) chains"
                      % (t_prefill, t_decode),
            "one_thread": {"prefill_tokens_per_s": round(p.T / t_1, 1),
                           "sample": "prefill T=8192 over %d of %d heads on 1 thread, scaled "
                                     "to all heads (%.2f s for the whole prefill)"
                                     % (heads_1t, p.H, t_1)}}


if __name__ == "__main__":
    main()
