"""Benchmark of the RAM-Net layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for a prefill workload, one ramnet_scan_prefill call (address decoding for
every token, CAPE, the Gated Sparse Update, read, RMSNorm and gate over all
B x T x H token-heads); for the decode workload, one ramnet_step_decode call
(one token for each of B sequences, all heads).  Inputs are resident in HBM
before the timed region.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload prefill_top8|prefill_top32|large_state|decode
                                   |layer_top8|layer_decode|backward_top8
                                   |backward_top32]
The layer_* workloads add the dense projections either side (the whole layer);
backward_top8 / backward_top32 time the gradients of those prefills.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("tokens/sec per RAM-Net layer (prefill scan + decode step), "
          "% of HBM roofline")
HBM_PEAK_GBS = 8000.0
# LDS: 128 bytes per clock per compute unit, 256 units at 2.4 GHz.
LDS_PEAK_GBS = 128 * 256 * 2.4




def byte_model(w, kind: str):
    """Algorithmic bytes per launch of each kernel (what the method must
    move, per the token-head byte model; no address round trip, no re-reads).
      decode_addresses: q and k logits, 2*U*d_p*b_in per token-head.
      scan_stage:       (the plan, scan and RMSNorm/gate kernels of one
                        prefill call with given addresses)
                        v, g (2*d_v*b_in), gamma (b_in) in, out (d_v*b_s),
                        plus the state traffic.  Each token-head's step
                        touches 3*K*d_v*b_s + 2*K*4 bytes of state (K write
                        rows read and written, K read rows read, K masses
                        read and written).  A state held on chip for the
                        whole launch (M <= 1024) costs HBM only its one
                        load and store per (batch, head) unit, and the
                        per-step traffic goes to LDS instead ("lds_state");
                        a state in HBM (decode step, 4^8 slots) costs the
                        per-step traffic in HBM.  The once-per-launch figure
                        of an HBM state is reported alongside as a lower
                        bound no chunked design reaches.
    """
    b_in = 2 if w.in_dtype == "bf16" else 4
    b_s = 2 if w.state_dtype == "bf16" else 4
    T = 1 if kind == "decode" else w.T
    n = w.B * T * w.H
    units = w.B * w.H
    dec = n * 2 * w.L * b_in
    io = n * (2 * w.d_v * b_in + b_in + w.d_v * b_s)
    once = units * 2 * (w.M * w.d_v * b_s + 4 * w.M)
    rows = n * (3 * w.K * w.d_v * b_s + 2 * w.K * 4)
    resident = kind == "prefill" and w.M <= 1024
    state = once if resident else rows
    out = {"decode_addresses": dec, "scan_stage": io + state,
           "total": dec + io + state, "state_term": state,
           "lds_state": rows if resident else 0, "once_per_launch_state": once}
    if kind == "decode":
        out["step_fused"] = out["total"]  # one kernel does the whole step
    return out


STAGE_KERNELS = {
    "decode_addresses": ("decode_kernel",),
    "scan_stage": ("plan_kernel", "mass_fanout_kernel", "scan_kernel", "rms_gate_kernel"),
    "step_fused": ("step_fused_kernel",),
}


# Sources of the kernels whose HBM counters profiles/hbm_traffic.json holds:
# the decoder, the prefill stages and the fused step, with their shared
# device helpers and argument structs.
TRAFFIC_SOURCES = ("decode.hip", "scan_chunked.hip", "scan_serial.hip", "step_fused.hip",
                   "device_common.h", "launch.h")


def kernel_source_hash():
    """sha256 over the measured kernels' sources, to tell whether recorded
    counters still describe the kernels being run."""
    import hashlib
    h = hashlib.sha256()
    here = os.path.dirname(os.path.abspath(__file__))
    for name in TRAFFIC_SOURCES:
        h.update(name.encode())
        with open(os.path.join(here, "sparse_slot_recurrent_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of a stage from rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (scaled by a device copy of known size), recorded in
    profiles/hbm_traffic.json; None when absent or when the kernel sources
    changed since the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("_kernel_source_sha256") != kernel_source_hash() or workload not in rec:
        return None
    total, found = 0.0, False
    for name, v in rec[workload]["kernels"].items():
        if name.split("<")[0] in STAGE_KERNELS.get(stage, ()):
            total += v["fetch_bytes"] + v["write_bytes"]
            found = True
    return total if found else None


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(w, kind: str, budget_s: float = 12.0):
    """Times the CPU oracle (as it is: brute-force Top-K, fp64, OpenMP over
    (batch, head) units) on a bounded sample of the same workload: a prefix
    of the sequences sized to about `budget_s` seconds, or the whole batch
    when that is cheaper; reports tokens/s."""
    import oracle
    from sparse_slot_recurrent_amd import synth
    oracle.load()
    threads = oracle.max_threads()
    sb = w.state_dtype == "bf16"
    if kind == "decode":
        steps = 0
        S = m = pos = None
        t_all = 0.0
        x0 = synth.make_inputs(w, T=1)
        S, m, pos = x0["S0"].copy(), x0["m0"].copy(), x0["pos0"].copy()
        while t_all < budget_s and steps < w.steps:
            s = synth.make_decode_step(w, steps)
            a = {n: s[n][:, None] for n in s}
            t0 = time.perf_counter()
            oracle.layer(a["q"], a["k"], a["v"], a["gamma"], a["g"], S, m,
                         d_p=w.d_p, U=w.U, K=w.K, state_bf16=sb, pos0=pos,
                         want_addresses=False)
            t_all += time.perf_counter() - t0
            pos = pos + 1
            steps += 1
        return {"value": w.B * steps / t_all, "unit": "tokens/s",
                "cores": threads, "kind": "oracle",
                "sample": f"{steps} decode steps of all {w.B} sequences x "
                          f"{w.H} heads, {t_all:.1f} s of oracle time",
                "cpu": cpu_info()}
    H = w.H
    B = max(1, min(w.B, threads // H))
    T = min(w.T, 64)
    while True:
        x = synth.make_inputs(w, B=B, T=T, H=H)
        S, m = x["S0"].copy(), x["m0"].copy()
        t0 = time.perf_counter()
        oracle.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S, m,
                     d_p=w.d_p, U=w.U, K=w.K, state_bf16=sb, pos0=x["pos0"],
                     want_addresses=False)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or (T == w.T and B == w.B):
            break
        grow = max(2.0, min(8.0, budget_s / 2 / max(dt, 1e-3)))
        if T < w.T:
            T = min(w.T, int(T * grow))
        else:
            B = min(w.B, int(B * grow) + 1)
    return {"value": B * T / dt, "unit": "tokens/s",
            "cores": min(threads, B * H), "kind": "oracle",
            "sample": f"B={B} x T={T} tokens x {H} heads of the workload "
                      f"(brute-force Top-K, fp64), {dt:.1f} s",
            "cpu": cpu_info()}


def to_dev(torch, a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def time_loop(torch, fn, steps):
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        fn(i)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prefill(torch, rn, w, steps, warmup):
    from sparse_slot_recurrent_amd import synth
    x = synth.make_inputs(w)
    d = {n: to_dev(torch, x[n], w.in_dtype) for n in ("q", "k", "v", "gamma", "g")}
    S = to_dev(torch, x["S0"], w.state_dtype)
    mass = to_dev(torch, x["m0"], "f32")
    pos0 = torch.from_numpy(x["pos0"]).cuda()
    del x
    sdt = torch.bfloat16 if w.state_dtype == "bf16" else torch.float32
    out = torch.empty((w.B, w.T, w.H, w.d_v), dtype=sdt, device="cuda")
    plan = rn.PrefillPlan(w.B, w.T, w.H, w.d_p, w.U, w.K, w.d_v,
                          rn.BF16 if w.in_dtype == "bf16" else rn.F32,
                          rn.BF16 if w.state_dtype == "bf16" else rn.F32,
                          cape=w.cape, eps_gsu=w.eps_gsu, eps_norm=w.eps_norm)
    addr = rn.new_addresses((w.B, w.T, w.H, w.K), "cuda")

    def step(_):
        plan(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, mass, out, pos0=pos0)

    def dec(_):
        rn.decode_addresses(d["q"], d["k"], d_p=w.d_p, U=w.U, K=w.K,
                            cape=w.cape, pos0=pos0, out=addr)

    def scan(_):
        plan(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, mass, out,
             pos0=pos0, addr_in=addr)

    for _ in range(warmup):
        step(0)
    torch.cuda.synchronize()
    ms = time_loop(torch, step, steps)
    torch.cuda.synchronize()
    # per-kernel averages over the same number of launches, same stream
    dec(0)
    ms_dec = time_loop(torch, dec, steps)
    scan(0)
    ms_scan = time_loop(torch, scan, steps)
    torch.cuda.synchronize()
    tokens = w.B * w.T
    return ms, {"decode_addresses": ms_dec, "scan_stage": ms_scan}, tokens


def bench_decode(torch, rn, w, steps, warmup):
    """1024 dependent decoding steps (one fused kernel each) from a
    pre-filled state, captured in one HIP graph; eager launches are timed
    too.  Returns (ms per step from the graph, per-kernel ms, tokens per
    step, extra fields)."""
    from sparse_slot_recurrent_amd import synth
    init = synth.make_inputs(w, T=1)
    S = to_dev(torch, init["S0"], "bf16")
    mass = to_dev(torch, init["m0"], "f32")
    pos0 = torch.from_numpy(init["pos0"]).cuda()
    del init
    # distinct per-step inputs for every step, drawn on the device
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    bdt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32

    def normal(*shape, sigma=1.0):
        return (torch.randn(*shape, generator=gen, device="cuda") * sigma).to(bdt)

    q = normal(steps, w.B, w.H, w.L, sigma=w.logit_sigma)
    k = normal(steps, w.B, w.H, w.L, sigma=w.logit_sigma)
    v = normal(steps, w.B, w.H, w.d_v)
    gam = normal(steps, w.B, w.H)
    g = normal(steps, w.B, w.H, w.d_v)
    pos = (pos0[None, :] + torch.arange(steps, device="cuda", dtype=torch.int32)[:, None]).contiguous()
    sdt = torch.bfloat16 if w.state_dtype == "bf16" else torch.float32
    out = torch.empty((w.B, w.H, w.d_v), dtype=sdt, device="cuda")
    plan = rn.StepPlan(w.B, w.H, w.d_p, w.U, w.K, w.d_v,
                       rn.BF16 if w.in_dtype == "bf16" else rn.F32,
                       rn.BF16 if w.state_dtype == "bf16" else rn.F32,
                       cape=w.cape, eps_gsu=w.eps_gsu, eps_norm=w.eps_norm)

    def step(i):
        plan(q[i], k[i], v[i], gam[i], g[i], pos[i], S, mass, out)

    for i in range(min(warmup, steps)):
        step(i)
    torch.cuda.synchronize()
    ms_eager = time_loop(torch, step, steps)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(steps):
                step(i)
    torch.cuda.current_stream().wait_stream(cap)
    graph.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(st)
    for _ in range(reps):
        graph.replay()
    e1.record(st)
    e1.synchronize()
    ms_graph = e0.elapsed_time(e1) / (reps * steps)
    return ms_graph, {"step_fused": ms_graph}, w.B, {"ms_per_step_eager": ms_eager}


# Whole-layer workloads: a configuration's recurrence with its dense
# projections, at a model width chosen for that configuration (d_model 1024
# for the 340M-like layer; 2048 = H*d_v for the 16-head decode layer).
LAYERS = {"layer_top8": ("prefill_top8", 1024), "layer_decode": ("decode", 2048)}


def layer_model(w, D, kind: str):
    """Algorithmic flops and bytes of the two projection stages (bf16
    operands and results; x read once, weights read once)."""
    T = 1 if kind == "decode" else w.T
    rows = w.B * T
    n_in = w.H * (2 * w.L + 2 * w.d_v + 1)
    hv = w.H * w.d_v
    return {
        "project_inputs_flop": 2 * rows * D * n_in,
        "project_inputs_bytes": 2 * (rows * D + D * n_in + rows * n_in),
        "project_output_flop": 2 * rows * hv * D,
        "project_output_bytes": 2 * (rows * hv + hv * D + rows * D),
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0

# Backward workloads: a prefill configuration's gradients (fp32 state).
BACKWARD = {"backward_top8": "prefill_top8", "backward_top32": "prefill_top32"}


def backward_model(w):
    """Algorithmic bytes of one backward call: per token-head the forward's
    inputs it reads (v, g, gamma, both logit rows, the K write and K read
    addresses as index and weight), dout, and the gradients it writes (dq, dk,
    dv, dg, dgamma, fp32); per (batch, head) unit the state and mass read
    once and their gradients written once.  The per-step state traffic stays
    on chip (registers) and is not counted; the records of the replay are
    implementation traffic and are reported separately."""
    b_in = 2 if w.in_dtype == "bf16" else 4
    n = w.B * w.T * w.H
    units = w.B * w.H
    per_th = (2 * w.d_v * b_in + b_in + 2 * w.L * b_in + 16 * w.K + 4 * w.d_v
              + 4 * (2 * w.L + 2 * w.d_v + 1))
    b_s = 2 if w.state_dtype == "bf16" else 4
    state = units * (w.M * w.d_v * (b_s + 4) + 8 * w.M)  # S0 read, dS0 (fp32) written
    records = n * (2 * w.K * w.d_v * 4 + 4 * w.K) * 2  # written by the replay, read back
    return {"backward": n * per_th + state, "records": records}


def bench_backward(torch, rn, w, steps, warmup):
    """ramnet_scan_backward on the forward's addresses (the forward runs once,
    outside the timed region)."""
    from sparse_slot_recurrent_amd import synth
    x = synth.make_inputs(w.replace(s0_sigma=0.3, m0_uniform=(0.2, 1.5)))
    bf = w.in_dtype == "bf16"
    d = {n: to_dev(torch, x[n], w.in_dtype) for n in ("q", "k", "v", "gamma", "g")}
    S0 = to_dev(torch, x["S0"], w.state_dtype)
    m0 = to_dev(torch, x["m0"], "f32")
    pos0 = torch.from_numpy(x["pos0"]).cuda()
    del x
    S, m = S0.clone(), m0.clone()
    _, addr = rn.scan_prefill(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, m, d_p=w.d_p,
                              U=w.U, K=w.K, cape=w.cape, pos0=pos0, export_addresses=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    dout = torch.randn(w.B, w.T, w.H, w.d_v, generator=gen, device="cuda")

    def step(_):
        rn.scan_backward(d["q"], d["k"], d["v"], d["gamma"], d["g"], S0, m0, addr, dout,
                         d_p=w.d_p, U=w.U, K=w.K, cape=w.cape, pos0=pos0)
    for _ in range(warmup):
        step(0)
    torch.cuda.synchronize()
    ms = time_loop(torch, step, steps)
    torch.cuda.synchronize()
    return ms, {"backward": ms}, w.B * w.T, {}


def bench_layer(torch, rn, w, D, steps, warmup):
    """A whole layer: ramnet_layer_forward (prefill, packing the input
    weights inside every call, as a training step would) or
    ramnet_layer_step (1024 dependent steps in one HIP graph, weights packed
    once beforehand).  Per-stage times (prefill): the recurrence alone on
    projected inputs, and the projections (packing, the input GEMM and the
    output GEMM) as the rest of the layer's time."""
    from sparse_slot_recurrent_amd import synth
    decode = bool(w.steps)
    T = 1 if decode else w.T
    wd = synth.make_layer_weights(w, D, T=1, kind="gauss", alpha="general")
    # the library takes weights as [out, in]; the generator writes [in, out]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a).T)).to(torch.bfloat16).cuda()
    W = rn.LayerWeights(bf(wd["w_q"]), bf(wd["w_k"]), bf(wd["w_v"]), bf(wd["w_g"]),
                        bf(wd["w_gamma"]), bf(wd["w_o"]), torch.from_numpy(wd["alpha"]).cuda())
    st = synth.make_inputs(w, T=1)
    sdt = torch.bfloat16 if w.state_dtype == "bf16" else torch.float32
    S = torch.from_numpy(st["S0"]).to(sdt).cuda()
    mass = torch.from_numpy(st["m0"]).cuda()
    pos0 = torch.from_numpy(st["pos0"]).cuda()
    del st
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    plan = rn.LayerPlan(w.B, T, w.H, w.d_p, w.U, w.K, w.d_v, D, sdt, cape=w.cape,
                        eps_gsu=w.eps_gsu, eps_norm=w.eps_norm, step=decode)
    if decode:
        # serving: the input weights are packed once, outside the steps
        W = rn.pack_weights(plan.p, W)
        xs = torch.randn(steps, w.B, D, generator=gen, device="cuda").to(torch.bfloat16)
        pos = (pos0[None, :] + torch.arange(steps, device="cuda", dtype=torch.int32)[:, None]).contiguous()
        y = torch.empty((w.B, D), dtype=torch.bfloat16, device="cuda")

        def step(i):
            plan(W, xs[i], S, mass, y, pos=pos[i])
        for i in range(min(warmup, steps)):
            step(i)
        torch.cuda.synchronize()
        ms_eager = time_loop(torch, step, steps)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(steps):
                    step(i)
        torch.cuda.current_stream().wait_stream(cap)
        graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            graph.replay()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / (3 * steps)
        return ms, {"layer_step": ms}, w.B, {"ms_per_step_eager": ms_eager}
    x = torch.randn(w.B, T, D, generator=gen, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(x)
    inp = plan.project_inputs(W, x)
    pre = rn.PrefillPlan(w.B, T, w.H, w.d_p, w.U, w.K, w.d_v, rn.BF16,
                         rn.BF16 if sdt == torch.bfloat16 else rn.F32, cape=w.cape,
                         eps_gsu=w.eps_gsu, eps_norm=w.eps_norm)
    out = torch.empty((w.B, T, w.H, w.d_v), dtype=sdt, device="cuda")

    def step(_):
        plan(W, x, S, mass, y, pos=pos0)

    def rec(_):
        pre(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["g"], S, mass, out, pos0=pos0)
    for _ in range(warmup):
        step(0)
    torch.cuda.synchronize()
    ms = time_loop(torch, step, steps)
    rec(0)
    ms_rec = time_loop(torch, rec, steps)
    torch.cuda.synchronize()
    kms = {"recurrence": ms_rec, "projections": max(ms - ms_rec, 1e-6)}
    return ms, kms, w.B * T, {}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="prefill_top8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device to device once (a plain copy "
                         "kernel of known size, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): every "
              "(batch, head) unit is independent, so more GPUs would each run "
              "this same kernel on their own share of B x H.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_slot_recurrent_amd import ramnet as rn
    from sparse_slot_recurrent_amd import synth
    rn.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    d_model = None
    backward = args.workload in BACKWARD
    if backward:
        w = synth.WORKLOADS[BACKWARD[args.workload]]
    elif args.workload in LAYERS:
        base, d_model = LAYERS[args.workload]
        w = synth.WORKLOADS[base]
    else:
        w = synth.WORKLOADS[args.workload]
    kind = "decode" if w.steps else "prefill"
    steps = args.steps or (w.steps if kind == "decode" else 10)
    warmup = args.warmup if args.warmup is not None else (8 if kind == "decode" else 2)
    torch.cuda.set_device(0)
    torch.cuda.synchronize()
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    extra = {}
    if backward:
        ms, kms, tokens, extra = bench_backward(torch, rn, w, steps, warmup)
    elif d_model is not None:
        ms, kms, tokens, extra = bench_layer(torch, rn, w, d_model, steps, warmup)
    elif kind == "decode":
        ms, kms, tokens, extra = bench_decode(torch, rn, w, steps, warmup)
    else:
        ms, kms, tokens = bench_prefill(torch, rn, w, steps, warmup)
    value = tokens / (ms / 1e3)
    bm = byte_model(w, kind)
    dom = max(kms, key=kms.get)
    roof = None
    if backward:
        bw = backward_model(w)
        extra["backward_model"] = bw
        a = bw["backward"] / (ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "backward", "achieved": a, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": a / HBM_PEAK_GBS, "traffic": None,
                "with_records_gbs": (bw["backward"] + bw["records"]) / (ms / 1e3) / 1e9}
    elif d_model is not None:
        lm = layer_model(w, d_model, kind)
        extra["layer_model"] = lm
        extra["d_model"] = d_model
        if "projections" in kms:
            flop = lm["project_inputs_flop"] + lm["project_output_flop"]
            tf = flop / (kms["projections"] / 1e3) / 1e12
            extra["projections_tflops"] = tf
            rec = bm["total"] / (kms["recurrence"] / 1e3) / 1e9
            extra["recurrence_gbs"] = rec
            if dom == "projections":
                roof = {"bound": "mfma", "kernel": dom, "achieved": tf,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None}
            elif dom == "recurrence":
                roof = {"bound": "hbm", "kernel": dom, "achieved": rec,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": rec / HBM_PEAK_GBS, "traffic": None}
        if roof is None:
            # one graph-replayed step: the whole layer's bytes (recurrence
            # plus both projections) over the step time
            by = bm["total"] + lm["project_inputs_bytes"] + lm["project_output_bytes"]
            a = by / (ms / 1e3) / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": a, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": a / HBM_PEAK_GBS, "traffic": None}
    else:
        # the bound is whichever of the HBM and LDS terms takes longer at
        # peak (LDS only for a state held on chip, in the scan stage)
        sec = kms[dom] / 1e3
        lds = bm["lds_state"] if dom == "scan_stage" else 0
        if lds / LDS_PEAK_GBS > bm[dom] / HBM_PEAK_GBS:
            achieved = lds / sec / 1e9
            roof = {"bound": "lds", "kernel": dom, "achieved": achieved,
                    "peak": LDS_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / LDS_PEAK_GBS, "hbm_frac": bm[dom] / sec / 1e9 / HBM_PEAK_GBS,
                    "traffic": measured_traffic(w.name, dom)}
        else:
            achieved = bm[dom] / sec / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": achieved,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS,
                    "traffic": measured_traffic(w.name, dom)}
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+f32" if d_model else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "T": 1 if kind == "decode" else w.T,
                   "H": w.H, "M": w.M, "d_p": w.d_p, "U": w.U, "K": w.K,
                   "d_v": w.d_v, "in_dtype": w.in_dtype,
                   "state_dtype": w.state_dtype, "cape": w.cape,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels_ms": kms,
        "algorithmic_bytes": bm,
        "whole_step_hbm_frac": bm["total"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
    }
    line.update(extra)
    if not args.no_cpu_baseline and d_model is None and not backward:
        line["cpu_baseline"] = cpu_baseline(w, kind)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
