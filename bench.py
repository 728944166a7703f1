"""Benchmark of the RAM-Net layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for a prefill workload, one ramnet_scan_prefill call (address decoding for
every token, CAPE, the Gated Sparse Update, read, RMSNorm and gate over all
B x T x H token-heads); for the decode workload, one ramnet_step_decode call
(one token for each of B sequences, all heads).  Inputs are resident in HBM
before the timed region.  Prints one JSON line.

Default: the headline is the largest single-GPU workload, the 4^8-slot
prefill (large_state: B 2, T 32768, H 16, K 32); the line carries the other
workloads as sub-records ("subrecords"), each the whole call with its own
roofline and CPU baseline: the Top-8 and Top-32 prefills (--steps calls
each) and the decode workload (1024 dependent steps in one HIP graph), then
the rows beyond the five configurations: the 4^8-slot backward
(backward_large_state) and the decoding workload on a tiered state
(decode_tiered).
Device peaks are measured first (a 256 MiB copy, an LDS read probe) and
every roofline fraction is given against both the vendor's figure and the
measured one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload prefill_top8|prefill_top32|large_state|decode
                                   |layer_top8|layer_decode|backward_top8
                                   |backward_top32|backward_large_state
                                   |decode_tiered]
--workload runs that workload alone (no sub-records).  The layer_* workloads
add the dense projections either side (the whole layer); backward_top8 /
backward_top32 / backward_large_state time the gradients of those prefills;
decode_tiered runs the decoding workload with its rows in pinned host memory
and a quarter of them cached in HBM.
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
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
# LDS has no vendor figure in bytes per second; this one is derived from
# 128 bytes per clock per compute unit, 256 units at 2.4 GHz.  The measured
# read bandwidth (probe below) is reported beside it.
LDS_PEAK_GBS = 128 * 256 * 2.4
HEADLINE = "large_state"
SUBRECORDS = ("prefill_top8", "prefill_top32", "decode")
# (workload, steps, warmup) of the records beyond the five configurations
EXTRA_SUBRECORDS = (("backward_large_state", 3, 1), ("decode_tiered", 256, 8))




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
    "decode_addresses": ("decode_fast_kernel", "decode_fallback_kernel", "decode_kernel"),
    "scan_stage": ("plan_kernel", "scan_kernel", "rms_gate_kernel", "plan_range_kernel",
                   "scan_range_kernel", "gate_partials_kernel"),
    "step_fused": ("step_fused_kernel",),
}


# Sources of the kernels whose HBM counters profiles/hbm_traffic.json holds:
# the decoder, the prefill stages and the fused step, with their shared
# device helpers and argument structs.
TRAFFIC_SOURCES = ("decode.hip", "scan_chunked.hip", "scan_ranges.hip", "scan_serial.hip",
                   "step_fused.hip", "chunk_common.h", "device_common.h", "launch.h")


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
        if name.split("<")[0].split("(")[0] in STAGE_KERNELS.get(stage, ()):
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


def cpu_baseline(w, kind: str, run_s: float = 2.5):
    """Times the CPU oracle as it stands (plain C, fp64, prefix-tree Top-K,
    OpenMP over the independent (batch, head) units) on a bounded sample of
    the same workload: a prefix of the sequences (prefill) or of the steps
    (decode) sized to about `run_s` seconds per run; one warm-up run, then
    the median of three.  Reports tokens/s."""
    import oracle
    from sparse_slot_recurrent_amd import synth
    oracle.load()
    threads = oracle.max_threads()
    sb = w.state_dtype == "bf16"
    tree = oracle.TOPK_TREE

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    if kind == "decode":
        x0 = synth.make_inputs(w, T=1)
        steps_in = []

        def run(n):
            S, m, pos = x0["S0"].copy(), x0["m0"].copy(), x0["pos0"].copy()
            while len(steps_in) < n:
                s = synth.make_decode_step(w, len(steps_in))
                steps_in.append({k: np.ascontiguousarray(s[k][:, None]) for k in s})
            t = 0.0
            for i in range(n):
                a = steps_in[i]
                t += timed(lambda: oracle.layer(a["q"], a["k"], a["v"], a["gamma"], a["g"],
                                                S, m, d_p=w.d_p, U=w.U, K=w.K,
                                                state_bf16=sb, pos0=pos + i, mode=tree,
                                                want_addresses=False))
            return t
        n = max(1, min(w.steps, int(run_s / max(run(1), 1e-4))))
        run(n)  # warm-up
        med = float(np.median([run(n) for _ in range(3)]))
        return {"value": w.B * n / med, "unit": "tokens/s",
                "cores": min(threads, w.B * w.H), "kind": "oracle",
                "sample": f"{n} of {w.steps} decode steps, all {w.B} sequences x {w.H} "
                          f"heads (prefix-tree Top-K, fp64); median of 3 runs of "
                          f"{med:.2f} s after a warm-up",
                "cpu": cpu_info()}
    H = w.H
    B = max(1, min(w.B, threads // H))
    T = min(w.T, 64)

    def run(x):
        S, m = x["S0"].copy(), x["m0"].copy()
        return timed(lambda: oracle.layer(x["q"], x["k"], x["v"], x["gamma"], x["g"], S, m,
                                          d_p=w.d_p, U=w.U, K=w.K, state_bf16=sb,
                                          pos0=x["pos0"], mode=tree, want_addresses=False))
    while True:
        x = synth.make_inputs(w, B=B, T=T, H=H)
        dt = run(x)
        if dt >= run_s / 2 or (T == w.T and B == w.B):
            break
        grow = max(1.2, min(8.0, run_s / max(dt, 1e-3)))
        if T < w.T:
            T = min(w.T, int(T * grow) + 1)
        else:
            B = min(w.B, int(B * grow) + 1)
    x = synth.make_inputs(w, B=B, T=T, H=H)
    run(x)  # warm-up
    med = float(np.median([run(x) for _ in range(3)]))
    return {"value": B * T / med, "unit": "tokens/s",
            "cores": min(threads, B * H), "kind": "oracle",
            "sample": f"B={B} x T={T} tokens x {H} heads of the workload (prefix-tree "
                      f"Top-K, fp64); median of 3 runs of {med:.2f} s after a warm-up",
            "cpu": cpu_info()}


def measure_peaks(torch):
    """Measured device peaks: HBM bandwidth of a 256 MiB device copy (bytes
    read plus bytes written per second) and LDS read bandwidth (ds_read_b128
    on every compute unit), each the best of 10 launches after 3 warm-ups,
    timed with HIP events on the launch stream."""
    import ctypes as C
    path = os.path.join(ROOT, "sparse_slot_recurrent_amd", "libramnet_probe.so")
    lib = C.CDLL(path)
    lib.probe_hbm_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int, C.c_void_p]
    lib.probe_lds_read.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    st = torch.cuda.current_stream()
    sp = C.c_void_p(st.cuda_stream)
    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    blocks = 256 * 8

    def best(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return min(ts)
    t_copy = best(lambda: lib.probe_hbm_copy(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()),
                                             nbytes // 16, blocks, sp))
    assert torch.equal(src, dst), "copy probe"
    del src, dst
    iters = 256
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    t_lds = best(lambda: lib.probe_lds_read(blocks, iters, C.c_void_p(out.data_ptr()), sp))
    lds_bytes = blocks * 256 * iters * 16 * 16
    return {"hbm_copy_gbs": 2 * nbytes / t_copy / 1e9, "lds_read_gbs": lds_bytes / t_lds / 1e9,
            "hbm_vendor_gbs": HBM_PEAK_GBS, "lds_derived_gbs": LDS_PEAK_GBS,
            "method": "256 MiB copy (read + write bytes) and ds_read_b128 on 2048 "
                      "workgroups; best of 10 after 3 warm-ups"}


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

    def export(_):
        plan(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, mass, out, pos0=pos0, addr_out=addr)

    def scan(_):
        plan(d["q"], d["k"], d["v"], d["gamma"], d["g"], S, mass, out,
             pos0=pos0, addr_in=addr)

    for _ in range(warmup):
        step(0)
    torch.cuda.synchronize()
    ms = time_loop(torch, step, steps)
    torch.cuda.synchronize()
    # The decoder's share of the call: the call minus its recurrence stage
    # (the same call with the addresses given), each timed over the same
    # number of launches on the same stream.
    export(0)
    scan(0)
    ms_scan = time_loop(torch, scan, steps)
    torch.cuda.synchronize()
    tokens = w.B * w.T
    return ms, {"decode_addresses": max(ms - ms_scan, 0.0), "scan_stage": ms_scan}, tokens


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

# The decoding workload on a tiered state (rows in pinned host memory, M / 4
# rows of each unit cached in HBM, a rebalance every 64 steps).
TIERED = {"decode_tiered": ("decode", 4, 64)}


def host_link_peaks(torch, rn):
    """Kernel copies between pinned host memory and HBM (64 MiB, 16-byte
    loads and stores, the probe's grid-stride copy): bytes per second over
    the host link each way, best of 5 after 2 warm-ups."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "sparse_slot_recurrent_amd", "libramnet_probe.so"))
    lib.probe_hbm_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int, C.c_void_p]
    rl = rn.load_library()
    nbytes = 64 << 20
    hp = C.c_void_p()
    if rl.ramnet_host_alloc(nbytes, C.byref(hp)) != 0:
        raise RuntimeError(rl.ramnet_last_error().decode())
    dev = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    sp = C.c_void_p(st.cuda_stream)

    def best(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return min(ts)
    try:
        dp = C.c_void_p(dev.data_ptr())
        t_rd = best(lambda: lib.probe_hbm_copy(hp, dp, nbytes // 16, 2048, sp))
        t_wr = best(lambda: lib.probe_hbm_copy(dp, hp, nbytes // 16, 2048, sp))
    finally:
        torch.cuda.synchronize()
        rl.ramnet_host_free(hp)
    return {"host_read_gbs": nbytes / t_rd / 1e9, "host_write_gbs": nbytes / t_wr / 1e9,
            "method": "64 MiB kernel copy pinned host -> HBM and HBM -> pinned host, best of 5"}


def bench_decode_tiered(torch, rn, w, frac_den, every, steps, warmup):
    """The decoding workload's steps on a tiered state: the rows in pinned
    host memory, M / frac_den rows of each unit cached in HBM, a rebalance
    after every `every` steps (inside the timed region).  Returns (ms per
    step, per-kernel ms, tokens per step, extra fields: cache hit fraction of
    one step's accesses, host-link bytes per step, device bytes held)."""
    from sparse_slot_recurrent_amd import synth
    init = synth.make_inputs(w, T=1)
    S = to_dev(torch, init["S0"], w.state_dtype)
    mass = to_dev(torch, init["m0"], "f32")
    pos0 = torch.from_numpy(init["pos0"]).cuda()
    del init
    lines = w.M // frac_den
    ts = rn.TieredState(S, lines)
    del S
    ind = rn.BF16 if w.in_dtype == "bf16" else rn.F32
    sd = rn.BF16 if w.state_dtype == "bf16" else rn.F32
    p = rn.make_params(w.B, 1, w.H, w.d_p, w.U, w.K, w.d_v, ind, sd, cape=w.cape,
                       eps_gsu=w.eps_gsu, eps_norm=w.eps_norm)
    rn.tier_reset(p, ts)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    bdt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    n_in = min(steps, 256)  # distinct inputs, cycled

    def normal(*shape, sigma=1.0):
        return (torch.randn(*shape, generator=gen, device="cuda") * sigma).to(bdt)
    q = normal(n_in, w.B, w.H, w.L, sigma=w.logit_sigma)
    k = normal(n_in, w.B, w.H, w.L, sigma=w.logit_sigma)
    v = normal(n_in, w.B, w.H, w.d_v)
    gam = normal(n_in, w.B, w.H)
    g = normal(n_in, w.B, w.H, w.d_v)
    pos = (pos0[None, :] + torch.arange(n_in, device="cuda", dtype=torch.int32)[:, None]).contiguous()
    sdt = torch.bfloat16 if w.state_dtype == "bf16" else torch.float32
    out = torch.empty((w.B, w.H, w.d_v), dtype=sdt, device="cuda")

    def one(i):
        j = i % n_in
        rn.step_decode_tiered(p, q[j], k[j], v[j], gam[j], g[j], pos[j], ts, mass, out)

    def step(i):
        one(i)
        if (i + 1) % every == 0:
            rn.tier_rebalance(p, ts)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms = time_loop(torch, step, steps)
    ms_step = time_loop(torch, one, min(steps, 64))
    ms_reb = time_loop(torch, lambda i: rn.tier_rebalance(p, ts), 4)
    # one step's accesses served from the cache (the maps do not change
    # during a step)
    ao = rn.new_addresses((w.B, w.H, w.K), "cuda")
    rn.step_decode_tiered(p, q[0], k[0], v[0], gam[0], g[0], pos[0], ts, mass, out, addr_out=ao)
    torch.cuda.synchronize()
    sl = ts.slot_line.view(w.B * w.H, w.M)
    u = torch.arange(w.B * w.H, device="cuda")[:, None]
    hw = (sl[u, ao.w_idx.view(w.B * w.H, w.K).long()] >= 0).float().mean().item()
    hr = (sl[u, ao.r_idx.view(w.B * w.H, w.K).long()] >= 0).float().mean().item()
    b_s = 2 if w.state_dtype == "bf16" else 4
    rb = w.d_v * b_s
    units = w.B * w.H
    link = units * w.K * rb * (2 * (1 - hw) + (1 - hr))  # missed rows: writes read + written, reads read
    dev_bytes = units * (lines * rb + lines * 4 + w.M * 12)  # cache, line map, slot map, counts, mass
    extra = {"cache_lines_per_unit": lines, "rebalance_every": every,
             "hit_fraction": {"write_rows": hw, "read_rows": hr},
             "host_link_bytes_per_step": link, "device_bytes": dev_bytes,
             "full_state_bytes": units * w.M * (rb + 4)}
    return ms, {"step_tiered": ms_step, "rebalance": ms_reb}, w.B, extra



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
BACKWARD = {"backward_top8": "prefill_top8", "backward_top32": "prefill_top32",
            "backward_large_state": "large_state"}


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
    if w.M > 1024 or w.d_v != 64:
        # the per-token walk keeps the state in HBM: per token-head the replay
        # reads and writes K write rows and reads K read rows, and the adjoint
        # reads and writes K rows of dS (fp32) for the writes and K for the reads
        state += n * w.K * w.d_v * (3 * b_s + 4 * 4)
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


def prefill_roofline(w, kind, kms, bm, peaks):
    """Roofline of the dominant stage: algorithmic bytes over its measured
    time, against the HBM or the LDS peak, whichever term takes longer at
    peak (LDS only for a state held on chip, in the scan stage); the
    fraction against the vendor's (or derived) peak and against the
    measured one."""
    dom = max(kms, key=kms.get)
    sec = kms[dom] / 1e3
    lds = bm["lds_state"] if dom == "scan_stage" else 0
    if lds / LDS_PEAK_GBS > bm.get(dom, 0) / HBM_PEAK_GBS:
        a = lds / sec / 1e9
        return {"bound": "lds", "kernel": dom, "achieved": a, "peak": LDS_PEAK_GBS,
                "unit": "GB/s", "frac": a / LDS_PEAK_GBS,
                "peak_measured": peaks.get("lds_read_gbs"),
                "frac_measured": a / peaks["lds_read_gbs"] if peaks.get("lds_read_gbs") else None,
                "hbm_frac": bm[dom] / sec / 1e9 / HBM_PEAK_GBS,
                "traffic": measured_traffic(w.name, dom)}
    a = bm[dom] / sec / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a / HBM_PEAK_GBS, "peak_measured": peaks.get("hbm_copy_gbs"),
            "frac_measured": a / peaks["hbm_copy_gbs"] if peaks.get("hbm_copy_gbs") else None,
            "traffic": measured_traffic(w.name, dom)}


def workload_config(name, w, kind):
    return {"workload": name, "B": w.B, "T": 1 if kind == "decode" else w.T, "H": w.H,
            "M": w.M, "d_p": w.d_p, "U": w.U, "K": w.K, "d_v": w.d_v,
            "in_dtype": w.in_dtype, "state_dtype": w.state_dtype, "cape": w.cape,
            "steps": w.steps if kind == "decode" else None, "parallelism": "single GPU"}


def measure_workload(torch, rn, name, steps, warmup, peaks, cpu: bool):
    """One workload's record: tokens/s of the whole call, per-stage times,
    the roofline of the dominant stage and the CPU oracle beside it."""
    from sparse_slot_recurrent_amd import synth
    w = synth.WORKLOADS[name]
    kind = "decode" if w.steps else "prefill"
    extra = {}
    if kind == "decode":
        # the 1024 dependent steps of the workload, replayed as one graph
        steps = w.steps
        ms, kms, tokens, extra = bench_decode(torch, rn, w, steps, warmup)
    else:
        ms, kms, tokens = bench_prefill(torch, rn, w, steps, warmup)
    bm = byte_model(w, kind)
    if kind == "decode":
        a = bm["step_fused"] / (kms["step_fused"] / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "step_fused", "achieved": a, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": a / HBM_PEAK_GBS,
                "peak_measured": peaks.get("hbm_copy_gbs"),
                "frac_measured": a / peaks["hbm_copy_gbs"] if peaks.get("hbm_copy_gbs") else None,
                "traffic": measured_traffic(w.name, "step_fused")}
    else:
        roof = prefill_roofline(w, kind, kms, bm, peaks)
    rec = {"workload": name, "value": tokens / (ms / 1e3), "unit": "tokens/s",
           "ms_per_step": ms, "steps": steps, "config": workload_config(name, w, kind),
           "roofline": roof, "kernels_ms": kms, "algorithmic_bytes": bm,
           "whole_step_hbm_frac": bm["total"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
    rec.update(extra)
    if cpu:
        rec["cpu_baseline"] = cpu_baseline(w, kind)
    return rec


def measure_extra(torch, rn, name, steps, warmup):
    """A record for a workload beyond the five configurations: a whole layer
    (layer_*), a backward pass (backward_*) or the tiered decoding state
    (decode_tiered)."""
    from sparse_slot_recurrent_amd import synth
    backward, tiered = name in BACKWARD, name in TIERED
    d_model = None
    if backward:
        w = synth.WORKLOADS[BACKWARD[name]]
    elif tiered:
        w = synth.WORKLOADS[TIERED[name][0]]
    else:
        base, d_model = LAYERS[name]
        w = synth.WORKLOADS[base]
    kind = "decode" if w.steps else "prefill"
    extra = {}
    if tiered:
        _, den, every = TIERED[name]
        ms, kms, tokens, extra = bench_decode_tiered(torch, rn, w, den, every, steps, warmup)
        hl = host_link_peaks(torch, rn)
        a = extra["host_link_bytes_per_step"] / (kms["step_tiered"] / 1e3) / 1e9
        peak = min(hl["host_read_gbs"], hl["host_write_gbs"])
        roof = {"bound": "host_link", "kernel": "step_tiered", "achieved": a, "peak": peak,
                "unit": "GB/s", "frac": a / peak, "traffic": None, "host_link": hl}
    elif backward:
        ms, kms, tokens, extra = bench_backward(torch, rn, w, steps, warmup)
        bw = backward_model(w)
        extra["backward_model"] = bw
        a = bw["backward"] / (ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "backward", "achieved": a, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": a / HBM_PEAK_GBS, "traffic": None,
                "with_records_gbs": (bw["backward"] + bw["records"]) / (ms / 1e3) / 1e9}
    else:
        ms, kms, tokens, extra = bench_layer(torch, rn, w, d_model, steps, warmup)
        roof = layer_roofline(w, d_model, kind, kms, ms, extra)
    rec = {"workload": name, "value": tokens / (ms / 1e3), "unit": "tokens/s",
           "ms_per_step": ms, "steps": steps, "config": workload_config(name, w, kind),
           "roofline": roof, "kernels_ms": kms}
    rec.update(extra)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    help="run one workload alone (default: the headline with sub-records)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subrecords", action="store_true")
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
    torch.cuda.set_device(0)
    torch.cuda.synchronize()
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    name = args.workload or HEADLINE
    single = args.workload is not None
    cpu = not args.no_cpu_baseline
    d_model = None
    if name in LAYERS:
        # time hipBLASLt's candidates once per GEMM shape, before the timed
        # region (the library's opt-in tuning)
        os.environ["RAMNET_GEMM_TUNE"] = "1"
    backward = name in BACKWARD
    tiered = name in TIERED
    if backward:
        w = synth.WORKLOADS[BACKWARD[name]]
    elif tiered:
        w = synth.WORKLOADS[TIERED[name][0]]
    elif name in LAYERS:
        base, d_model = LAYERS[name]
        w = synth.WORKLOADS[base]
    else:
        w = synth.WORKLOADS[name]
    kind = "decode" if w.steps else "prefill"
    steps = args.steps or (w.steps if kind == "decode" else 10)
    warmup = args.warmup if args.warmup is not None else (8 if kind == "decode" else 2)
    peaks = {} if single else measure_peaks(torch)
    line = {"metric": METRIC}
    if backward or tiered or d_model is not None:
        rec = measure_extra(torch, rn, name, steps, warmup)
    else:
        rec = measure_workload(torch, rn, name, steps, warmup, peaks, cpu)
        steps = rec["steps"]
    line.update({
        "value": rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        # arithmetic: fp32 (Top-K decisions exact: integer or fp64 logit sums); storage in "config"
        "dtype": "f32", "data": "synthetic",
    })
    for k in ("config", "roofline", "cpu_baseline", "kernels_ms", "algorithmic_bytes",
              "whole_step_hbm_frac"):
        if k in rec:
            line[k] = rec[k]
    for k, v in rec.items():
        if k not in line and k not in ("workload", "steps"):
            line[k] = v
    if peaks:
        line["device_peaks"] = peaks
    if not single and not args.no_subrecords:
        line["subrecords"] = [measure_workload(torch, rn, n, steps if n != "decode" else None,
                                               warmup, peaks, cpu) for n in SUBRECORDS]
        # rows beyond the five configurations: the 4^8-slot backward and the
        # tiered decoding state, a few steps each
        line["subrecords"] += [measure_extra(torch, rn, n, st, wu) for n, st, wu in EXTRA_SUBRECORDS]
    print(json.dumps(line), flush=True)


def layer_roofline(w, d_model, kind, kms, ms, extra):
    """Roofline of a whole-layer workload: the projections against the bf16
    matrix-core peak, or the recurrence against HBM, whichever stage is
    longer; a graph-replayed step against HBM for its whole bytes."""
    bm = byte_model(w, kind)
    lm = layer_model(w, d_model, kind)
    extra["layer_model"] = lm
    extra["d_model"] = d_model
    dom = max(kms, key=kms.get)
    if "projections" in kms:
        flop = lm["project_inputs_flop"] + lm["project_output_flop"]
        tf = flop / (kms["projections"] / 1e3) / 1e12
        extra["projections_tflops"] = tf
        rec = bm["total"] / (kms["recurrence"] / 1e3) / 1e9
        extra["recurrence_gbs"] = rec
        if dom == "projections":
            return {"bound": "mfma", "kernel": dom, "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS, "traffic": None}
        return {"bound": "hbm", "kernel": dom, "achieved": rec, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": rec / HBM_PEAK_GBS, "traffic": None}
    by = bm["total"] + lm["project_inputs_bytes"] + lm["project_output_bytes"]
    a = by / (ms / 1e3) / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a / HBM_PEAK_GBS, "traffic": None}


if __name__ == "__main__":
    main()
