#!/usr/bin/env python3
"""Throughput of the MI355X KDA forward on one GPU; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one KDA forward over the whole batch of the workload (default: B=2,
H=64, T=8192, dk=dv=128, chunk 64, fp32 beta, initial state ~ 0.1 N(0,1)) with
all inputs, outputs and the workspace already resident in HBM, in one of the
library's two forms: kda_fwd_fused (one launch of the single-pass kernel) or
kda_fwd_ws (the two kernels of kda_fwd on a caller-owned workspace).  With
--form auto (the default) both forms are timed, each for 20 calls after a
settle phase of its own, and the faster one is the step (settled again before
its warm-up); the JSON names it and gives both probe times.  The K timed
steps are bracketed by device synchronisation; value = tokens / wall time per
step.  `call_events` then times 50 more calls of the same form, each between
HIP events on the launch stream: median, minimum, mean and maximum.

Roofline (HBM-bound): the forward's algorithmic bytes (q, k, v, g, beta read
once, o written once, the initial state read if given, the final state
written) divided by the step's kernel time (HIP events on the launch stream): the
mean of `call_events` when kda_fused_kernel is the step, or the summed average
durations of the two-pass kernels, timed in batches of their own through the
stage entry points kda_fwd_intra and kda_fwd_scan.  Each two-pass kernel is also reported
against its own algorithmic bytes (the intra kernel reads q, k, g, beta and
writes one 61,952-byte record per chunk and value head; the scan kernel reads
v and the records and writes o and the states).  The MFMA side uses the
algorithmic flop count of the chunked method (4,512,416 MAC per full 64-token
chunk and value head).

cpu_baseline: the fp64 CPU oracle (token recurrence, OpenMP over sequence x head)
timed on a bounded sample of the same workload (by default all of it, run
repeatedly for at least 10 s), scaled to tokens/s of the full head count.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens/s (B=2,H=64,d=128,T=8192); ms/call; % of HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MAC_PER_CHUNK_HEAD = 4_512_416
# The forward kernels' sources and the build script that holds their compiler
# flags: counters taken on other code than these are not reported.
KERNEL_SOURCES = [os.path.join(ROOT, "gated_delta_rule_35_amd", "csrc", f)
                  for f in ("kda_intra.hip", "kda_scan.hip", "kda_fused.hip", "kda_device.h", "kda_kernel.h")] + \
                 [os.path.join(ROOT, "gated_delta_rule_35_amd", "build.py")]
RECORD_BYTES = 61952   # workspace record per (chunk, value head)
# The pages' own time for this exact workload ("cuLA PR #131: SM100/SM103 KDA
# forward to pure CuTeDSL", Performance table, fp32 beta, T=8192, B=2, H=64,
# CuTeDSL column), measured on NVIDIA SM100/SM103: context, not the target.
PAGES_MS = {"mha_b2_h64_t8192": 0.8564,
            # the same table: fp32 beta rows for T = 512, 1024, 4096; bf16 beta for T = 4096
            # without initial state; the grouped-value row (bf16 beta)
            "mha_b2_h64_t512": 0.0810, "mha_b2_h64_t1024": 0.1326, "mha_b2_h64_t4096_h0": 0.4263,
            "mha_b2_h64_t4096": 0.4362, "gva_b1_hq16_hv64_t4096": 0.2379}
KERNELS = ("kda_intra_kernel", "kda_scan_kernel")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


SETTLE_S = 0.25


def settle(call):
    """Runs `call` untimed for at least SETTLE_S seconds before the warm-up steps.
    From idle (as while the inputs are generated on the host) the GPU takes about
    35 ms of work to reach its steady clocks: the headline forward measured 0.99,
    0.80, 0.75, 0.73 ms per call over its first four blocks of ten calls and 0.72
    ms from the fifth on.  The timed steps then measure the steady state."""
    import torch
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < 1 or time.perf_counter() - t0 < SETTLE_S:
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"settled: {n} untimed calls in {time.perf_counter() - t0:.2f} s")



def algorithmic_bytes(n_tok, N, Hq, Hv, beta_bytes, has_h0, d=128):
    per_tok = Hq * d * 2 * 2 + Hv * d * 2 * 2 + Hv * d * 4 + Hv * beta_bytes
    states = N * Hv * d * d * 4 * (2 if has_h0 else 1)
    return n_tok * per_tok + states


def chunk_heads(lengths, Hv, C=64):
    return sum((L + C - 1) // C for L in lengths) * Hv


def kernel_bytes(n_tok, n_ch, N, Hq, Hv, beta_bytes, has_h0, d=128):
    """Algorithmic bytes of each kernel (n_ch = chunk-heads)."""
    qk = n_tok * Hq * d * 2 * 2
    g = n_tok * Hv * d * 4
    v = o = n_tok * Hv * d * 2
    b = n_tok * Hv * beta_bytes
    states = N * Hv * d * d * 4 * (2 if has_h0 else 1)
    rec = n_ch * RECORD_BYTES
    return {"kda_intra_kernel": qk + g + b + rec, "kda_scan_kernel": v + rec + o + states}


def kernel_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def load_traffic(workload):
    """HBM bytes per launch of each kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_kda_fwd_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def torch_float32():
    import torch
    return torch.float32


def _counter_medians(folder, counter):
    """Median per dispatch of `counter` for every kernel name in the rocprofv3
    counter-collection CSV files under `folder`."""
    import csv
    import glob
    vals = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    for f in files:
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    out = {}
    for name, v in vals.items():
        v = sorted(v)
        out[name] = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    return out


def write_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """profiles/traffic_kda_fwd_<workload>.json from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch, median over dispatches), each scaled by what
    the same counter reads for a 1 GiB device copy (bench.py --calibrate-copy)."""
    from gated_delta_rule_35_amd.inputs import WORKLOADS, varlen_lengths
    w = WORKLOADS[workload]
    lengths = varlen_lengths(w.varlen_total, w.length_seed) if w.varlen_total else [w.T] * w.B
    n_tok, N = sum(lengths), len(lengths)
    beta_bytes = 4 if w.beta_dtype == torch_float32() else 2
    copy_bytes = 1 << 30
    cf = [v for k, v in _counter_medians(copy_fetch_dir, "FETCH_SIZE").items() if "copyBuffer" in k]
    cw = [v for k, v in _counter_medians(copy_write_dir, "WRITE_SIZE").items() if "copyBuffer" in k]
    if not cf or not cw:
        raise SystemExit("no copy kernel in the calibration runs")
    fetch_scale = copy_bytes / (cf[0] * 1024.0)
    write_scale = copy_bytes / (cw[0] * 1024.0)
    fetch = _counter_medians(fetch_dir, "FETCH_SIZE")
    write = _counter_medians(write_dir, "WRITE_SIZE")
    alg = kernel_bytes(n_tok, chunk_heads(lengths, w.Hv), N, w.Hq, w.Hv, beta_bytes, w.has_h0)
    alg["kda_fused_kernel"] = algorithmic_bytes(n_tok, N, w.Hq, w.Hv, beta_bytes, w.has_h0)
    per, hbm = {}, {}
    for short in ("kda_intra_kernel", "kda_scan_kernel", "kda_fused_kernel"):
        fk = [k for k in fetch if short in k]
        wk = [k for k in write if short in k]
        if not fk or not wk:
            continue
        rd, wr = fetch[fk[0]] * 1024.0 * fetch_scale, write[wk[0]] * 1024.0 * write_scale
        per[short] = {"fetch_size_kib_per_dispatch": fetch[fk[0]], "write_size_kib_per_dispatch": write[wk[0]],
                      "hbm_read_bytes": int(rd), "hbm_write_bytes": int(wr), "hbm_bytes": int(rd + wr),
                      "algorithmic_bytes": alg.get(short)}
        hbm[short] = int(rd + wr)
    rec = {"workload": workload, "kernel_source_sha256": kernel_sha(),
           "copy_calibration": {"bytes": copy_bytes, "fetch_size_kib": cf[0], "write_size_kib": cw[0],
                                "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
           "per_kernel": per, "hbm_bytes_per_launch": hbm,
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o kda -- python3 bench.py "
               f"--workload {workload} --steps 3 --warmup 1 --no-cpu-baseline",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o kda -- python3 bench.py "
               f"--workload {workload} --steps 3 --warmup 1 --no-cpu-baseline",
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {copy_fetch_dir} -o copy -- python3 bench.py "
               "--calibrate-copy",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {copy_write_dir} -o copy -- python3 bench.py "
               "--calibrate-copy",
               f"python3 bench.py --workload {workload} --write-traffic {fetch_dir} {write_dir} "
               f"{copy_fetch_dir} {copy_write_dir}"]}
    path = os.path.join(ROOT, "profiles", f"traffic_kda_fwd_{workload}.json")
    json.dump(rec, open(path, "w"), indent=1)
    print(json.dumps(rec["hbm_bytes_per_launch"]))


def decode_bytes(N, Hq, Hv, beta_bytes, d=128):
    """Algorithmic bytes of one decode step: the state read and written once, the
    token's q, k (per q/k head), v, g, beta and o (per value head)."""
    return N * Hv * (2 * d * d * 4 + d * (2 + 4 + 2) + beta_bytes) + N * Hq * d * 2 * 2


def bench_decode(args):
    """kda_decode on a batch of N single tokens (Hq = Hv = 64, fp32 beta, fp32
    state updated in place): HIP events around each launch on its stream."""
    import torch
    from gated_delta_rule_35_amd import kda_decode
    from gated_delta_rule_35_amd.inputs import make_inputs
    if args.gpus != 1:
        print("bench.py measures one GPU only", file=sys.stderr, flush=True)
        sys.exit(2)
    N, H = args.decode, 64
    log(f"generating decode inputs: N={N} sequences x {H} heads")
    x = make_inputs(N, 1, H, H, torch.float32, h0=True, seed=0)
    dev = torch.device("cuda:0")
    s = {k: x[k][:, 0].contiguous().to(dev) for k in ("q", "k", "v", "g", "beta")}
    state = x["h0"].to(dev)
    out = torch.empty_like(s["v"])
    scale = 128 ** -0.5

    def one():
        kda_decode(s["q"], s["k"], s["v"], s["g"], s["beta"], scale, state, out=out)

    per_launch = args.graph if args.graph > 0 else 1
    if args.graph > 0:
        # K steps (the state updated in place each time) captured once into a HIP
        # graph; a timed launch replays all K
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.graph):
                one()
        launch = graph.replay
        log(f"decode: {args.graph} steps per graph replay")
    else:
        launch = one
    stream = torch.cuda.current_stream(dev)
    settle(launch)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        launch()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / per_launch
    ms = [e[0].elapsed_time(e[1]) / per_launch for e in ev]
    t = sum(ms) / len(ms) / 1e3
    nbytes = decode_bytes(N, H, H, 4)
    gbs = nbytes / t / 1e9
    log(f"decode N={N}: kernel avg {t * 1e3:.4f} ms (min {min(ms):.4f}), {gbs:.0f} GB/s")
    rec = {"metric": "KDA decode step tokens/s (one token per sequence, H=64, d=128, fp32 state)",
           "value": round(N / t, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"decode_n{N}_h{H}", "N_sequences": N, "Hq": H, "Hv": H, "dk": 128, "dv": 128,
                      "beta_dtype": "fp32", "state": "fp32, updated in place", "steps_per_graph": args.graph or None},
           "kernel_ms_avg": round(t * 1e3, 5), "algorithmic_bytes_per_step": nbytes,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "scope": ("kda_decode_kernel: algorithmic bytes over its average duration" if not args.graph else
                                  f"kda_decode_kernel: algorithmic bytes over the time per step of a {args.graph}-step "
                                  "HIP graph replay")},
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


FP32_MFMA_PEAK_TFLOPS = 157.3   # dense v_mfma_f32 (fp32 operands) on MI355X


def bwd_macs_per_chunk(C=64, d=128):
    """Multiply-adds of the chunk-form backward per (64-token chunk, value head),
    each product of the equations counted once: the operands (Aqk, Abar, the
    inverse), the forward walk (Z, v_new, h'), the backward walk (dv_new, dZ, dh)
    and the chunk-parallel gradients (d(qg), d(kg), d(kh), dAqk, dTb, the inverse's
    gradient and the four pairwise sums per channel)."""
    tri = C * (C + 1) // 2
    prep = 2 * tri * d + C * (C - 1) * (C + 1) // 6
    fwd = C * d * d + tri * d + d * C * d
    bwd = (tri * d + C * d * d) + tri * d + 2 * C * d * d
    grad = 3 * C * d * d + (tri + C * C) * d + 2 * C ** 3 + 4 * tri * d
    return prep + fwd + bwd + grad


def bench_bwd(args):
    """kda_bwd on --workload (fixed-length rows, or packed sequences with
    cu_seqlens): HIP events around each call on its stream, with a caller
    workspace so no allocation is timed."""
    import torch
    from gated_delta_rule_35_amd import kda_bwd, kda_bwd_workspace_size
    from gated_delta_rule_35_amd.inputs import WORKLOADS, workload_inputs
    if args.gpus != 1:
        print("bench.py measures one GPU only", file=sys.stderr, flush=True)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    log(f"generating inputs for {args.workload}")
    x, cu = workload_inputs(w)
    B, T = x["q"].shape[0], x["q"].shape[1]
    lens = [T] * B if cu is None else [int(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]
    gen = torch.Generator("cpu").manual_seed(1)
    do = torch.randn(B, T, w.Hv, 128, generator=gen).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    do_d = do.to(dev)
    cu_d = None if cu is None else cu.to(dev)
    ws = torch.empty(kda_bwd_workspace_size(B * T, len(lens), w.Hq, w.Hv), dtype=torch.uint8, device=dev)
    grads = None

    def one():
        nonlocal grads
        grads = kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, do_d, initial_state=d["h0"],
                        grads=grads, workspace=ws, cu_seqlens=cu_d)

    stream = torch.cuda.current_stream(dev)
    settle(one)
    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        one()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    t = sum(ms) / len(ms) / 1e3
    n_tok = sum(lens)
    units = sum((n + 63) // 64 for n in lens) * w.Hv
    flops = 2 * bwd_macs_per_chunk() * units
    tf = flops / t / 1e12
    log(f"backward {args.workload}: call avg {t * 1e3:.3f} ms (min {min(ms):.3f}), {n_tok / t / 1e6:.2f} M tok/s, "
        f"{tf:.1f} TFLOP/s algorithmic")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import grad as og
        heads = list(range(min(2, w.Hv)))
        group = w.Hv // w.Hq
        f64 = lambda a: a.float().numpy().astype("float64")  # noqa: E731
        sub = [f64(x["q"][:, :, [h // group for h in heads]]), f64(x["k"][:, :, [h // group for h in heads]]),
               f64(x["v"][:, :, heads]), f64(x["g"][:, :, heads]), f64(x["beta"][:, :, heads])]
        h0 = f64(x["h0"][:, heads]) if x["h0"] is not None else None
        dos = f64(do[:, :, heads])
        reps, c0 = 0, time.perf_counter()
        while True:
            if cu is None:
                og.chunked_grads(*sub, w.scale, h0, dos, None, chunk=64)
            else:   # each packed sequence on its own
                for n in range(len(lens)):
                    a, z = int(cu[n]), int(cu[n + 1])
                    og.chunked_grads(*[t[:, a:z] for t in sub], w.scale, None if h0 is None else h0[n:n + 1],
                                     dos[:, a:z], None, chunk=64)
            reps += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - c0
        tok_s = n_tok * len(heads) / w.Hv * reps / el
        cpu = {"value": round(tok_s, 1), "unit": "tokens/s", "cores": torch.get_num_threads(), "kind": "oracle",
               "sample": f"fp64 chunk-form gradients (numpy) on value heads {heads} of the full batch, "
                         f"{reps} run(s) in {el:.1f} s, scaled to all {w.Hv} heads"}
        log(f"cpu oracle: {tok_s:.1f} tok/s")
    rec = {"metric": "KDA backward tokens/s (gradients of q, k, v, g, beta)", "value": round(n_tok / t, 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": args.workload, "B": B, "T": T, "Hq": w.Hq, "Hv": w.Hv, "dk": 128, "dv": 128,
                      "sequences": len(lens), "packed": cu is not None},
           "call_ms_avg": round(t * 1e3, 4), "algorithmic_flops_per_call": flops,
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                        "scope": "the whole kda_bwd call (five kernels): algorithmic fp32 flops over its duration, "
                                 "against the fp32 MFMA peak (the contractions run on v_mfma_f32_16x16x4f32)"},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def oracle_cpu_baseline(x, cu, w, N, n_tok, scale, seconds, heads):
    """The fp64 oracle (token recurrence) on value heads 0 .. heads-1 of the
    workload, run repeatedly for at least `seconds`; tokens/s scaled to all heads."""
    import torch
    import oracle
    hs = list(range(min(heads, w.Hv)))
    group = w.Hv // w.Hq
    qk = [h // group for h in hs]
    sub = dict(q=x["q"][:, :, qk], k=x["k"][:, :, qk], v=x["v"][:, :, hs], g=x["g"][:, :, hs],
               beta=x["beta"][:, :, hs], h0=x["h0"][:, hs] if x["h0"] is not None else None)
    # widen to fp64 before the clock starts: the conversion is marshalling, not the oracle
    sub = {k: (v.to(torch.float64).contiguous().numpy() if v is not None else None) for k, v in sub.items()}
    log(f"cpu baseline: oracle on {len(hs)} of {w.Hv} value heads, all {N} sequences, repeated for >= {seconds:.0f} s")
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrence(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale, cu_seqlens=cu, h0=sub["h0"])
        reps += 1
        cpu_s = time.perf_counter() - t0
        if cpu_s >= seconds:
            break
    cpu_tok = n_tok * len(hs) / w.Hv * reps / cpu_s
    cpu = {"value": round(cpu_tok, 1), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
           "sample": f"fp64 token recurrence over value heads 0..{len(hs) - 1} of {w.Hv} (all {N} sequences, "
                     f"{n_tok} tokens each head), {reps} runs in {cpu_s:.1f} s, scaled to {w.Hv} heads"}
    log(f"cpu baseline {cpu_tok:.1f} tokens/s on {cpu['cores']} threads ({reps} runs, {cpu_s:.1f} s)")
    # the same oracle on one OpenMP thread (value head 0 only, for about a quarter
    # of the time), and the host CPU's model name
    one = one_thread_oracle(sub, cu, w, N, n_tok, scale, max(seconds / 4, 2.0))
    if one is not None:
        cpu["one_thread"] = one
    cpu["cpu_model"] = cpu_model_name()
    return cpu


def cpu_model_name():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def one_thread_oracle(sub, cu, w, N, n_tok, scale, seconds):
    """tokens/s of the oracle on one OpenMP thread over value head 0 (scaled to all
    heads), or None when the OpenMP runtime cannot be reached."""
    import ctypes
    import numpy as np
    import oracle
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    before = oracle.threads()
    # value head 0 and its q/k head (index 0 of each head axis)
    one = {k: (np.ascontiguousarray(v[:, :, 0:1]) if v is not None else None) for k, v in sub.items() if k != "h0"}
    one["h0"] = np.ascontiguousarray(sub["h0"][:, 0:1]) if sub.get("h0") is not None else None
    gomp.omp_set_num_threads(1)
    try:
        if oracle.threads() != 1:
            return None
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.recurrence(one["q"], one["k"], one["v"], one["g"], one["beta"], scale, cu_seqlens=cu,
                              h0=one["h0"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        gomp.omp_set_num_threads(before)
    tok = n_tok / w.Hv * reps / el
    log(f"cpu baseline, one thread: {tok:.1f} tokens/s ({reps} runs of value head 0, {el:.1f} s)")
    return {"value": round(tok, 1), "unit": "tokens/s", "cores": 1,
            "sample": f"value head 0 of {w.Hv} (all {N} sequences), {reps} runs in {el:.1f} s, scaled to {w.Hv} heads"}


def bench_cp(args):
    """kda_fwd_cp (the segmented forward) on a fixed-length workload with few heads:
    HIP events around each whole call (intra kernel, two scan launches and the
    composition) on its stream, and kda_fwd on the same inputs for comparison."""
    import torch
    from gated_delta_rule_35_amd import (kda_fwd, kda_fwd_cp, kda_fwd_cp_packed_workspace_size, kda_fwd_cp_plan,
                                         kda_fwd_cp_workspace_size, kda_fwd_workspace_size)
    from gated_delta_rule_35_amd.inputs import WORKLOADS, workload_inputs
    if args.gpus != 1:
        print("bench.py measures one GPU only", file=sys.stderr, flush=True)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    log(f"generating inputs for {w.name}")
    x, cu = workload_inputs(w)
    B, T = x["q"].shape[0], x["q"].shape[1]
    n_tok = B * T
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    cu_d = cu.to(dev) if cu is not None else None
    N = B if cu is None else len(cu) - 1
    out = torch.empty_like(d["v"])
    hT = torch.empty((N, w.Hv, 128, 128), dtype=torch.float32, device=dev)
    if args.cp > 0:
        L, L0 = args.cp, (args.cp_first or args.cp)
    elif cu is not None:
        print("packed workloads: pass --cp N (and --cp-first N0); the plan needs the lengths", file=sys.stderr,
              flush=True)
        sys.exit(2)
    else:
        pl = kda_fwd_cp_plan(B, T, w.Hv)
        if pl is None:
            print(f"{w.name}: the segment plan picks the ordinary path (B * Hv fills the GPU or T is short); "
                  "pass --cp N to force N chunks per segment", file=sys.stderr, flush=True)
            sys.exit(2)
        L, L0 = pl
    lens = [T] * B if cu is None else [int(cu[i + 1] - cu[i]) for i in range(N)]
    P = max(1 if (n + 63) // 64 <= L0 else 1 + -(-((n + 63) // 64 - L0) // L) for n in lens)
    if cu is None:
        ws_cp = torch.empty(kda_fwd_cp_workspace_size(B, T, w.Hv, L, L0), dtype=torch.uint8, device=dev)
    else:
        ws_cp = torch.empty(kda_fwd_cp_packed_workspace_size(n_tok, N, w.Hv, L, L0), dtype=torch.uint8, device=dev)
    ws = torch.empty(kda_fwd_workspace_size(B * T, N, w.Hv), dtype=torch.uint8, device=dev)
    a = (d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale)
    stream = torch.cuda.current_stream(dev)

    def timed(call):
        settle(call)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for e in ev:
            e[0].record(stream)
            call()
            e[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        return wall / args.steps * 1e3, sum(ms) / len(ms)

    log(f"kda_fwd_cp: first segment {L0} chunks, then {L} per segment, up to {P} segments per sequence; "
        f"{args.steps} steps")
    step_ms, call_ms = timed(lambda: kda_fwd_cp(*a, L, L0, initial_state=d["h0"], out=out, final_state=hT,
                                                workspace=ws_cp, cu_seqlens=cu_d))
    log(f"kda_fwd (ordinary): {args.steps} steps")
    plain_step_ms, plain_call_ms = timed(lambda: kda_fwd(*a, cu_seqlens=cu_d, initial_state=d["h0"], out=out,
                                                         final_state=hT, workspace=ws))
    log(f"segmented {call_ms:.4f} ms/call, ordinary {plain_call_ms:.4f} ms/call ({plain_call_ms / call_ms:.2f}x)")
    beta_bytes = 4 if w.beta_dtype == torch.float32 else 2
    nbytes = algorithmic_bytes(n_tok, N, w.Hq, w.Hv, beta_bytes, w.has_h0)
    gbs = nbytes / (call_ms / 1e3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_cpu_baseline(x, cu, w, N, n_tok, w.scale, args.cpu_seconds, args.cpu_heads)
    rec = {"metric": "KDA fwd tokens/s, segmented scan (context parallelism inside one GPU); ms/call",
           "value": round(n_tok / (step_ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": w.name, "B": B, "T": T, "N_sequences": N, "Hq": w.Hq, "Hv": w.Hv, "dk": 128,
                      "dv": 128, "chunk": 64, "segment_chunks": L, "first_segment_chunks": L0,
                      "max_segments_per_sequence": P, "packed": cu is not None,
                      "beta_dtype": "fp32" if beta_bytes == 4 else "bf16", "initial_state": bool(w.has_h0)},
           "call_ms_avg": round(call_ms, 5), "ordinary_kda_fwd_ms_avg": round(plain_call_ms, 5),
           "speedup_vs_ordinary": round(plain_call_ms / call_ms, 3),
           "algorithmic_bytes_per_step": nbytes,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "scope": "whole segmented forward: the forward's algorithmic bytes over the average duration "
                                 "of a call (all its launches)"},
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha_b2_h64_t8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--form", choices=("auto", "two-pass", "fused"), default="auto",
                    help="forward form of the timed step (auto: the faster of the two in a short probe)")
    ap.add_argument("--cpu-heads", type=int, default=64, help="value heads in the oracle's timing sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the oracle's sample is run repeatedly until this much wall time has passed")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="instead of the forward, time kda_decode: one step for N sequences x 64 heads")
    ap.add_argument("--graph", type=int, default=0, metavar="K",
                    help="with --decode: capture K steps in one HIP graph and time its replays (per step)")
    ap.add_argument("--cp", type=int, default=-1, metavar="L",
                    help="instead of the headline, time kda_fwd_cp on --workload with L chunks per segment "
                         "(0: the library's suggestion) against kda_fwd")
    ap.add_argument("--cp-first", type=int, default=0, metavar="L0",
                    help="with --cp L: chunks of the first segment (default L)")
    ap.add_argument("--bwd", action="store_true",
                    help="instead of the forward, time the backward kda_bwd on --workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="instead of the benchmark, run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU: turn four rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of this "
                         "benchmark on --workload, then of --calibrate-copy) into profiles/traffic_kda_fwd_<workload>.json")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic)
        return
    if args.calibrate_copy:
        import torch
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4, "launches": 3}))
        return
    if args.decode:
        bench_decode(args)
        return
    if args.bwd:
        bench_bwd(args)
        return
    if args.cp >= 0:
        bench_cp(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: each GPU would run its own shard of sequences or heads independently.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    from gated_delta_rule_35_amd import kda_fwd_intra, kda_fwd_scan, kda_fwd_workspace_size, kda_dv_slices
    from gated_delta_rule_35_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    log(f"generating inputs for {w.name}")
    x, cu = workload_inputs(w)
    B, T = x["q"].shape[0], x["q"].shape[1]
    lengths = [int(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)] if cu is not None else [T] * B
    N = len(lengths)
    n_tok = sum(lengths)
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    cu_d = cu.to(dev) if cu is not None else None
    out = torch.empty_like(d["v"])
    hT = torch.empty((N, w.Hv, 128, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kda_fwd_workspace_size(B * T, N, w.Hv), dtype=torch.uint8, device=dev)
    scale = w.scale
    stream = torch.cuda.current_stream(dev)

    from gated_delta_rule_35_amd import kda_fwd, kda_fwd_fused, kda_fwd_ws

    def step_two_pass():
        # the whole forward with a caller-owned workspace (kda_fwd_ws): the two
        # kernels and nothing else
        kda_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, cu_seqlens=cu_d, initial_state=d["h0"],
                   out=out, final_state=hT, workspace=ws)

    def step_fused():
        # the whole forward in one launch of kda_fused_kernel (nothing allocated)
        kda_fwd_fused(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, cu_seqlens=cu_d, initial_state=d["h0"],
                      out=out, final_state=hT)

    forms = {"two-pass": step_two_pass, "fused": step_fused}
    entry = {"two-pass": "kda_fwd_ws", "fused": "kda_fwd_fused"}

    def events_list(call, n):
        # n calls, HIP events on the launch stream around each call: ms per call
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for e in ev:
            e[0].record(stream)
            call()
            e[1].record(stream)
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in ev]

    def events_ms(call, n):
        return sum(events_list(call, n)) / n

    probe = None
    if args.form == "auto":
        # each form in its own steady state: a settle phase of its own, then 20
        # calls (the first calls of one form after the other run slower)
        probe = {}
        for k, f in forms.items():
            settle(f)
            probe[k] = round(events_ms(f, 20), 5)
        form = min(probe, key=probe.get)
        log(f"form probe (ms per call, 20 calls each after its own settle phase): {probe} -> {form}")
    else:
        form = args.form
    step = forms[form]
    settle(step)
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps of {entry[form]}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    t_enq = (time.perf_counter() - t0) / args.steps   # host time to enqueue a call
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    tokens_per_s = n_tok / (ms_per_step / 1e3)
    log(f"{ms_per_step:.4f} ms/step (wall), {tokens_per_s / 1e6:.2f} M tokens/s")
    # the same form call by call: 50 calls, each between HIP events
    per_call = sorted(events_list(step, 50))
    call_events = {"calls": 50, "median_ms": round((per_call[24] + per_call[25]) / 2, 5), "min_ms": round(per_call[0], 5),
                   "mean_ms": round(sum(per_call) / 50, 5), "max_ms": round(per_call[-1], 5)}
    log(f"{entry[form]} per call (HIP events, 50 calls): median {call_events['median_ms']:.4f} ms, "
        f"min {call_events['min_ms']:.4f} ms")

    # Per-kernel durations, in passes of their own so that no timing event sits inside
    # the timed steps: args.steps launches of each kernel back to back (the scan reads
    # the records the last intra launch wrote), HIP events on the launch stream around
    # each batch.
    def batch_ms(launch):
        launch()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(args.steps):
            launch()
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / args.steps

    t_intra = batch_ms(lambda: kda_fwd_intra(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, ws, cu_seqlens=cu_d,
                                              initial_state=d["h0"], out=out, final_state=hT)) / 1e3
    t_scan = batch_ms(lambda: kda_fwd_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, ws, cu_seqlens=cu_d,
                                            initial_state=d["h0"], out=out, final_state=hT)) / 1e3
    t_kern = t_intra + t_scan
    log(f"intra kernel avg {t_intra * 1e3:.4f} ms, scan kernel avg {t_scan * 1e3:.4f} ms")

    # The eleven-argument kda_fwd (the single-pass kernel on fixed-length batches
    # that fill the device; else the two-pass kernels on a workspace from
    # hipMallocAsync / hipFreeAsync on the stream inside the call), timed like the
    # steps above right after its own warm-up.
    def call11():
        kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, cu_seqlens=cu_d, initial_state=d["h0"],
                out=out, final_state=hT)
    settle(call11)
    for _ in range(args.warmup):
        call11()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call11()
    t_enq11 = (time.perf_counter() - t0) / args.steps
    torch.cuda.synchronize()
    t_call11 = (time.perf_counter() - t0) / args.steps
    log(f"kda_fwd (eleven arguments) {t_call11 * 1e3:.4f} ms per call (wall)")

    # The same step with the last-level cache flushed before each call: a 1 GiB
    # buffer (four times the 256 MB MALL) is read between the calls, outside the
    # events, so each call finds its inputs in HBM rather than in the cache the
    # previous call left them in.  The flush only reads, so it leaves no dirty
    # lines for the timed call to write back.  Workloads whose inputs fit in the
    # cache (T = 512, 1024) read faster without the flush.
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    flush_sum = torch.zeros((), dtype=torch.float32, device=dev)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evc:
        torch.sum(flush, 0, out=flush_sum)
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    cold = [e[0].elapsed_time(e[1]) for e in evc]
    t_cold = sum(cold) / len(cold) / 1e3
    del flush, flush_sum
    log(f"{entry[form]} after a cache flush: {t_cold * 1e3:.4f} ms per call (min {min(cold):.4f})")

    # kda_fwd_fused, the single-pass kernel (one launch of kda_fused_kernel): when
    # it is the step, the 50 calls between HIP events right after the timed steps;
    # else a settle phase of its own and then K calls between HIP events
    if form == "fused":
        t_fused = call_events["mean_ms"] / 1e3
    else:
        settle(step_fused)
        t_fused = events_ms(step_fused, args.steps) / 1e3
    log(f"kda_fwd_fused avg {t_fused * 1e3:.4f} ms per call")

    beta_bytes = 4 if w.beta_dtype == torch.float32 else 2
    nbytes = algorithmic_bytes(n_tok, N, w.Hq, w.Hv, beta_bytes, w.has_h0)
    n_ch = chunk_heads(lengths, w.Hv)
    flops = 2 * MAC_PER_CHUNK_HEAD * n_ch
    kbytes = kernel_bytes(n_tok, n_ch, N, w.Hq, w.Hv, beta_bytes, w.has_h0)
    traffic = load_traffic(w.name)
    kt = {"kda_intra_kernel": t_intra, "kda_scan_kernel": t_scan}
    kernels = {}
    for name in KERNELS:
        a = kbytes[name] / kt[name] / 1e9
        kernels[name] = {"ms_avg": round(kt[name] * 1e3, 5), "algorithmic_bytes": kbytes[name],
                         "achieved": round(a, 1), "frac": round(a / HBM_PEAK_GBS, 4),
                         "traffic": traffic.get(name) if traffic else None}
    two_gbs = nbytes / t_kern / 1e9
    two_pass = {"ms_avg": round(t_kern * 1e3, 5), "achieved": round(two_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(two_gbs / HBM_PEAK_GBS, 4),
                "traffic": sum(traffic[k] for k in KERNELS) if traffic else None,
                "scope": "kda_fwd_ws: algorithmic bytes of the forward over the summed average durations of "
                         "kda_intra_kernel and kda_scan_kernel",
                "kernels": kernels}
    fused_gbs = nbytes / t_fused / 1e9
    fused = {"ms_avg": round(t_fused * 1e3, 5), "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
             "traffic": traffic.get("kda_fused_kernel") if traffic else None,
             "scope": "kda_fwd_fused: algorithmic bytes of the forward over the average duration of "
                      "kda_fused_kernel"}
    # the roofline of the step's own form; the other form's figures stay beside it
    t_step_kern = t_fused if form == "fused" else t_kern
    roofline = {"bound": "hbm", **{k: v for k, v in (fused if form == "fused" else two_pass).items()
                                   if k in ("achieved", "peak", "unit", "frac", "traffic", "scope")}}
    roofline["kernel"] = "kda_fused_kernel" if form == "fused" else "kda_intra_kernel + kda_scan_kernel"
    roofline["kernel_ms_avg"] = round(t_step_kern * 1e3, 5)
    mfma = {"achieved": round(flops / t_step_kern / 1e12, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(flops / t_step_kern / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "algorithmic_flop_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_cpu_baseline(x, cu, w, N, n_tok, scale, args.cpu_seconds, args.cpu_heads)

    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(tokens_per_s / (n_tok / (PAGES_MS[w.name] / 1e3)), 4) if w.name in PAGES_MS else None),
        "vs_baseline_ref": (f"pages' CuTeDSL forward {PAGES_MS[w.name]} ms for this workload on NVIDIA SM100/SM103 "
                            f"({n_tok / (PAGES_MS[w.name] / 1e3):.0f} tokens/s); another machine, context only"
                            if w.name in PAGES_MS else None),
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "N_sequences": N, "tokens": n_tok, "Hq": w.Hq, "Hv": w.Hv,
                   "dk": 128, "dv": 128, "chunk": 64,
                   "beta_dtype": "fp32" if beta_bytes == 4 else "bf16", "initial_state": bool(w.has_h0),
                   "dv_slices": kda_dv_slices(N, w.Hv), "mfma_operands": "f16", "accumulate": "f32",
                   "io": "bf16 q/k/v/o, f32 g/state"},
        "step": ("kda_fwd_fused: the whole forward in one launch of kda_fused_kernel" if form == "fused" else
                 "kda_fwd_ws: the whole forward on a caller-owned workspace (the two kernels)"),
        "form": form,
        "form_probe_ms": probe,
        "settle_s": SETTLE_S,
        "kernel_ms_avg": round(t_step_kern * 1e3, 5),
        "call_events": call_events,
        "kda_fwd_call_ms_avg": round(t_call11 * 1e3, 5),
        "host_enqueue_ms": {entry[form]: round(t_enq * 1e3, 4), "kda_fwd": round(t_enq11 * 1e3, 4),
                            "scope": "host time from the first call of the timed loop to the return of the last, "
                                     "before the synchronisation, per call (argument checks, descriptor "
                                     "marshalling, launches; kda_fwd also its stream-ordered allocation)"},
        "cold_cache": {"ms_avg": round(t_cold * 1e3, 5), "tokens_per_s": round(n_tok / t_cold, 1),
                       "scope": f"{entry[form]} with a 1 GiB buffer read before each call (outside the HIP "
                                "events), so no input is left in the 256 MB last-level cache"},
        "algorithmic_bytes_per_step": nbytes,
        "roofline": roofline,
        "two_pass": two_pass,
        "fused": fused,
        "mfma": mfma,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
