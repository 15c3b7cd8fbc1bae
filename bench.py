#!/usr/bin/env python3
"""Throughput of the MI355X KDA forward on one GPU; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one kda_fwd call over the whole batch of the workload (default: B=2,
H=64, T=8192, dk=dv=128, chunk 64, fp32 beta, initial state ~ 0.1 N(0,1)), with
all inputs and outputs already resident in HBM.  The K timed steps are bracketed
by device synchronisation; every launch is also bracketed by HIP events on the
stream it runs on, which gives the kernel's average duration for the roofline.

Roofline (HBM-bound kernel): algorithmic bytes per launch = q, k, v, g, beta read
once, o written once, the initial state read (if any) and the final state
written; achieved = bytes / average launch duration, against 8 TB/s.  The MFMA
side uses the algorithmic flop count of the chunked method (4,512,416 MAC per
full 64-token chunk and value head).

cpu_baseline: the fp64 CPU oracle (token recurrence, OpenMP over sequence x head)
timed on a bounded sample of the same workload, scaled to tokens/s of the full
head count.
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
KERNEL_SOURCE = os.path.join(ROOT, "gated_delta_rule_35_amd", "csrc", "kda_fwd_kernel.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(n_tok, N, Hq, Hv, beta_bytes, has_h0, d=128):
    per_tok = Hq * d * 2 * 2 + Hv * d * 2 * 2 + Hv * d * 4 + Hv * beta_bytes
    states = N * Hv * d * d * 4 * (2 if has_h0 else 1)
    return n_tok * per_tok + states


def chunk_heads(lengths, Hv, C=64):
    return sum((L + C - 1) // C for L in lengths) * Hv


def kernel_sha():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()


def load_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_kda_fwd_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha_b2_h64_t8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=64, help="value heads in the oracle's timing sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="instead of the benchmark, run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: each GPU would run its own shard of sequences or heads independently.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    from gated_delta_rule_35_amd import kda_fwd, kda_dv_slices
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
    scale = w.scale

    def step():
        kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, cu_seqlens=cu_d, initial_state=d["h0"],
                out=out, final_state=hT)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    tokens_per_s = n_tok / (ms_per_step / 1e3)
    log(f"{ms_per_step:.4f} ms/step (wall), kernel avg {avg_launch_s * 1e3:.4f} ms, "
        f"min {min(launch_ms):.4f} ms, {tokens_per_s / 1e6:.2f} M tokens/s")

    beta_bytes = 4 if w.beta_dtype == torch.float32 else 2
    nbytes = algorithmic_bytes(n_tok, N, w.Hq, w.Hv, beta_bytes, w.has_h0)
    flops = 2 * MAC_PER_CHUNK_HEAD * chunk_heads(lengths, w.Hv)
    achieved_gbs = nbytes / avg_launch_s / 1e9
    traffic = load_traffic(w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    mfma = {"achieved": round(flops / avg_launch_s / 1e12, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(flops / avg_launch_s / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "algorithmic_flop_per_launch": flops}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        hs = list(range(min(args.cpu_heads, w.Hv)))
        group = w.Hv // w.Hq
        qk = [h // group for h in hs]
        sub = dict(q=x["q"][:, :, qk], k=x["k"][:, :, qk], v=x["v"][:, :, hs], g=x["g"][:, :, hs],
                   beta=x["beta"][:, :, hs], h0=x["h0"][:, hs] if x["h0"] is not None else None)
        # widen to fp64 before the clock starts: the conversion is marshalling, not the oracle
        sub = {k: (v.to(torch.float64).contiguous().numpy() if v is not None else None) for k, v in sub.items()}
        log(f"cpu baseline: oracle on {len(hs)} of {w.Hv} value heads, all {N} sequences")
        t0 = time.perf_counter()
        oracle.recurrence(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], scale, cu_seqlens=cu, h0=sub["h0"])
        cpu_s = time.perf_counter() - t0
        cpu_tok = n_tok * len(hs) / w.Hv / cpu_s
        cpu = {"value": round(cpu_tok, 1), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"fp64 token recurrence over value heads 0..{len(hs) - 1} of {w.Hv} (all {N} sequences, "
                         f"{n_tok} tokens each head) in {cpu_s:.1f} s, scaled to {w.Hv} heads"}
        log(f"cpu baseline {cpu_tok:.1f} tokens/s on {cpu['cores']} threads ({cpu_s:.1f} s)")

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
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "N_sequences": N, "tokens": n_tok, "Hq": w.Hq, "Hv": w.Hv,
                   "dk": 128, "dv": 128, "chunk": 64,
                   "beta_dtype": "fp32" if beta_bytes == 4 else "bf16", "initial_state": bool(w.has_h0),
                   "dv_slices": kda_dv_slices(N, w.Hv), "mfma_operands": "f16", "accumulate": "f32",
                   "io": "bf16 q/k/v/o, f32 g/state"},
        "kernel_ms_avg": round(avg_launch_s * 1e3, 5),
        "kernel_ms_min": round(min(launch_ms), 5),
        "algorithmic_bytes_per_launch": nbytes,
        "roofline": roofline,
        "mfma": mfma,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
