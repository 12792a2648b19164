#!/usr/bin/env python3
"""Benchmark of the fused UNet attention path on one MI355X.

One step = the attention of one SD-1.5 transformer block at a 64x64 latent
(512x512 image, classifier-free-guidance batch 2): self-attention
B=2, H=8, Lq=Lk=4096, d=40 (streaming kernel) followed by cross-attention to
the 77-token text context, B=2, H=8, Lq=4096, Lk=77, d=40 (short-key kernel).
bf16 inputs and outputs (fp16 for the *_f16 step), fp32 accumulation;
inputs are seeded N(0,1) synthetic tensors resident in HBM before timing
starts.

Metric: attention TFLOP/s = 4*B*H*Lq*Lk*d summed over the step's calls,
divided by the step time.  The JSON line also carries the roofline fraction
of the dominant kernel (self-attention vs the 16-bit dense MFMA peak, per-launch
duration from HIP events recorded around each launch on its stream), the
cross-attention kernel's HBM fraction, and the CPU oracle timed on the host.

Input sets are rotated across more than 512 MB of buffers so that the
HBM-bound cross-attention kernel is not served from the 256 MB Infinity
Cache (a warm-cache figure for the same kernels is reported separately).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
       [--no-cpu-baseline] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import GN_WORKLOADS, WORKLOADS, make_gn_inputs, make_inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 (and fp16) MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
ROTATE_BYTES = 640 << 20       # > 2x the 256 MB Infinity Cache
METRIC = "attention TFLOP/s (4·B·H·Lq·Lk·d) and % of MI355X MFMA/HBM roofline"

# Step definitions: name -> list of (workload, entry point).
STEPS = {
    "sd15_64x64_block": [("2", "fwd"), ("3", "cross")],
    "sd15_64x64_block_f16": [("2h", "fwd"), ("3h", "cross")],
}
for _n in WORKLOADS:
    if _n != "1":
        # the cross entry takes contexts up to the LDS-resident cap (128)
        _w = WORKLOADS[_n]
        STEPS[f"workload_{_n}"] = [(_n, "cross" if _w.kind == "cross" and _w.Lk <= 128 else "fwd")]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "unet_attention_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(step_name: str, kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if the kernel sources have not changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{step_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    k = rec.get("kernels", {}).get(kernel_key)
    return None if k is None else float(k["hbm_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="sd15_64x64_block",
                    choices=sorted(STEPS) + sorted(f"gn_{n}" for n in GN_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path shards over "
              "(batch, head) with no communication, and no multi-GPU run is "
              "part of this build; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import unet_attention_amd as sd
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload.startswith("gn_"):
        bench_group_norm(args, args.workload[3:])
        return
    if args.copy_calibration:
        copy_calibration()
        return
    sd.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    calls = STEPS[args.workload]
    ws = [WORKLOADS[n] for n, _ in calls]
    inputs = [make_inputs(w) for w in ws]

    elt = ws[0].dtype  # "bf16" or "f16"; one element type per step
    assert all(w.dtype == elt for w in ws) and elt in ("bf16", "f16")
    tdt = torch.bfloat16 if elt == "bf16" else torch.float16
    dtype_code = sd.SDATTN_DTYPE_BF16 if elt == "bf16" else sd.SDATTN_DTYPE_F16

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    base = [tuple(dev16(b) for b in (x.q_bits, x.k_bits, x.v_bits)) for x in inputs]
    set_bytes = sum(2 * (q.numel() + k.numel() + v.numel() + q.numel()) for q, k, v in base)
    nsets = max(2, -(-ROTATE_BYTES // set_bytes))
    sets = []
    for s in range(nsets):
        one = []
        for (q, k, v), w in zip(base, ws):
            qq, kk, vv = (q, k, v) if s == 0 else (q.clone(), k.clone(), v.clone())
            out = torch.empty_like(qq)
            one.append((qq, kk, vv, out))
        sets.append(one)
    torch.cuda.synchronize()

    fns = {"fwd": sd.load().sdattn_fwd, "cross": sd.load().sdattn_cross_fwd}
    argv = []
    for s in range(nsets):
        row = []
        for (n, entry), w, (q, k, v, o) in zip(calls, ws, sets[s]):
            row.append((fns[entry], (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     w.B, w.H, w.Lq, w.Lk, w.d, w.scale,
                                     dtype_code, sh)))
        argv.append(row)

    def launch(fn, a):
        rc = fn(*a)
        if rc != sd.SDATTN_OK:
            raise sd.SdattnError(rc, "bench launch")

    # warmup
    for i in range(args.warmup):
        for fn, a in argv[i % nsets]:
            launch(fn, a)
    torch.cuda.synchronize()

    # timed region: one event on the launch stream before every call and one
    # after the last, so each call is timed between consecutive events (an
    # event pair around every call would add its own GPU time to the step)
    K = args.steps
    nc = len(calls)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K * nc + 1)]
    torch.cuda.synchronize()
    for i in range(K):
        for j, (fn, a) in enumerate(argv[i % nsets]):
            ev[i * nc + j].record(stream)
            launch(fn, a)
    ev[K * nc].record(stream)
    torch.cuda.synchronize()
    ms_step = ev[0].elapsed_time(ev[K * nc]) / K
    per_call_ms = [float(np.mean([ev[i * nc + j].elapsed_time(ev[i * nc + j + 1])
                                  for i in range(K)])) for j in range(nc)]

    # warm-cache figure: same kernels, one buffer set
    warm_ms = []
    for j, (fn, a) in enumerate(argv[0]):
        for _ in range(5):
            launch(fn, a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        n = 50
        e0.record(stream)
        for _ in range(n):
            launch(fn, a)
        e1.record(stream)
        torch.cuda.synchronize()
        warm_ms.append(e0.elapsed_time(e1) / n)

    step_flops = sum(w.flops for w in ws)
    value = step_flops / (ms_step * 1e-3) / 1e12

    kernels = []
    for (n, entry), w, t_ms, tw in zip(calls, ws, per_call_ms, warm_ms):
        t = t_ms * 1e-3
        kernels.append({
            "workload": n, "entry": f"sdattn_{entry}" if entry != "fwd" else "sdattn_fwd",
            "shape": f"B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} d{w.d}",
            "us_per_launch": round(t_ms * 1e3, 3),
            "tflops": round(w.flops / t / 1e12, 2),
            "gbs_alg": round(w.bytes_alg(2) / t / 1e9, 1),
            "mfma_frac": round(w.flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(w.bytes_alg(2) / t / 1e9 / PEAK_HBM_GBS, 4),
            "warm_cache_us": round(tw * 1e3, 3),
        })

    # dominant kernel = the call with the largest share of step time
    jd = int(np.argmax(per_call_ms))
    wd = ws[jd]
    mfma_bound = wd.flops / wd.bytes_alg(2) > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3
    td = per_call_ms[jd] * 1e-3
    traffic = load_traffic(args.workload, f"{calls[jd][0]}")
    if mfma_bound:
        ach = wd.flops / td / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic}
    else:
        ach = wd.bytes_alg(2) / td / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}
    roof["kernel"] = kernels[jd]["entry"] + " " + kernels[jd]["shape"]
    roof["flops_per_launch"] = wd.flops
    roof["alg_bytes_per_launch"] = wd.bytes_alg(2)
    roof["us_per_launch"] = kernels[jd]["us_per_launch"]

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(args, calls, ws, inputs, sets[0], step_flops)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": elt, "data": "synthetic",
        "config": {"workload": args.workload,
                   "calls": [f"{k['entry']} {k['shape']}" for k in kernels],
                   "io": f"{elt} in/out, fp32 accumulation",
                   "buffer_sets_rotated": nsets,
                   "rotated_bytes": nsets * set_bytes},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "parity_vs_oracle": parity,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(args, calls, ws, inputs, set0, step_flops):
    """Time the fp64 CPU oracle on the same step (test infrastructure only),
    and compare the benchmarked GPU output with it."""
    import oracle
    import torch
    threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
    orc = oracle.get()
    total = 0.0
    worst = {}
    for (n, _), w, x, (_, _, _, out) in zip(calls, ws, inputs, set0):
        q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (x.q, x.k, x.v))
        t0 = time.perf_counter()
        want = orc.attn(q, k, v, w.scale, nthreads=threads)
        total += time.perf_counter() - t0
        got = out.float().cpu().numpy().astype(np.float64)
        e = np.abs(got - want)
        worst[n] = {"max_abs": float(e.max()), "mean_abs": float(e.mean())}
    with open("/proc/cpuinfo") as f:
        model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "?")
    cpu = {"value": round(step_flops / total / 1e12, 6), "unit": "TFLOP/s",
           "cores": threads, "kind": "oracle",
           "sample": f"one full step ({' + '.join(w.name for w in ws)}), fp64, "
                     f"{total:.2f} s on {threads} threads of {model}"}
    return cpu, worst


def bench_group_norm(args, name):
    """GroupNorm (+ SiLU) of one UNet level: an HBM-bound kernel, measured in
    GB/s of algorithmic traffic (x read once, y written once, gamma/beta)."""
    import torch
    import unet_attention_amd as sd
    w = GN_WORKLOADS[name]
    x = make_gn_inputs(w)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    code = {"bf16": sd.SDATTN_DTYPE_BF16, "f16": sd.SDATTN_DTYPE_F16,
            "f32": sd.SDATTN_DTYPE_F32}[w.dtype]
    if w.dtype == "f32":
        x0 = torch.from_numpy(np.ascontiguousarray(x.x)).to(dev)
    else:
        x0 = torch.from_numpy(np.ascontiguousarray(x.x_bits).view(np.int16)).view(tdt).to(dev)
    g = torch.from_numpy(x.gamma).to(dev)
    b = torch.from_numpy(x.beta).to(dev)
    set_bytes = 2 * x0.numel() * x0.element_size()
    nsets = max(2, -(-ROTATE_BYTES // set_bytes))
    sets = [(x0 if s == 0 else x0.clone(), torch.empty_like(x0)) for s in range(nsets)]
    torch.cuda.synchronize()
    fn = sd.load().sdattn_group_norm

    def launch(xx, yy):
        rc = fn(xx.data_ptr(), g.data_ptr(), b.data_ptr(), yy.data_ptr(), w.N, w.C, w.HW, w.G,
                w.eps, int(w.silu), code, sh)
        if rc != sd.SDATTN_OK:
            raise sd.SdattnError(rc, "bench group norm")

    for i in range(args.warmup):
        launch(*sets[i % nsets])
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        launch(*sets[i % nsets])
        ev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    per_ms = float(np.mean([a.elapsed_time(c) for a, c in ev]))
    nbytes = w.bytes_alg()
    value = nbytes / (ms_step * 1e-3) / 1e9
    ach = nbytes / (per_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": load_traffic(args.workload, name),
            "kernel": f"sdattn_group_norm N{w.N} C{w.C} HW{w.HW} G{w.G}",
            "alg_bytes_per_launch": nbytes, "us_per_launch": round(per_ms * 1e3, 3)}
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        import oracle
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        t = time.perf_counter()
        want = oracle.group_norm(x.x, x.gamma, x.beta, w.G, w.eps, w.silu, nthreads=threads)
        el = time.perf_counter() - t
        got = sets[0][1].float().cpu().numpy().astype(np.float64)
        e = np.abs(got - want)
        parity = {name: {"max_abs": float(e.max()), "mean_abs": float(e.mean())}}
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                         "?")
        cpu = {"value": round(nbytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "sample": f"the whole workload {name}, fp64, {el:.3f} s on "
                                           f"{threads} threads of {model}"}
    line = {
        "metric": "GroupNorm+SiLU GB/s (x read once, y written once)", "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "shape": f"N{w.N} C{w.C} H{w.H} W{w.W} G{w.G}",
                   "silu": w.silu, "eps": w.eps, "buffer_sets_rotated": nsets,
                   "rotated_bytes": nsets * set_bytes},
        "roofline": roof, "cpu_baseline": cpu, "parity_vs_oracle": parity,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
