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
divided by the step time (K steps back to back between two HIP events on
the launch stream).  The JSON line also carries the roofline fraction of the
dominant kernel (self-attention vs the 16-bit dense MFMA peak; its per-launch
duration from HIP events around chunks of that call's launches alone, same
buffer rotation, on the same stream), the cross-attention kernel's HBM
fraction, and the CPU oracle timed on the host.

Input sets are rotated across more than 512 MB of buffers so that the
HBM-bound cross-attention kernel is not served from the 256 MB Infinity
Cache (a warm-cache figure for the same kernels is reported separately).

The line also carries the chip's attainable rates measured in the same run
(dense bf16 MFMA with and without softmax-like vector work beside it, device
copies of the step's size and of 1 GiB, LDS reads), the GPU clock and power
sampled while the step runs, and per-launch median and minimum times.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
       [--no-cpu-baseline] [--no-peaks] [--copy-calibration] [--suite]
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
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak microbenchmarks")
    ap.add_argument("--suite", action="store_true",
                    help="run every row of SUITE a few times (for profiler runs) and exit")
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


# Rows run by --suite (one process, so a profiler pass covers every row):
# each row is a step name; kernel launches happen in this order.
SUITE = ["sd15_64x64_block", "sd15_64x64_block_f16", "workload_4a", "workload_4b",
         "workload_4c", "workload_4d", "workload_5", "workload_6a", "workload_6b"]
SUITE_GN = ["gn64", "gn128"]


class Step:
    """Device buffers and C-ABI argument tuples for one step: input sets are
    rotated over more than ROTATE_BYTES so HBM-bound kernels read HBM."""

    def __init__(self, torch, sd, name, stream, rotate=True):
        self.name = name
        self.calls = STEPS[name]
        self.ws = [WORKLOADS[n] for n, _ in self.calls]
        self.inputs = [make_inputs(w) for w in self.ws]
        elt = self.ws[0].dtype  # one element type per step
        assert all(w.dtype == elt for w in self.ws) and elt in ("bf16", "f16")
        self.elt = elt
        tdt = torch.bfloat16 if elt == "bf16" else torch.float16
        code = sd.SDATTN_DTYPE_BF16 if elt == "bf16" else sd.SDATTN_DTYPE_F16
        dev = torch.device("cuda:0")

        def dev16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

        base = [tuple(dev16(b) for b in (x.q_bits, x.k_bits, x.v_bits)) for x in self.inputs]
        self.set_bytes = sum(2 * (q.numel() + k.numel() + v.numel() + q.numel())
                             for q, k, v in base)
        self.nsets = max(2, -(-ROTATE_BYTES // self.set_bytes)) if rotate else 1
        self.sets = []
        for s in range(self.nsets):
            self.sets.append([((q, k, v) if s == 0 else (q.clone(), k.clone(), v.clone()))
                              + (torch.empty_like(q),) for q, k, v in base])
        torch.cuda.synchronize()
        lib = sd.load()
        fns = {"fwd": lib.sdattn_fwd, "cross": lib.sdattn_cross_fwd}
        sh = stream.cuda_stream
        self.argv = [[(fns[entry], (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    w.B, w.H, w.Lq, w.Lk, w.d, w.scale, code, sh))
                      for (n, entry), w, (q, k, v, o) in zip(self.calls, self.ws, row)]
                     for row in self.sets]
        self._sd = sd

    def launch_set(self, i):
        for fn, a in self.argv[i % self.nsets]:
            rc = fn(*a)
            if rc != self._sd.SDATTN_OK:
                raise self._sd.SdattnError(rc, "bench launch")


def sample_clock(run_for, seconds=1.0):
    """GPU clock (MHz) and socket power (W) sampled every ~5 ms while
    run_for(seconds) keeps the GPU busy: amd-smi's GFX clock of the first
    XCD, and the current GFX clock of every XCD from its metrics table."""
    import threading
    try:
        import amdsmi
        import torch
        amdsmi.amdsmi_init()
        # amd-smi may list GPUs this process does not use: take the one whose
        # PCI address is torch's device 0
        pr = torch.cuda.get_device_properties(0)
        want = (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
        h, bdf = None, None
        for cand in amdsmi.amdsmi_get_processor_handles():
            b = amdsmi.amdsmi_get_gpu_device_bdf(cand)
            dom, bus, rest = b.split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                h, bdf = cand, b
                break
        if h is None:
            raise RuntimeError(f"no amd-smi device at PCI {want}")
    except Exception as e:  # no amd-smi or no match: report why
        run_for(seconds)
        return {"error": f"amdsmi unavailable: {e}"}
    clk, pw, xcd, stop = [], [], [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                clk.append(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"])
                pw.append(amdsmi.amdsmi_get_power_info(h)["current_socket_power"])
                m = amdsmi.amdsmi_get_gpu_metrics_info(h).get("current_gfxclks")
                if isinstance(m, (list, tuple)):
                    xcd.extend(x for x in m if isinstance(x, (int, float)) and 0 < x < 10000)
            except Exception:
                pass
            time.sleep(0.005)

    t = threading.Thread(target=poll)
    t.start()
    try:
        run_for(seconds)
    finally:
        stop.set()
        t.join()
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
    # drop the first and last tenth (ramp up / drain)
    k = len(clk) // 10
    c = [x for x in clk[k:len(clk) - k] if isinstance(x, (int, float))] or clk
    p_ = [x for x in pw[k:len(pw) - k] if isinstance(x, (int, float))] or pw
    num = lambda v: [x for x in v if isinstance(x, (int, float))]
    return {"gfx_mhz_median": float(np.median(num(c))) if num(c) else None,
            "gfx_mhz_min": float(np.min(num(c))) if num(c) else None,
            "xcd_gfx_mhz_median": float(np.median(xcd)) if xcd else None,
            "socket_w_median": float(np.median(num(p_))) if num(p_) else None,
            "samples": len(clk), "device_bdf": bdf,
            "source": "amdsmi: GFX clock of the first XCD; metrics table, every XCD"}


def attainable_peaks(torch, stream, copy_bytes):
    """The chip's attainable rates in this run (libsdattn_peak.so): dense bf16
    MFMA alone and with n exp2 + n add (the softmax's per-score vector work)
    or n FMA per matrix instruction; device copies of copy_bytes of traffic
    (rotated over > 512 MB, so from HBM) and of 1 GiB; LDS 16-byte reads."""
    import ctypes
    from unet_attention_amd import build as hb
    if not os.path.exists(hb.PEAK_LIB):
        return {"error": "libsdattn_peak.so not built"}
    lib = ctypes.CDLL(hb.PEAK_LIB)
    lib.peak_mfma.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                              ctypes.c_int, ctypes.c_void_p]
    lib.peak_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sh = stream.cuda_stream

    seq = []  # (label, launches, work per launch) in launch order, for profilers

    def timed(launch, reps, label, work):
        seq.append([label, reps + 1, work])
        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    nwg, iters = 512, 8000   # 2 waves per SIMD
    sink = torch.empty(nwg * 256, dtype=torch.float32, device="cuda")
    flops = nwg * 4 * iters * 4 * 2 * 32 * 32 * 16
    mf = {}
    for ne, nf in ((0, 0), (2, 0), (4, 0), (8, 0), (0, 4), (0, 8), (2, 4), (4, 4)):
        def go(ne=ne, nf=nf):
            rc = lib.peak_mfma(nwg, iters, ne, nf, sink.data_ptr(), sh)
            if rc:
                raise RuntimeError(f"peak_mfma failed ({rc})")
        mf[f"exp{ne}_fma{nf}"] = round(flops / timed(go, 3, f"mfma exp{ne}_fma{nf}", flops) / 1e12, 1)
    out["mfma_bf16_tflops"] = mf.pop("exp0_fma0")
    out["mfma_bf16_tflops_with_vector_work_per_mfma"] = mf
    # copies: copy_bytes of traffic (half read, half written), rotated
    half = (copy_bytes // 2) // 16 * 16
    nbuf = max(2, -(-ROTATE_BYTES // (2 * half)))
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(nbuf)]
    for a_, b_ in bufs:
        a_.fill_(1)
    ci = [0]

    def cp():
        a_, b_ = bufs[ci[0] % nbuf]
        ci[0] += 1
        rc = lib.peak_copy(a_.data_ptr(), b_.data_ptr(), half, 1024, sh)
        if rc:
            raise RuntimeError(f"peak_copy failed ({rc})")
    t_small = timed(cp, 4 * nbuf, f"copy {2 * half} bytes", 2 * half)
    out["copy"] = {f"{2 * half / 1e6:.2f}MB_us": round(t_small * 1e6, 2),
                   f"{2 * half / 1e6:.2f}MB_gbs": round(2 * half / t_small / 1e9, 1)}
    del bufs
    big = 1 << 30
    a_ = torch.empty(big, dtype=torch.uint8, device="cuda")
    b_ = torch.empty(big, dtype=torch.uint8, device="cuda")
    a_.fill_(1)
    t_big = timed(lambda: lib.peak_copy(a_.data_ptr(), b_.data_ptr(), big, 8192, sh), 5,
                  f"copy {2 * big} bytes", 2 * big)
    out["copy"]["1GiB_gbs"] = round(2 * big / t_big / 1e9, 1)
    del a_, b_
    lnwg, liters = 1024, 4000
    lsink = torch.empty(lnwg * 256, dtype=torch.float32, device="cuda")
    t_lds = timed(lambda: lib.peak_lds(lnwg, liters, lsink.data_ptr(), sh), 3,
                  "lds b128 reads", lnwg * 256 * liters * 8 * 16)
    out["lds_read_gbs"] = round(lnwg * 256 * liters * 8 * 16 / t_lds / 1e9, 1)
    out["method"] = ("HIP events around back-to-back launches; MFMA: 512 workgroups of 4 waves, "
                     "v_mfma_f32_32x32x16_bf16 on 4 accumulators per wave; copies with 16-byte "
                     "lanes")
    out["_sequence"] = seq
    return out


def load_kernel_profile(step_name: str):
    """Kernel-only durations (rocprofv3 averages) from the committed trace
    summary of this step, if the kernel sources have not changed since."""
    path = os.path.join(ROOT, "profiles", f"trace_{step_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("kernels")


def suite(args, torch, sd):
    """Every SUITE row (and the GroupNorm rows) a few times each, in a fixed
    order, for profiler passes: warmup launches, then args.steps launches."""
    stream = torch.cuda.current_stream()
    for name in SUITE:
        st = Step(torch, sd, name, stream, rotate=name != "workload_5")
        n = args.steps if name != "workload_5" else max(1, args.steps // 4)
        for i in range(args.warmup + n):
            st.launch_set(i)
        torch.cuda.synchronize()
        print(json.dumps({"suite_row": name, "launches_per_call": args.warmup + n,
                          "warmup": args.warmup,
                          "calls": [f"{e} {w.name}" for (_, e), w in zip(st.calls, st.ws)],
                          "kernel_source_sha": kernel_source_sha()}), flush=True)
        del st
        torch.cuda.empty_cache()
    for name in SUITE_GN:
        args.workload = f"gn_{name}"
        bench_group_norm(args, name, quiet=True)
        print(json.dumps({"suite_row": f"gn_{name}", "launches_per_call": args.warmup + args.steps,
                          "warmup": args.warmup, "calls": [f"group_norm {name}"],
                          "kernel_source_sha": kernel_source_sha()}), flush=True)
    # attainable-peak microbenchmarks (libsdattn_peak.so), copy sized like the
    # cross-attention call of the default step
    peaks = attainable_peaks(torch, stream, WORKLOADS["3"].bytes_alg(2))
    seq = peaks.pop("_sequence", [])
    print(json.dumps({"suite_row": "peaks", "sequence": seq, "event_timed": peaks}), flush=True)


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
    sd.load()
    if args.suite:
        suite(args, torch, sd)
        return
    if args.workload.startswith("gn_"):
        bench_group_norm(args, args.workload[3:])
        return
    if args.copy_calibration:
        copy_calibration()
        return
    # a stream of its own (default priority): launches on the legacy null
    # stream carry its implicit synchronisation
    stream = torch.cuda.Stream(device=torch.device("cuda:0"))
    st = Step(torch, sd, args.workload, stream)
    calls, ws, nsets = st.calls, st.ws, st.nsets

    for i in range(args.warmup):
        st.launch_set(i)
    torch.cuda.synchronize()

    # timed region: K steps back to back between two events on the launch
    # stream (an event recorded between calls costs the step a few
    # microseconds of GPU time, so none is)
    K = args.steps
    nc = len(calls)
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(stream)
    for i in range(K):
        st.launch_set(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    ms_step = e_start.elapsed_time(e_end) / K

    # per call: the same launches (same buffer rotation) of that call alone,
    # in chunks timed between two events each; a launch's time therefore
    # includes the gap to the next launch.  Mean over all chunks, median
    # and minimum over the chunk means.
    chunks = 10
    per_chunk = max(5, K // chunks)
    per_call = []
    for j in range(nc):
        for i in range(5):
            fn, a = st.argv[i % nsets][j]
            fn(*a)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(chunks + 1)]
        evs[0].record(stream)
        i = 0
        for c in range(chunks):
            for _ in range(per_chunk):
                fn, a = st.argv[i % nsets][j]
                rc = fn(*a)
                if rc != sd.SDATTN_OK:
                    raise sd.SdattnError(rc, "bench launch")
                i += 1
            evs[c + 1].record(stream)
        torch.cuda.synchronize()
        per_call.append(np.array([evs[c].elapsed_time(evs[c + 1]) / per_chunk
                                  for c in range(chunks)]))
    per_call_ms = [float(x.mean()) for x in per_call]

    # warm-cache figure: same kernels, one buffer set
    warm_ms = []
    for j, (fn, a) in enumerate(st.argv[0]):
        for _ in range(5):
            fn(*a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        n = 50
        e0.record(stream)
        for _ in range(n):
            fn(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        warm_ms.append(e0.elapsed_time(e1) / n)

    # clock and power while the step runs back to back
    def run_for(sec):
        n = max(1, int(sec / (ms_step * 1e-3)))
        for i in range(n):
            st.launch_set(i)
        torch.cuda.synchronize()
    clock = sample_clock(run_for)

    step_flops = sum(w.flops for w in ws)
    value = step_flops / (ms_step * 1e-3) / 1e12
    prof = load_kernel_profile(args.workload) or {}
    # Some boards report an idle-level GFX clock while busy.  The dense bf16
    # peak is 2.5 PFLOP/s at 2.4 GHz, so the step's own FLOP rate needs at
    # least value / (2.5e15 / 2.4e9) cycles per second; a lower reading is
    # flagged.  The profile's SQ busy cycles per microsecond of kernel time
    # give a second, counter-based figure.
    if isinstance(clock, dict):
        floor_mhz = value * 1e12 / (PEAK_BF16_TFLOPS * 1e12 / 2.4e9) / 1e6
        clock["min_mhz_implied_by_step_rate"] = round(floor_mhz, 1)
        med = clock.get("gfx_mhz_median")
        clock["reading_plausible"] = None if med is None else bool(med >= floor_mhz)
        sq = {k: v.get("sq_busy_ghz") for k, v in prof.items() if v.get("sq_busy_ghz")}
        if sq:
            clock["sq_busy_ghz_from_profile"] = sq

    kernels = []
    for (n, entry), w, t_all, tw in zip(calls, ws, per_call, warm_ms):
        t = float(t_all.mean()) * 1e-3
        kp = prof.get(n)
        kernels.append({
            "workload": n, "entry": f"sdattn_{entry}" if entry != "fwd" else "sdattn_fwd",
            "shape": f"B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} d{w.d}",
            "us_per_launch": round(t * 1e6, 3),
            "us_per_launch_median": round(float(np.median(t_all)) * 1e3, 3),
            "us_per_launch_min": round(float(t_all.min()) * 1e3, 3),
            "tflops": round(w.flops / t / 1e12, 2),
            "gbs_alg": round(w.bytes_alg(2) / t / 1e9, 1),
            "mfma_frac": round(w.flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(w.bytes_alg(2) / t / 1e9 / PEAK_HBM_GBS, 4),
            "warm_cache_us": round(tw * 1e3, 3),
            "timing_note": "this call alone, back to back, chunks of launches between two events "
                           "(a launch's time includes the gap to the next launch); median and "
                           "min over the chunk means",
            "kernel_only_us_rocprof": None if kp is None else kp["avg_us"],
            "hbm_frac_kernel_only": None if kp is None else
            round(w.bytes_alg(2) / (kp["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        })

    peaks = None
    if not args.no_peaks:
        peaks = attainable_peaks(torch, stream, ws[-1].bytes_alg(2))
        peaks.pop("_sequence", None)

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
        if peaks and "mfma_bf16_tflops" in peaks:
            roof["frac_of_attainable"] = round(ach / peaks["mfma_bf16_tflops"], 4)
    else:
        ach = wd.bytes_alg(2) / td / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}
    roof["kernel"] = kernels[jd]["entry"] + " " + kernels[jd]["shape"]
    roof["flops_per_launch"] = wd.flops
    roof["alg_bytes_per_launch"] = wd.bytes_alg(2)
    roof["us_per_launch"] = kernels[jd]["us_per_launch"]
    roof["us_per_launch_median"] = kernels[jd]["us_per_launch_median"]
    roof["us_per_launch_min"] = kernels[jd]["us_per_launch_min"]

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(args, calls, ws, st.inputs, st.sets[0], step_flops)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": st.elt, "data": "synthetic",
        "config": {"workload": args.workload,
                   "calls": [f"{k['entry']} {k['shape']}" for k in kernels],
                   "io": f"{st.elt} in/out, fp32 accumulation",
                   "buffer_sets_rotated": nsets,
                   "rotated_bytes": nsets * st.set_bytes},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "attainable": peaks,
        "gpu_clock": clock,
        "parity_vs_oracle": parity,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


def oracle_threads(args):
    """Threads for the oracle: --cpu-threads, else OMP_NUM_THREADS (the host's
    CPU share where it is set), else every core in this process's affinity."""
    if args.cpu_threads:
        return args.cpu_threads
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_model():
    with open("/proc/cpuinfo") as f:
        return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "?")


def cpu_baseline(args, calls, ws, inputs, set0, step_flops):
    """Time the fp64 CPU oracle on the same step (test infrastructure only),
    and compare the benchmarked GPU output with it.  Steps of more than
    2 TFLOP are timed on a stated row sample (rows are independent and cost
    the same, so the rate extrapolates); small calls (under 10 GFLOP) are
    also timed on one thread."""
    import oracle
    from workloads import sample_rows
    threads = oracle_threads(args)
    orc = oracle.get()
    total, flops_done = 0.0, 0
    worst, single, samples = {}, {}, []
    for (n, _), w, x, (_, _, _, out) in zip(calls, ws, inputs, set0):
        q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (x.q, x.k, x.v))
        got = out.float().cpu().numpy().astype(np.float64)
        if w.flops > 2e12:
            rows = sample_rows(w, 2048)
            t0 = time.perf_counter()
            want = orc.attn_rows(q, k, v, w.scale, rows, nthreads=threads)
            total += time.perf_counter() - t0
            flops_done += 4 * rows.size * w.Lk * w.d
            e = np.abs(got.reshape(-1, w.d)[rows] - want)
            samples.append(f"workload {n}: {rows.size} sampled rows of {w.B * w.H * w.Lq}")
        else:
            t0 = time.perf_counter()
            want = orc.attn(q, k, v, w.scale, nthreads=threads)
            total += time.perf_counter() - t0
            flops_done += w.flops
            e = np.abs(got - want)
            samples.append(f"workload {n}: every row")
            if w.flops < 10e9:
                t0 = time.perf_counter()
                orc.attn(q, k, v, w.scale, nthreads=1)
                t1 = time.perf_counter() - t0
                single[n] = {"value": round(w.flops / t1 / 1e12, 6), "unit": "TFLOP/s",
                             "seconds": round(t1, 3)}
        worst[n] = {"max_abs": float(e.max()), "mean_abs": float(e.mean())}
    # one thread on the smaller workloads of the pages' UNet levels as well
    # (cheap: ~1 s in all), for the single-core rate at those shapes
    for n in ("1", "3", "4a", "4b", "4c", "4d"):
        if n in single or n in [c for c, _ in calls]:
            continue
        w = WORKLOADS[n]
        x = make_inputs(w)
        q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (x.q, x.k, x.v))
        t0 = time.perf_counter()
        orc.attn(q, k, v, w.scale, nthreads=1)
        t1 = time.perf_counter() - t0
        single[n] = {"value": round(w.flops / t1 / 1e12, 6), "unit": "TFLOP/s",
                     "seconds": round(t1, 3)}
    cpu = {"value": round(flops_done / total / 1e12, 6), "unit": "TFLOP/s",
           "cores": threads, "kind": "oracle",
           "sample": f"{'; '.join(samples)}; fp64, {total:.2f} s on {threads} threads of "
                     f"{cpu_model()} ({len(os.sched_getaffinity(0))} cores in affinity)",
           "single_thread": single or None}
    return cpu, worst


def bench_group_norm(args, name, quiet=False):
    """GroupNorm (+ SiLU) of one UNet level: an HBM-bound kernel, measured in
    GB/s of algorithmic traffic (x read once, y written once, gamma/beta).
    quiet: launch only (warmup + steps), no timing or output (profiler suite)."""
    import torch
    import unet_attention_amd as sd
    w = GN_WORKLOADS[name]
    x = make_gn_inputs(w)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)  # its own stream, default priority
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
    if quiet:
        for i in range(args.steps):
            launch(*sets[i % nsets])
        torch.cuda.synchronize()
        return
    # K launches back to back between two events (one launch per step; an
    # event recorded between launches would add its own GPU time)
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        launch(*sets[i % nsets])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    per_ms = ms_step
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
        threads = oracle_threads(args)
        t = time.perf_counter()
        want = oracle.group_norm(x.x, x.gamma, x.beta, w.G, w.eps, w.silu, nthreads=threads)
        el = time.perf_counter() - t
        got = sets[0][1].float().cpu().numpy().astype(np.float64)
        e = np.abs(got - want)
        parity = {name: {"max_abs": float(e.max()), "mean_abs": float(e.mean())}}
        model = cpu_model()
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
