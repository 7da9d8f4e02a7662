"""Benchmark of the rational-softmax attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode fwd_bwd|fwd] [--no-cpu]

A step is one forward (ra_attn_fwd) plus one backward (ra_attn_bwd) over the causal bf16
workload B=4, H=16, N=8192, D=128 (inputs resident in HBM before timing starts).  The value is
counted TFLOP/s: 4*B*Hq*Nq*Nk*D for the forward, halved when causal, times 3.5 for forward +
backward.  Prints one JSON line.

Also reported, each timed with HIP events on the stream the library launches on (5 warm-up
calls, then at least 20 calls and at least 1 s; median, min and mean):
  * every attention workload's forward (fp32 B=1 H=2 N=128 D=64 non-causal; bf16 causal
    B=2 H=12 N=128 D=64; bf16 causal B=8 H=16 N=2048 D=64 with Q, K of sigma 2; bf16 causal
    grouped-query B=4 Hq=32 Hkv=8 N=4096 D=128 with host RoPE; the step's workload), with the
    skipped-tile fraction from ra_attn_fwd_counted and the SHA-256 of every input buffer;
  * the step's forward, dQ and dK/dV kernels alone (ra_attn_fwd, ra_attn_bwd_dq,
    ra_attn_bwd_dkdv) and a roofline object for the longest of them, the dominant kernel;
  * a structured workload whose scores fall off away from the diagonal (whole tiles skipped)
    beside an i.i.d. workload of the same shape (nothing skipped);
  * the grouped-query workload with the NEOX rotation on the device: forward and backward,
    unfused (rotation passes plus the attention) beside the fused entry points
    (ra_attn_fwd_rope, ra_attn_bwd_rope); a padded batch through the key padding path, packed
    documents through the general explicit-mask path, the
    split-KV decode step, the row softmax and its backward (fp32 and bf16);
  * the fp64 oracle timed on a bounded sample of each workload on the host cores.

Algorithmic work per visited score element (i, j), D = head dim: forward 4*D flops (S = QK^T
and PV); dQ phase 6*D (S, dP = dO V^T, dQ += dS K); dK/dV phase 8*D (S, dP, dV += P^T dO,
dK += dS^T Q).  A causal launch visits B*Hq*Nq*Nk/2 elements (the counting convention of the
headline metric).
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
# VALU lane operations per second: 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz, the published fp32
# vector peak of 157.3 TFLOP/s counted as FMAs of two flops.  Without packed fp32 instructions
# (the library is built without them) one wave issues a 64-lane instruction about every 4
# cycles, but two waves on one SIMD each keep that rate (measured with plain FMAs), so a SIMD
# with two waves reaches 32 lanes per cycle.
PEAK_VALU_LANE_OPS = 256 * 4 * 32 * 2.4e9

MAIN = "bf16_causal_B4_H16_N8192_D128_fwd_bwd"
GQA = "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope"

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch) on the
# main workload, each scaled by what the counter read for a plain copy of 256 MiB read + 256
# MiB written (FETCH_SIZE counted half the bytes read: x2; WRITE_SIZE all of them: x1).  Valid
# only for the kernel source the counters were taken on (sha256 of the files listed; moved on to
# a later source only when the kernels' gfx950 assembly is unchanged).
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC = {
    # kernel: (sha256 of its KERNEL_SOURCES concatenated, FETCH_SIZE KiB, WRITE_SIZE KiB)
    "attn_fwd_kernel": ("3177d22ee600e987d71867dc1a06396f1cee3dc3bd89d4d64d0e183a1935de6d",
                        286919.0, 135180.3),
    "attn_bwd_dq_bf16_kernel": ("9c9406fdab48c334200ef155bcff02395064a245e4dddcb0a21ac4dc604f330b",
                                441266.4, 143463.7),
    "attn_bwd_dkdv_bf16_kernel": ("9c9406fdab48c334200ef155bcff02395064a245e4dddcb0a21ac4dc604f330b",
                                  272491.0, 274299.0),
}
# VALU and MFMA instructions per dispatch (rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA, one run)
# of the forward on a workload, for its VALU-roofline fraction; valid for the recorded kernel
# source only.  SQ_INSTS_VALU counts the MFMA instructions too (they issue through the VALU: the
# forward's loops hold about 283 vector and 48 matrix instructions per wave and 64-key tile at
# D = 128, against 345 counted), so the vector lane operations are 64 x (VALU - MFMA).
VALU_INSTS = {
    # workload: (sha256 of the forward's sources, SQ_INSTS_VALU, SQ_INSTS_MFMA per dispatch)
    "fp32_noncausal_B1_H2_N128_D64": ("3177d22ee600e987d71867dc1a06396f1cee3dc3bd89d4d64d0e183a1935de6d", 11560, 3072),
    "bf16_causal_B2_H12_N128_D64": ("3177d22ee600e987d71867dc1a06396f1cee3dc3bd89d4d64d0e183a1935de6d", 101160, 3456),
    "bf16_causal_B8_H16_N2048_D64_sigma2": ("3177d22ee600e987d71867dc1a06396f1cee3dc3bd89d4d64d0e183a1935de6d", 45893632, 3244032),
    "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope": ("3177d22ee600e987d71867dc1a06396f1cee3dc3bd89d4d64d0e183a1935de6d", 189317120, 25559040),
    "bf16_causal_B4_H16_N8192_D128_fwd_bwd": ("3177d22ee600e987d71867dc1a06396f1cee3dc3bd89d4d64d0e183a1935de6d", 364273664, 50724864),
}
KERNEL_SOURCES = {
    "attn_fwd_kernel": ["ra_fwd.hip", "ra_device.h"],
    "attn_bwd_dq_bf16_kernel": ["ra_bwd.hip", "ra_device.h"],
    "attn_bwd_dkdv_bf16_kernel": ["ra_bwd.hip", "ra_device.h"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["fwd_bwd", "fwd"], default="fwd_bwd")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--min-time", type=float, default=1.0,
                    help="seconds each secondary measurement runs at least")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Attn:
    """Device-resident inputs/outputs of one workload and the C-ABI calls on them."""

    def __init__(self, ra, w, need_grad, inp=None):
        import torch
        import workloads as wl
        self.ra, self.w = ra, w
        inp = wl.make_attention_inputs(w) if inp is None else inp
        self.host = inp
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dev = lambda a: torch.from_numpy(a).to(dt).cuda()   # exact: values are dtype-representable
        self.q, self.k, self.v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
        self.o = torch.empty_like(self.q)
        self.stats = torch.empty((w.B, w.Hq, w.Nq, 2), dtype=torch.float32, device="cuda")
        self.code = ra.RA_BF16 if w.dtype == "bf16" else ra.RA_F32
        if need_grad:
            self.do = dev(inp["do"])
            self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
            self.ws_bytes = ra.ra_attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, self.code)
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream()

    def _ok(self, st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {self.ra.ra_status_string(st)}")

    def fwd(self):
        w = self.w
        self._ok(self.ra.ra_attn_fwd(self.q, self.k, self.v, self.o, self.stats, w.B, w.Hq, w.Hkv,
                                     w.Nq, w.Nk, w.D, int(w.causal), w.scale, self.code, self.stream),
                 "ra_attn_fwd")

    def fwd_counted(self):
        """Skipped-tile counters of one forward: (wave tiles, wave tiles skipped, workgroup
        tiles, workgroup tiles not loaded)."""
        import torch
        w = self.w
        cnt = torch.zeros(4, dtype=torch.int64, device="cuda")
        self._ok(self.ra.ra_attn_fwd_counted(self.q, self.k, self.v, self.o, self.stats, w.B, w.Hq,
                                             w.Hkv, w.Nq, w.Nk, w.D, int(w.causal), w.scale,
                                             self.code, cnt, self.stream), "ra_attn_fwd_counted")
        torch.cuda.synchronize()
        c = [int(x) for x in cnt.cpu().numpy()]
        return {"wave_tiles": c[0], "wave_tiles_skipped": c[1],
                "skipped_fraction": round(c[1] / c[0], 6) if c[0] else 0.0,
                "workgroup_tiles": c[2], "workgroup_tiles_not_loaded": c[3],
                "not_loaded_fraction": round(c[3] / c[2], 6) if c[2] else 0.0}

    def bwd(self):
        w = self.w
        self._ok(self.ra.ra_attn_bwd(self.q, self.k, self.v, self.o, self.do, self.stats, self.dq,
                                     self.dk, self.dv, self.ws, self.ws_bytes, w.B, w.Hq, w.Hkv, w.Nq,
                                     w.Nk, w.D, int(w.causal), w.scale, self.code, self.stream),
                 "ra_attn_bwd")

    def fwd_masked(self, mask, causal=None):
        w = self.w
        cc = int(w.causal) if causal is None else causal
        self._ok(self.ra.ra_attn_fwd_masked(self.q, self.k, self.v, self.o, self.stats, w.B, w.Hq,
                                            w.Hkv, w.Nq, w.Nk, w.D, cc, w.scale, self.code,
                                            *mask, self.stream), "ra_attn_fwd_masked")

    def bwd_masked(self, mask):
        w = self.w
        self._ok(self.ra.ra_attn_bwd_masked(self.q, self.k, self.v, self.o, self.do, self.stats,
                                            self.dq, self.dk, self.dv, self.ws, self.ws_bytes, w.B,
                                            w.Hq, w.Hkv, w.Nq, w.Nk, w.D, int(w.causal), w.scale,
                                            self.code, *mask, self.stream), "ra_attn_bwd_masked")

    def bwd_dq(self):
        w = self.w
        self._ok(self.ra.ra_attn_bwd_dq(self.q, self.k, self.v, self.o, self.do, self.stats, self.dq,
                                        self.ws, self.ws_bytes, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D,
                                        int(w.causal), w.scale, self.code, self.stream),
                 "ra_attn_bwd_dq")

    def bwd_dkdv(self):
        w = self.w
        self._ok(self.ra.ra_attn_bwd_dkdv(self.q, self.k, self.v, self.do, self.stats, self.dk,
                                          self.dv, self.ws, self.ws_bytes, w.B, w.Hq, w.Hkv, w.Nq,
                                          w.Nk, w.D, int(w.causal), w.scale, self.code, self.stream),
                 "ra_attn_bwd_dkdv")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "rational_softmax_tiled_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """HBM bytes per launch from the recorded counters, or None if the kernel has changed."""
    rec = TRAFFIC.get(kernel)
    if rec is None or source_digest(KERNEL_SOURCES[kernel]) != rec[0]:
        return None
    return int(rec[1] * 1024 * FETCH_SCALE + rec[2] * 1024 * WRITE_SCALE)


def timed(stream, fn, min_s, min_calls=20, warm=5):
    """Durations of fn() from HIP events recorded on `stream` around each call: `warm` untimed
    calls, then batches until at least min_calls calls and min_s seconds are timed."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    times = []
    while len(times) < min_calls or sum(times) < 1e3 * min_s:
        n = max(min_calls - len(times), 10)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            ev[2 * i].record(stream)
            fn()
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        times += [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]
        if len(times) >= 20000:
            break
    t = np.asarray(times)
    return {"median_ms": round(float(np.median(t)), 5), "min_ms": round(float(t.min()), 5),
            "mean_ms": round(float(t.mean()), 5), "calls": int(t.size)}


def timed_graph(run, fn, calls=64, reps=20):
    """Per-call duration of fn() with no launch overhead: `calls` calls captured in one HIP
    graph on a side stream (run.stream pointed at it during capture), replayed `reps` times
    between HIP events.  Median and min over the replays, divided by `calls`."""
    import torch
    keep = run.stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.stream = side
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.stream = torch.cuda.current_stream()
        for _ in range(calls):
            fn()
    run.stream = keep
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b) / calls)
    t = np.asarray(times)
    return {"median_ms": round(float(np.median(t)), 5), "min_ms": round(float(t.min()), 5),
            "calls_per_graph": calls, "replays": reps}


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def environment():
    import torch
    dev = torch.cuda.get_device_properties(0)
    env = {"device": dev.name, "arch": getattr(dev, "gcnArchName", None),
           "compute_units": dev.multi_processor_count, "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None), "rocm": None, "sclk_mhz": None,
           "host": platform.node(), "host_cpus": os.cpu_count()}
    try:
        with open("/opt/rocm/.info/version") as fh:
            env["rocm"] = fh.read().strip()
    except OSError:
        pass
    # shader clock levels of the card (the one marked * is current); max = the part's peak
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            levels = open(path).read().split("\n")
        except OSError:
            continue
        mhz = [int(l.split(":")[1].strip().split("Mhz")[0]) for l in levels if "Mhz" in l]
        cur = [int(l.split(":")[1].strip().split("Mhz")[0]) for l in levels if "*" in l]
        if mhz:
            env["sclk_mhz"] = {"max": max(mhz), "current": cur[0] if cur else None}
            break
    return env


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = None, None
    try:
        import threadpoolctl
        for d in threadpoolctl.threadpool_info():
            if d.get("user_api") == "blas":
                blas = f"{d.get('internal_api')} {d.get('version')}"
                threads = d.get("num_threads")
                break
    except Exception:                      # pragma: no cover
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas": blas,
            "blas_threads": threads}


def oracle_time(w, inp, heads, with_bwd):
    """Wall time of the fp64 oracle on the first `heads` (batch 0) query heads of workload w
    (with their K/V heads), forward or forward + backward, and the counted TFLOP/s."""
    import oracle
    rep = w.Hq // w.Hkv
    nkv = (heads + rep - 1) // rep
    q, k, v = inp["q"][:1, :heads], inp["k"][:1, :nkv], inp["v"][:1, :nkv]
    reps = 0
    t0 = time.perf_counter()
    while True:          # small samples are repeated until a measurable time has passed
        oracle.ra_attention_fwd(q, k, v, w.causal, w.scale)
        if with_bwd:
            oracle.ra_attention_bwd(q, k, v, inp["do"][:1, :heads], w.causal, w.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 0.25:
            break
    f = w.counted_flops_fwd() * heads / (w.B * w.Hq) * (3.5 if with_bwd else 1.0)
    return dt / reps, f * reps / dt / 1e12


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs on one GPU and has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import rational_softmax_tiled_amd as ra
    import workloads as wl
    ra.load_library()
    env = environment()
    log(f"device {env['device']} CUs={env['compute_units']} arch={env['arch']} rocm={env['rocm']} "
        f"sclk={env['sclk_mhz']}")
    min_s = args.min_time

    if args.copy_calibration:
        # a plain copy kernel of known size: 256 MiB read + 256 MiB written
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 268435456 bytes read, 268435456 bytes written")
        del src, dst

    need_grad = args.mode == "fwd_bwd"
    cpu_samples = {}            # workload -> (inputs, heads, with_bwd) for the oracle leg

    # ---- the step (the headline measurement)
    w = wl.WORKLOADS[MAIN]
    log(f"generating {w.name}")
    main_inp = wl.make_attention_inputs(w)
    main_run = Attn(ra, w, need_grad, inp=main_inp)
    stream = main_run.stream

    def step():
        main_run.fwd()
        if need_grad:
            main_run.bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    flops_step = w.counted_flops_fwd_bwd() if need_grad else w.counted_flops_fwd()
    value = tflops(flops_step, ms_step)
    log(f"step {ms_step:.3f} ms ({wall:.2f} s wall for {args.steps} steps): {value:.1f} TFLOP/s")
    step_t = timed(stream, step, min_s, warm=0)
    log(f"step per call: median {step_t['median_ms']:.3f} ms, min {step_t['min_ms']:.3f} ms")

    # ---- the step's kernels alone (one launch per entry-point call)
    elems = w.B * w.Hq * w.Nq * w.Nk / (2 if w.causal else 1)   # visited score elements
    fwd_t = timed(stream, main_run.fwd, min_s)
    # (name, C entry point, timing, algorithmic flops per launch)
    kernels = [("attn_fwd_kernel", "ra_attn_fwd", fwd_t, 4 * w.D * elems)]
    if need_grad:
        bwd_t = timed(stream, main_run.bwd, min_s)
        dq_t = timed(stream, main_run.bwd_dq, min_s)        # leaves the row terms in place
        dkdv_t = timed(stream, main_run.bwd_dkdv, min_s)
        log(f"backward {bwd_t['median_ms']:.3f} ms: dQ {dq_t['median_ms']:.3f} ms, "
            f"dK/dV {dkdv_t['median_ms']:.3f} ms")
        kernels += [("attn_bwd_dq_bf16_kernel", "ra_attn_bwd_dq", dq_t, 6 * w.D * elems),
                    ("attn_bwd_dkdv_bf16_kernel", "ra_attn_bwd_dkdv", dkdv_t, 8 * w.D * elems)]
    main_skip = main_run.fwd_counted()
    del main_run
    torch.cuda.empty_cache()

    # ---- every attention workload's forward
    configs = {}
    for name in wl.WORKLOAD_ORDER:
        wc = wl.WORKLOADS[name]
        if name == MAIN:
            inp, t = main_inp, fwd_t
            skip = main_skip
        else:
            log(f"generating {name}")
            inp = wl.make_attention_inputs(wc)
            run = Attn(ra, wc, False, inp=inp)
            t = timed(run.stream, run.fwd, min_s)
            if t["median_ms"] < 0.1:   # launch-bound: the kernel's own time from a HIP graph
                t = {**t, "graph": timed_graph(run, run.fwd)}
            skip = run.fwd_counted()
            del run
            torch.cuda.empty_cache()
        tf = tflops(wc.counted_flops_fwd(), t["median_ms"])
        configs[name] = {
            "pass": "fwd", "dtype": wc.dtype, "causal": wc.causal, "B": wc.B, "Hq": wc.Hq,
            "Hkv": wc.Hkv, "N": wc.Nq, "D": wc.D, "seed": wc.seed, **t,
            "tflops": round(tf, 3), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 5),
            "skip": skip, "inputs_sha256": wl.storage_sha256(inp, wc.dtype)}
        rec = VALU_INSTS.get(name)
        if rec is not None and rec[0] == source_digest(KERNEL_SOURCES["attn_fwd_kernel"]):
            lane_ops = (rec[1] - rec[2]) * 64
            configs[name]["valu"] = {
                "lane_ops_per_launch": lane_ops, "peak_lane_ops_per_s": PEAK_VALU_LANE_OPS,
                "frac": round(lane_ops / (t["median_ms"] * 1e-3) / PEAK_VALU_LANE_OPS, 4)}
        if name == MAIN and need_grad:
            configs[name]["fwd_bwd"] = {**step_t, "tflops": round(tflops(flops_step, step_t["median_ms"]), 3)}
        log(f"{name}: forward median {t['median_ms']:.4f} ms ({tf:.1f} TFLOP/s), "
            f"skipped tiles {skip['skipped_fraction']:.4f}"
            + (f"; in a HIP graph {t['graph']['median_ms']:.4f} ms per call" if "graph" in t else ""))
        heads = {"fp32_noncausal_B1_H2_N128_D64": 2, "bf16_causal_B2_H12_N128_D64": 12,
                 "bf16_causal_B8_H16_N2048_D64_sigma2": 8, GQA: 4, MAIN: 3}[name]
        cpu_samples[name] = (wc, inp, heads, name == MAIN and need_grad)

    # ---- tile skipping: the structured workload beside an i.i.d. one of the same shape
    loc = wl.LOCAL
    wloc = wl.AttnWorkload("bf16_causal_local_B1_H16_N2048_D64_amp4", "bf16", True, loc["B"],
                           loc["H"], loc["H"], loc["N"], loc["N"], loc["D"], seed=loc["seed"])
    inp_loc = wl.make_local_inputs(B=loc["B"], H=loc["H"], N=loc["N"], D=loc["D"],
                                   amplitude=loc["amplitude"], seed=loc["seed"])
    runl = Attn(ra, wloc, False, inp=inp_loc)
    tl = timed(runl.stream, runl.fwd, min_s)
    skl = runl.fwd_counted()
    del runl
    runi = Attn(ra, wl.LOCAL_IID, False)
    ti = timed(runi.stream, runi.fwd, min_s)
    ski = runi.fwd_counted()
    del runi
    torch.cuda.empty_cache()
    local = {"workload": wloc.name, "inputs": "Q = K = RoPE(4 c + 0.5 e), one c per head",
             "with_skipping": {**tl, "skip": skl},
             "iid_same_shape": {"workload": wl.LOCAL_IID.name, **ti, "skip": ski},
             "speedup": round(ti["median_ms"] / tl["median_ms"], 3)}
    log(f"local workload: {tl['median_ms']:.4f} ms with {skl['skipped_fraction']:.3f} of wave tiles "
        f"skipped; i.i.d. same shape {ti['median_ms']:.4f} ms")

    # ---- grouped-query attention with the rotation on the device: unfused (two rotation passes,
    # then the attention) beside the fused entry points (Q rotated inside the attention kernel)
    wg = wl.WORKLOADS[GQA]
    gqa = Attn(ra, wg, True, inp=wl.make_unrotated_inputs(wg))
    q_rot, k_rot = torch.empty_like(gqa.q), torch.empty_like(gqa.k)
    dims = (wg.B, wg.Hq, wg.Hkv, wg.Nq, wg.Nk, wg.D)
    theta = wg.rope_theta

    def ok(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {ra.ra_status_string(st)}")

    def rope_qk():
        for x, y, H in ((gqa.q, q_rot, wg.Hq), (gqa.k, k_rot, wg.Hkv)):
            ok(ra.ra_rope_neox(x, y, None, wg.B * H, wg.Nq, wg.D, theta, False, gqa.code, gqa.stream),
               "ra_rope_neox")

    def unfused_fwd():
        rope_qk()
        ok(ra.ra_attn_fwd(q_rot, k_rot, gqa.v, gqa.o, gqa.stats, *dims, 1, wg.scale, gqa.code,
                          gqa.stream), "ra_attn_fwd")

    def fused_fwd(qr=True):
        ok(ra.ra_attn_fwd_rope(gqa.q, gqa.k, gqa.v, gqa.o, gqa.stats, q_rot if qr else None, k_rot,
                               None, None, theta, *dims, 1, wg.scale, gqa.code, stream=gqa.stream),
           "ra_attn_fwd_rope")

    def unfused_bwd():
        ok(ra.ra_attn_bwd(q_rot, k_rot, gqa.v, gqa.o, gqa.do, gqa.stats, gqa.dq, gqa.dk, gqa.dv,
                          gqa.ws, gqa.ws_bytes, *dims, 1, wg.scale, gqa.code, gqa.stream), "ra_attn_bwd")
        for t, H in ((gqa.dq, wg.Hq), (gqa.dk, wg.Hkv)):
            ok(ra.ra_rope_neox(t, t, None, wg.B * H, wg.Nq, wg.D, theta, True, gqa.code, gqa.stream),
               "ra_rope_neox")

    def fused_bwd():
        ok(ra.ra_attn_bwd_rope(q_rot, k_rot, gqa.v, gqa.o, gqa.do, gqa.stats, gqa.dq, gqa.dk, gqa.dv,
                               gqa.ws, gqa.ws_bytes, None, None, theta, *dims, 1, wg.scale, gqa.code,
                               stream=gqa.stream), "ra_attn_bwd_rope")

    rope_t = timed(gqa.stream, rope_qk, min_s)
    rope_bytes = 2 * (gqa.q.numel() + gqa.k.numel()) * gqa.q.element_size()
    rope_gbs = rope_bytes / (rope_t["median_ms"] * 1e-3) / 1e9
    unf_t = timed(gqa.stream, unfused_fwd, min_s)
    fus_t = timed(gqa.stream, fused_fwd, min_s)
    fus_nq_t = timed(gqa.stream, lambda: fused_fwd(False), min_s)
    fused_fwd()
    unfb_t = timed(gqa.stream, unfused_bwd, min_s)
    fusb_t = timed(gqa.stream, fused_bwd, min_s)
    log(f"GQA RoPE: rotation of Q and K {rope_t['median_ms']:.3f} ms ({rope_gbs:.0f} GB/s); forward "
        f"unfused {unf_t['median_ms']:.3f} ms, fused {fus_t['median_ms']:.3f} ms (without q_rot "
        f"{fus_nq_t['median_ms']:.3f}); backward unfused {unfb_t['median_ms']:.3f} ms, fused "
        f"{fusb_t['median_ms']:.3f} ms")
    rope_out = {"workload": wg.name, "inputs": "Q, K unrotated; theta 10000, positions 0..N-1",
                "rotation_q_k": rope_t, "rotation_GB/s": round(rope_gbs, 1),
                "fwd_unfused": unf_t, "fwd_fused": fus_t, "fwd_fused_without_q_rot": fus_nq_t,
                "bwd_unfused": unfb_t, "bwd_fused": fusb_t}
    del gqa, q_rot, k_rot
    torch.cuda.empty_cache()

    # ---- explicit-mask path: a padded batch, key padding mask [B, N] (1 = attend), causal
    wp = wl.padded_batch_workload()
    pad = Attn(ra, wp, True)
    keep = torch.from_numpy(wl.padded_batch_keep(wp)).cuda()
    kpm = (keep, ra.RA_MASK_BOOL, (wp.Nk, 0, 0, 1))
    pm_t = timed(pad.stream, lambda: (pad.fwd_masked(kpm), pad.bwd_masked(kpm)), min_s)
    pp_t = timed(pad.stream, lambda: (pad.fwd(), pad.bwd()), min_s)
    pmf_t = timed(pad.stream, lambda: pad.fwd_masked(kpm), min_s)
    log(f"padded batch fwd+bwd {pm_t['median_ms']:.3f} ms (forward {pmf_t['median_ms']:.3f} ms); "
        f"unmasked {pp_t['median_ms']:.3f} ms")
    del pad, keep
    torch.cuda.empty_cache()

    # ---- general explicit mask: packed documents, one [B, N, N] boolean mask over all heads
    wdoc = wl.documents_workload()
    doc = Attn(ra, wdoc, True)
    dkeep = wl.documents_keep(wdoc)
    dmask = (torch.from_numpy(dkeep).cuda(), ra.RA_MASK_BOOL, (wdoc.Nq * wdoc.Nk, 0, wdoc.Nk, 1))
    # visited entries: the causal ones the mask keeps
    doc_entries = float(np.tril(dkeep).sum()) * wdoc.Hq
    dm_t = timed(doc.stream, lambda: doc.fwd_masked(dmask), min_s)
    dmb_t = timed(doc.stream, lambda: (doc.fwd_masked(dmask), doc.bwd_masked(dmask)), min_s)
    dc_t = timed(doc.stream, lambda: doc.fwd(), min_s)
    # the same documents as an additive bf16 mask, 0 where kept and -inf where not
    dadd = torch.zeros(dkeep.shape, dtype=torch.bfloat16, device="cuda")
    dadd[~dmask[0]] = float("-inf")
    amask = (dadd, ra.RA_MASK_ADD, dmask[2])
    da_t = timed(doc.stream, lambda: doc.fwd_masked(amask), min_s)
    dab_t = timed(doc.stream, lambda: (doc.fwd_masked(amask), doc.bwd_masked(amask)), min_s)
    log(f"packed documents: masked forward {dm_t['median_ms']:.3f} ms, fwd+bwd {dmb_t['median_ms']:.3f} ms; "
        f"as a 0/-inf additive mask {da_t['median_ms']:.3f} / {dab_t['median_ms']:.3f} ms; "
        f"causal forward without the mask {dc_t['median_ms']:.3f} ms")
    doc_out = {"workload": wdoc.name, "mask": "[B, N, N] bool (same document), causal top-left",
               "kept_causal_entries": int(doc_entries),
               "kept_fraction_of_causal": round(doc_entries / (wdoc.B * wdoc.Hq * wdoc.Nq * (wdoc.Nq + 1) / 2), 4),
               "fwd": dm_t, "fwd_bwd": dmb_t, "unmasked_causal_fwd": dc_t,
               "additive_0_neginf_bf16": {"fwd": da_t, "fwd_bwd": dab_t},
               "fwd_tflops_on_kept_entries": round(4 * wdoc.D * doc_entries / (dm_t["median_ms"] * 1e-3) / 1e12, 2)}
    del doc, dkeep, dmask, dadd, amask
    torch.cuda.empty_cache()

    # ---- split-KV decode: one query row per head against caches of per-sample lengths
    wd = wl.decode_workload()
    dec = Attn(ra, wd, False)
    lens_np = wl.decode_seqlens(wd)
    lens = torch.from_numpy(lens_np).cuda()
    dws_bytes = ra.ra_attn_decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.Nq, wd.Nk, wd.D, dec.code)
    dws = torch.empty(dws_bytes, dtype=torch.uint8, device="cuda")

    def decode_step():
        st = ra.ra_attn_decode(dec.q, dec.k, dec.v, dec.o, None, lens, dws, dws_bytes, wd.B, wd.Hq,
                               wd.Hkv, wd.Nq, wd.Nk, wd.D, ra.RA_CAUSAL_BOTTOM_RIGHT, wd.scale,
                               dec.code, dec.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_decode: {ra.ra_status_string(st)}")
    dec_t = timed(dec.stream, decode_step, min_s)
    dec_t["graph"] = timed_graph(dec, decode_step, calls=32)   # the three kernels, no launch gaps
    kv_bytes = int(lens_np.astype(np.int64).sum()) * wd.Hkv * wd.D * 2 * dec.q.element_size()
    dec_gbs = kv_bytes / (dec_t["median_ms"] * 1e-3) / 1e9
    dec_t["graph"]["GB/s"] = round(kv_bytes / (dec_t["graph"]["median_ms"] * 1e-3) / 1e9, 1)
    keep = torch.arange(wd.Nk, device="cuda")[None, :] < lens[:, None]
    kpm = (keep, ra.RA_MASK_BOOL, (wd.Nk, 0, 0, 1))
    br = ra.RA_CAUSAL_BOTTOM_RIGHT   # one query row: every key below the sample's length
    decf_t = timed(dec.stream, lambda: dec.fwd_masked(kpm, br), min_s)
    log(f"decode: {dec_t['median_ms']:.4f} ms, {dec_gbs:.0f} GB/s of K/V (in a HIP graph "
        f"{dec_t['graph']['median_ms']:.4f} ms, {dec_t['graph']['GB/s']:.0f} GB/s); tiled forward "
        f"with the lengths as a mask {decf_t['median_ms']:.4f} ms")
    del dec, dws, keep
    torch.cuda.empty_cache()
    # the same step with fp32 caches (twice the bytes per key)
    wd32 = wl.decode_workload("f32")
    dec32 = Attn(ra, wd32, False)
    dws32_bytes = ra.ra_attn_decode_workspace_bytes(wd32.B, wd32.Hq, wd32.Hkv, wd32.Nq, wd32.Nk,
                                                    wd32.D, dec32.code)
    dws32 = torch.empty(dws32_bytes, dtype=torch.uint8, device="cuda")

    def decode_step_f32():
        st = ra.ra_attn_decode(dec32.q, dec32.k, dec32.v, dec32.o, None, lens, dws32, dws32_bytes,
                               wd32.B, wd32.Hq, wd32.Hkv, wd32.Nq, wd32.Nk, wd32.D,
                               ra.RA_CAUSAL_BOTTOM_RIGHT, wd32.scale, dec32.code, dec32.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_decode: {ra.ra_status_string(st)}")
    dec32_t = timed(dec32.stream, decode_step_f32, min_s)
    kv32_bytes = int(lens_np.astype(np.int64).sum()) * wd32.Hkv * wd32.D * 2 * 4
    dec32_gbs = kv32_bytes / (dec32_t["median_ms"] * 1e-3) / 1e9
    log(f"decode fp32: {dec32_t['median_ms']:.4f} ms, {dec32_gbs:.0f} GB/s of K/V")
    del dec32, dws32
    torch.cuda.empty_cache()

    # ---- row softmax and its backward (HBM-bound)
    x = torch.from_numpy(wl.make_rows(16384, 8192, seed=11)).cuda()
    p = torch.empty_like(x)
    sm_t = timed(stream, lambda: ra.ra_softmax_rows(x, p, 16384, 8192, ra.RA_F32, stream), min_s)
    sm_gbs = 2 * x.numel() * 4 / (sm_t["median_ms"] * 1e-3) / 1e9
    g = torch.from_numpy(np.random.default_rng(12).standard_normal((16384, 8192), dtype=np.float32)).cuda()
    dx = torch.empty_like(x)
    smb_t = timed(stream, lambda: ra.ra_softmax_rows_bwd(x, g, dx, 16384, 8192, ra.RA_F32, stream), min_s)
    smb_gbs = 3 * x.numel() * 4 / (smb_t["median_ms"] * 1e-3) / 1e9
    log(f"softmax rows {sm_t['median_ms']:.3f} ms ({sm_gbs:.0f} GB/s), backward "
        f"{smb_t['median_ms']:.3f} ms ({smb_gbs:.0f} GB/s)")
    # the same rows in bf16 (the values rounded to bf16), half the bytes per element
    xh = torch.from_numpy(wl.make_rows(16384, 8192, seed=11, dtype="bf16")).cuda().to(torch.bfloat16)
    gh = g.to(torch.bfloat16)
    ph, dxh = torch.empty_like(xh), torch.empty_like(xh)
    smh_t = timed(stream, lambda: ra.ra_softmax_rows(xh, ph, 16384, 8192, ra.RA_BF16, stream), min_s)
    smh_gbs = 2 * xh.numel() * 2 / (smh_t["median_ms"] * 1e-3) / 1e9
    smbh_t = timed(stream, lambda: ra.ra_softmax_rows_bwd(xh, gh, dxh, 16384, 8192, ra.RA_BF16, stream), min_s)
    smbh_gbs = 3 * xh.numel() * 2 / (smbh_t["median_ms"] * 1e-3) / 1e9
    log(f"softmax rows bf16 {smh_t['median_ms']:.3f} ms ({smh_gbs:.0f} GB/s), backward "
        f"{smbh_t['median_ms']:.3f} ms ({smbh_gbs:.0f} GB/s)")
    del x, p, g, dx, xh, gh, ph, dxh
    # reference for the HBM-bound kernels: torch's device copy of 1 GiB (read, then written)
    src = torch.empty(256 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    cp_t = timed(stream, lambda: dst.copy_(src), min_s)
    cp_gbs = 2 * src.numel() * 4 / (cp_t["median_ms"] * 1e-3) / 1e9
    log(f"device copy of 1 GiB {cp_t['median_ms']:.3f} ms ({cp_gbs:.0f} GB/s)")
    del src, dst

    # ---- dominant kernel: the longest launch of the step (one launch per entry-point call)
    dom_name, dom_call, dom_t, dom_flops = max(kernels, key=lambda t: t[2]["mean_ms"])
    achieved = tflops(dom_flops, dom_t["mean_ms"])
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_bytes(dom_name), "kernel": f"{dom_name} ({dom_call})",
                "avg_launch_ms": dom_t["mean_ms"], "median_launch_ms": dom_t["median_ms"],
                "flops_per_launch": dom_flops}
    kernel_table = {n: {**t, "tflops": round(tflops(f, t["median_ms"]), 2),
                        "traffic": traffic_bytes(n),
                        "frac_of_peak": round(tflops(f, t["median_ms"]) / PEAK_BF16_TFLOPS, 4)}
                    for n, _, t, f in kernels}

    # ---- the oracle on the host cores (bounded samples)
    cpu = None
    if not args.no_cpu:
        info = cpu_info()
        per = {}
        for name, (wc, inp, heads, with_bwd) in cpu_samples.items():
            dt, tf = oracle_time(wc, inp, heads, with_bwd)
            gpu_tf = configs[name]["fwd_bwd"]["tflops"] if with_bwd else configs[name]["tflops"]
            per[name] = {"heads": heads, "of_heads": wc.B * wc.Hq,
                         "pass": "fwd_bwd" if with_bwd else "fwd", "seconds": round(dt, 3),
                         "tflops": round(tf, 6), "gpu_over_oracle": round(gpu_tf / tf, 1)}
            log(f"oracle {name}: {heads} heads in {dt:.2f} s ({tf:.5f} TFLOP/s)")
        m = per[MAIN]
        cpu = {"value": m["tflops"], "unit": "TFLOP/s", "cores": info["blas_threads"] or info["os_cpu_count"],
               "kind": "oracle",
               "sample": f"{m['heads']} of {m['of_heads']} (batch, head) pairs of {MAIN}, "
                         f"{'forward+backward' if m['pass'] == 'fwd_bwd' else 'forward'}, fp64 NumPy "
                         f"with the full score matrix, {m['seconds']} s; scaled by heads",
               **info, "per_workload": per}

    out = {
        "metric": "ra_attention fwd & fwd+bwd TFLOP/s (bf16, causal) + % of MFMA bf16 peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": args.mode, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "seq_len": w.Nq, "head_dim": w.D, "causal": w.causal, "global_batch": w.B,
                   "seed": w.seed},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "step": step_t,
        "fwd": {"workload": w.name, **fwd_t, "tflops": round(tflops(w.counted_flops_fwd(), fwd_t["median_ms"]), 2),
                "frac_of_peak": round(tflops(w.counted_flops_fwd(), fwd_t["median_ms"]) / PEAK_BF16_TFLOPS, 4)},
        "bwd": bwd_t if need_grad else None,
        "kernels": kernel_table,
        "configs": configs,
        "tile_skipping": local,
        "gqa_device_rope": rope_out,
        "masked_padded_batch": {"workload": wp.name, "lengths": list(wl.padded_batch_lengths(wp)),
                                "mask": "key padding [B, N] bool, causal top-left",
                                "fwd_bwd": pm_t, "fwd": pmf_t, "unmasked_fwd_bwd": pp_t,
                                "tflops_counted": round(tflops(wp.counted_flops_fwd_bwd(), pm_t["median_ms"]), 2)},
        "masked_documents": doc_out,
        "decode": {"workload": wd.name, "entry": "ra_attn_decode", **dec_t, "kv_bytes": kv_bytes,
                   "GB/s": round(dec_gbs, 1), "frac_of_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "tiled_fwd_masked": decf_t,
                   "f32": {"workload": wd32.name, **dec32_t, "kv_bytes": kv32_bytes,
                           "GB/s": round(dec32_gbs, 1),
                           "frac_of_hbm_peak": round(dec32_gbs / PEAK_HBM_GBS, 4)}},
        "softmax_rows": {"shape": [16384, 8192], "dtype": "f32", **sm_t, "GB/s": round(sm_gbs, 1),
                         "frac_of_hbm_peak": round(sm_gbs / PEAK_HBM_GBS, 4)},
        "softmax_rows_bwd": {"shape": [16384, 8192], "dtype": "f32", **smb_t, "GB/s": round(smb_gbs, 1),
                             "frac_of_hbm_peak": round(smb_gbs / PEAK_HBM_GBS, 4)},
        "softmax_rows_bf16": {"shape": [16384, 8192], "dtype": "bf16", **smh_t, "GB/s": round(smh_gbs, 1),
                              "frac_of_hbm_peak": round(smh_gbs / PEAK_HBM_GBS, 4)},
        "softmax_rows_bwd_bf16": {"shape": [16384, 8192], "dtype": "bf16", **smbh_t,
                                  "GB/s": round(smbh_gbs, 1), "frac_of_hbm_peak": round(smbh_gbs / PEAK_HBM_GBS, 4)},
        "hbm_copy_reference": {"what": "torch device copy, 1 GiB read + 1 GiB written", **cp_t,
                               "GB/s": round(cp_gbs, 1), "frac_of_hbm_peak": round(cp_gbs / PEAK_HBM_GBS, 4)},
        "environment": env,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
