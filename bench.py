"""Benchmark of the rational-softmax attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode fwd_bwd|fwd] [--no-cpu]

A step is one forward (ra_attn_fwd) plus one backward (ra_attn_bwd) over the causal bf16
workload B=4, H=16, N=8192, D=128 (inputs resident in HBM before timing starts).  The
value is counted TFLOP/s: 4*B*Hq*Nq*Nk*D for the forward, halved when causal, times 3.5 for
forward + backward.  Prints one JSON line.

Also reported: the forward alone on this workload and on the grouped-query workload
(B=4, Hq=32, Hkv=8, N=4096, D=128, host RoPE), the two backward phases (ra_attn_bwd_dq,
ra_attn_bwd_dkdv) alone, a padded batch through the explicit-mask entry points (B=4, H=16,
N=4096, D=128, causal, key padding mask with per-sample lengths) beside the same workload
unmasked, the split-KV decode step (B=16, Hq=32, Hkv=8, one query row per head, caches of up to
16384 keys with per-sample lengths; HBM GB/s of the K/V bytes the lengths require), the row
softmax and its backward at [16384, 8192], a roofline object for the
dominant kernel (the longest of the forward, dQ and dK/dV kernels, each timed alone with HIP
events on the stream the library launches it on) and the fp64 oracle timed on a bounded
sample on the host cores.

Algorithmic work per visited score element (i, j), D = head dim: forward 4*D flops (S = QK^T
and PV); dQ phase 6*D (S, dP = dO V^T, dQ += dS K); dK/dV phase 8*D (S, dP, dV += P^T dO,
dK += dS^T Q).  A causal launch visits B*Hq*Nq*Nk/2 elements (the counting convention of
the headline metric).
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published

MAIN = "bf16_causal_B4_H16_N8192_D128_fwd_bwd"

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch) on the
# main workload, each scaled by what the counter read for a plain copy of 256 MiB read + 256
# MiB written (FETCH_SIZE counted half the bytes read: x2; WRITE_SIZE all of them: x1).  Valid
# only for the kernel source the counters were taken on (sha256 of the files listed).
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC = {
    # kernel: (sha256 of its KERNEL_SOURCES concatenated, FETCH_SIZE KiB, WRITE_SIZE KiB)
    "attn_fwd_kernel": ("5191ac9713841e501c5ee88fc3313d0c516b3e2b02b8545f115dda5e5ce62863",
                        264250.1, 135189.8),
    "attn_bwd_dq_bf16_kernel": ("9b3a2dbb18ee6b36d70d6c4f61ee3603c2d3caf4f48283efa1afbd9614afda05",
                                435292.8, 143457.0),
    "attn_bwd_dkdv_bf16_kernel": ("9b3a2dbb18ee6b36d70d6c4f61ee3603c2d3caf4f48283efa1afbd9614afda05",
                                  267503.8, 262144.0),
}
KERNEL_SOURCES = {
    "attn_fwd_kernel": ["ra_fwd.hip", "ra_device.h"],
    "attn_bwd_dq_bf16_kernel": ["ra_bwd.hip", "ra_device.h"],
    "attn_bwd_dkdv_bf16_kernel": ["ra_bwd.hip", "ra_device.h"],
}
GQA = "bf16_causal_gqa_B4_Hq32_Hkv8_N4096_D128_rope"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["fwd_bwd", "fwd"], default="fwd_bwd")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-heads", type=int, default=3,
                    help="(batch, head) pairs of the workload the oracle times")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Attn:
    """Device-resident inputs/outputs of one workload and the C-ABI calls on them."""

    def __init__(self, ra, w, need_grad):
        import torch
        import workloads as wl
        self.ra, self.w = ra, w
        inp = wl.make_attention_inputs(w)
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

    def fwd(self):
        w = self.w
        st = self.ra.ra_attn_fwd(self.q, self.k, self.v, self.o, self.stats, w.B, w.Hq, w.Hkv,
                                 w.Nq, w.Nk, w.D, int(w.causal), w.scale, self.code, self.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_fwd: {self.ra.ra_status_string(st)}")

    def bwd(self):
        w = self.w
        st = self.ra.ra_attn_bwd(self.q, self.k, self.v, self.o, self.do, self.stats, self.dq,
                                 self.dk, self.dv, self.ws, self.ws_bytes, w.B, w.Hq, w.Hkv, w.Nq,
                                 w.Nk, w.D, int(w.causal), w.scale, self.code, self.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_bwd: {self.ra.ra_status_string(st)}")

    def fwd_masked(self, mask, causal=None):
        w = self.w
        cc = int(w.causal) if causal is None else causal
        st = self.ra.ra_attn_fwd_masked(self.q, self.k, self.v, self.o, self.stats, w.B, w.Hq,
                                        w.Hkv, w.Nq, w.Nk, w.D, cc, w.scale, self.code,
                                        *mask, self.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_fwd_masked: {self.ra.ra_status_string(st)}")

    def bwd_masked(self, mask):
        w = self.w
        st = self.ra.ra_attn_bwd_masked(self.q, self.k, self.v, self.o, self.do, self.stats,
                                        self.dq, self.dk, self.dv, self.ws, self.ws_bytes, w.B,
                                        w.Hq, w.Hkv, w.Nq, w.Nk, w.D, int(w.causal), w.scale,
                                        self.code, *mask, self.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_bwd_masked: {self.ra.ra_status_string(st)}")

    def bwd_dq(self):
        w = self.w
        st = self.ra.ra_attn_bwd_dq(self.q, self.k, self.v, self.o, self.do, self.stats, self.dq,
                                    self.ws, self.ws_bytes, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D,
                                    int(w.causal), w.scale, self.code, self.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_bwd_dq: {self.ra.ra_status_string(st)}")

    def bwd_dkdv(self):
        w = self.w
        st = self.ra.ra_attn_bwd_dkdv(self.q, self.k, self.v, self.do, self.stats, self.dk, self.dv,
                                      self.ws, self.ws_bytes, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D,
                                      int(w.causal), w.scale, self.code, self.stream)
        if st != 0:
            raise RuntimeError(f"ra_attn_bwd_dkdv: {self.ra.ra_status_string(st)}")


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


def time_calls(stream, fn, n):
    """Average duration (ms) of fn() over n calls, from HIP events recorded on `stream`."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for i in range(n):
        ev[2 * i].record(stream)
        fn()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]))


def cpu_baseline(w, heads, mode):
    """The fp64 oracle on `heads` (batch, head) pairs of workload w (bounded sample)."""
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    except Exception:                      # pragma: no cover
        cores = os.cpu_count() or 1
    import workloads as wl
    sub = wl.AttnWorkload(w.name + "_sample", w.dtype, w.causal, 1, heads, heads, w.Nq, w.Nk,
                          w.D, seed=w.seed, with_grad=True)
    inp = wl.make_attention_inputs(sub)
    t0 = time.perf_counter()
    oracle.ra_attention_fwd(inp["q"], inp["k"], inp["v"], w.causal, w.scale)
    if mode == "fwd_bwd":
        oracle.ra_attention_bwd(inp["q"], inp["k"], inp["v"], inp["do"], w.causal, w.scale)
    dt = time.perf_counter() - t0
    flops = sub.counted_flops_fwd_bwd() if mode == "fwd_bwd" else sub.counted_flops_fwd()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.Hq} (batch, head) pairs of {w.name}, "
                      f"{'forward+backward' if mode == 'fwd_bwd' else 'forward'}, fp64 NumPy, "
                      f"{dt:.1f} s", "seconds": dt}


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
    dev = torch.cuda.get_device_properties(0)
    log(f"device {dev.name} CUs={dev.multi_processor_count} arch={getattr(dev, 'gcnArchName', '?')}")

    if args.copy_calibration:
        # a plain copy kernel of known size: 256 MiB read + 256 MiB written
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 268435456 bytes read, 268435456 bytes written")
        del src, dst

    w = wl.WORKLOADS[MAIN]
    need_grad = args.mode == "fwd_bwd"
    log(f"generating {w.name}")
    main_run = Attn(ra, w, need_grad)
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
    value = flops_step / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms ({wall:.2f} s wall for {args.steps} steps): {value:.1f} TFLOP/s")

    # per-entry-point durations over the same kind of calls
    n_k = max(5, args.steps)
    fwd_ms = time_calls(stream, main_run.fwd, n_k)
    fwd_tflops = w.counted_flops_fwd() / (fwd_ms * 1e-3) / 1e12
    log(f"forward {fwd_ms:.3f} ms: {fwd_tflops:.1f} TFLOP/s")
    elems = w.B * w.Hq * w.Nq * w.Nk / (2 if w.causal else 1)   # visited score elements
    # (name, C entry point, ms per launch, algorithmic flops per launch)
    kernels = [("attn_fwd_kernel", "ra_attn_fwd", fwd_ms, 4 * w.D * elems)]
    bwd_ms = dq_ms = dkdv_ms = None
    if need_grad:
        bwd_ms = time_calls(stream, main_run.bwd, n_k)
        log(f"backward {bwd_ms:.3f} ms")
        dq_ms = time_calls(stream, main_run.bwd_dq, n_k)       # leaves the row terms in place
        dkdv_ms = time_calls(stream, main_run.bwd_dkdv, n_k)
        log(f"backward phases: dQ {dq_ms:.3f} ms, dK/dV {dkdv_ms:.3f} ms")
        kernels += [("attn_bwd_dq_bf16_kernel", "ra_attn_bwd_dq", dq_ms, 6 * w.D * elems),
                    ("attn_bwd_dkdv_bf16_kernel", "ra_attn_bwd_dkdv", dkdv_ms, 8 * w.D * elems)]
    del main_run
    torch.cuda.empty_cache()

    log(f"generating {GQA}")
    wg = wl.WORKLOADS[GQA]
    gqa = Attn(ra, wg, False)
    for _ in range(3):
        gqa.fwd()
    gqa_ms = time_calls(gqa.stream, gqa.fwd, n_k)
    gqa_tflops = wg.counted_flops_fwd() / (gqa_ms * 1e-3) / 1e12
    log(f"GQA forward {gqa_ms:.3f} ms: {gqa_tflops:.1f} TFLOP/s")
    # the same workload with the NEOX rotation of Q and K done on the device (in place; the
    # inputs are then rotated again each call, which changes values but not the work)
    def rope_qk():
        for t, H in ((gqa.q, wg.Hq), (gqa.k, wg.Hkv)):
            st = ra.ra_rope_neox(t, t, None, wg.B * H, wg.Nq, wg.D, 10000.0, False, gqa.code, gqa.stream)
            if st != 0:
                raise RuntimeError(f"ra_rope_neox: {ra.ra_status_string(st)}")
    for _ in range(3):
        rope_qk()
    rope_ms = time_calls(gqa.stream, rope_qk, n_k)
    rope_bytes = 2 * (gqa.q.numel() + gqa.k.numel()) * gqa.q.element_size()
    rope_gbs = rope_bytes / (rope_ms * 1e-3) / 1e9
    log(f"GQA device RoPE on Q and K {rope_ms:.3f} ms: {rope_gbs:.0f} GB/s; forward incl. RoPE "
        f"{gqa_ms + rope_ms:.3f} ms")
    del gqa
    torch.cuda.empty_cache()

    # explicit-mask path: a padded batch, key padding mask [B, N] (1 = attend) on top of causal
    wp = wl.padded_batch_workload()
    log(f"generating {wp.name}")
    pad = Attn(ra, wp, True)
    keep = torch.from_numpy(wl.padded_batch_keep(wp)).cuda()
    kpm = (keep, ra.RA_MASK_BOOL, (wp.Nk, 0, 0, 1))
    pad_masked = lambda: (pad.fwd_masked(kpm), pad.bwd_masked(kpm))
    pad_plain = lambda: (pad.fwd(), pad.bwd())
    for _ in range(3):
        pad_masked()
        pad_plain()
    pm_ms = time_calls(pad.stream, pad_masked, n_k)
    pp_ms = time_calls(pad.stream, pad_plain, n_k)
    pmf_ms = time_calls(pad.stream, lambda: pad.fwd_masked(kpm), n_k)
    pm_tflops = wp.counted_flops_fwd_bwd() / (pm_ms * 1e-3) / 1e12
    log(f"padded batch (key padding, causal) fwd+bwd {pm_ms:.3f} ms ({pm_tflops:.1f} TFLOP/s "
        f"counted as the unmasked causal workload), forward {pmf_ms:.3f} ms; unmasked {pp_ms:.3f} ms")
    del pad, keep
    torch.cuda.empty_cache()

    # split-KV decode: one query row per head against caches of per-sample lengths (HBM-bound)
    wd = wl.decode_workload()
    log(f"generating {wd.name}")
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
    for _ in range(3):
        decode_step()
    dec_ms = time_calls(dec.stream, decode_step, max(20, n_k))
    kv_bytes = int(lens_np.astype(np.int64).sum()) * wd.Hkv * wd.D * 2 * dec.q.element_size()
    dec_gbs = kv_bytes / (dec_ms * 1e-3) / 1e9
    # the same step through the tiled forward, the cache lengths as a key padding mask
    keep = torch.arange(wd.Nk, device="cuda")[None, :] < lens[:, None]
    kpm = (keep, ra.RA_MASK_BOOL, (wd.Nk, 0, 0, 1))
    br = ra.RA_CAUSAL_BOTTOM_RIGHT   # one query row: every key below the sample's length
    for _ in range(2):
        dec.fwd_masked(kpm, br)
    decf_ms = time_calls(dec.stream, lambda: dec.fwd_masked(kpm, br), n_k)
    log(f"decode {wd.name}: {dec_ms:.4f} ms, {dec_gbs:.0f} GB/s of K/V ({kv_bytes / 2**20:.0f} MiB); "
        f"tiled forward with the lengths as a mask {decf_ms:.4f} ms")
    del dec, dws, keep
    torch.cuda.empty_cache()

    # row softmax (HBM-bound): read + write once
    x = torch.from_numpy(wl.make_rows(16384, 8192, seed=11)).cuda()
    p = torch.empty_like(x)
    sm = lambda: ra.ra_softmax_rows(x, p, 16384, 8192, ra.RA_F32, stream)
    for _ in range(3):
        sm()
    sm_ms = time_calls(stream, sm, n_k)
    sm_gbs = 2 * x.numel() * 4 / (sm_ms * 1e-3) / 1e9
    log(f"softmax rows [16384, 8192] fp32 {sm_ms:.3f} ms: {sm_gbs:.0f} GB/s")
    # its backward (x and dp read, dx written once)
    g = torch.from_numpy(np.random.default_rng(12).standard_normal((16384, 8192), dtype=np.float32)).cuda()
    dx = torch.empty_like(x)
    smb = lambda: ra.ra_softmax_rows_bwd(x, g, dx, 16384, 8192, ra.RA_F32, stream)
    for _ in range(3):
        smb()
    smb_ms = time_calls(stream, smb, n_k)
    smb_gbs = 3 * x.numel() * 4 / (smb_ms * 1e-3) / 1e9
    log(f"softmax rows backward [16384, 8192] fp32 {smb_ms:.3f} ms: {smb_gbs:.0f} GB/s")
    del g, dx

    # dominant kernel: the longest launch of the step (one launch per entry-point call)
    dom_name, dom_call, dom_ms, dom_flops = max(kernels, key=lambda t: t[2])
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_bytes(dom_name), "kernel": f"{dom_name} ({dom_call})",
                "avg_launch_ms": round(dom_ms, 4),
                "flops_per_launch": dom_flops}
    kernel_table = {n: {"ms": round(t, 4), "tflops": round(f / (t * 1e-3) / 1e12, 2),
                        "traffic": traffic_bytes(n),
                        "frac_of_peak": round(f / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
                    for n, _, t, f in kernels}

    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on a bounded sample")
        cpu = cpu_baseline(w, args.cpu_heads, args.mode)
        log(f"oracle: {cpu['value']:.4f} TFLOP/s in {cpu['seconds']:.1f} s on {cpu['cores']} threads")
        cpu.pop("seconds")

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
                   "seq_len": w.Nq, "head_dim": w.D, "causal": w.causal, "global_batch": w.B},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"workload": w.name, "ms": round(fwd_ms, 4), "tflops": round(fwd_tflops, 2),
                "frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4)},
        "bwd_ms": None if bwd_ms is None else round(bwd_ms, 4),
        "kernels": kernel_table,
        "fwd_gqa": {"workload": wg.name, "ms": round(gqa_ms, 4), "tflops": round(gqa_tflops, 2),
                    "frac_of_peak": round(gqa_tflops / PEAK_BF16_TFLOPS, 4),
                    "device_rope_ms": round(rope_ms, 4), "device_rope_GB/s": round(rope_gbs, 1)},
        "masked_padded_batch": {"workload": wp.name, "lengths": list(wl.padded_batch_lengths(wp)),
                                "mask": "key padding [B, N] bool, causal top-left",
                                "fwd_bwd_ms": round(pm_ms, 4), "fwd_ms": round(pmf_ms, 4),
                                "tflops_counted": round(pm_tflops, 2),
                                "unmasked_fwd_bwd_ms": round(pp_ms, 4)},
        "decode": {"workload": wd.name, "entry": "ra_attn_decode", "ms": round(dec_ms, 4),
                   "kv_bytes": kv_bytes, "GB/s": round(dec_gbs, 1),
                   "frac_of_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "tiled_fwd_masked_ms": round(decf_ms, 4)},
        "softmax_rows": {"shape": [16384, 8192], "dtype": "f32", "ms": round(sm_ms, 4),
                         "GB/s": round(sm_gbs, 1), "frac_of_hbm_peak": round(sm_gbs / PEAK_HBM_GBS, 4)},
        "softmax_rows_bwd": {"shape": [16384, 8192], "dtype": "f32", "ms": round(smb_ms, 4),
                             "GB/s": round(smb_gbs, 1),
                             "frac_of_hbm_peak": round(smb_gbs / PEAK_HBM_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
