#!/usr/bin/env python3
"""EFLA chunked-forward benchmark on one MI355X.

One step = one efla_chunk_fwd pass (coefficients + UT transform + sequential
recurrence with the fused output) over the 1.3B-model-shaped layer:
B=4, H=16, L=4096, d_k=d_v=128, chunk=64, bf16 q/k/v/beta/o, fp32 states.
Inputs are synthetic and seeded, resident in HBM before timing starts.

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      the dominant kernel (the recurrence) against the HBM peak,
                from HIP events recorded around it inside the timed loop
  stages        per-stage event times and the whole-path fraction of peak
  decode        efla_step at [256, 16, 128, 128] (fp32 state), back to back
  euler         the same path under the Euler (delta-rule) update, alpha = beta,
                timed the same way: the pages' throughput comparison of the two
  varlen        efla_chunk_fwd_varlen on the same 16384 tokens and 16 heads packed
                as 16 sequences of mixed length (varlen_1p3b)
  backward      efla_chunk_bwd on the benchmark workload (gradients of q, k, v,
                beta and the initial state), and forward + backward together
  segmented     the stiff long-context workload (B=1, H=16, L=65536): the plain
                chunked pass against efla_chunk_fwd_segmented
  cpu_baseline  the fp64 oracle on the same workload, on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EFLA chunked-fwd tokens/s at H=16,d=128,L=4096; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "delta_rule_sequence_efla_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "recurrence_shape_1p3b_traffic.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "efla_fwd_shape_1p3b_kernel_trace.txt")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="shape_1p3b")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-euler", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-segmented", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--event-every", type=int, default=8,
                    help="record per-kernel HIP events on one timed step in this many")
    ap.add_argument("--cold-iters", type=int, default=10,
                    help="extra iterations each preceded by a 1 GiB cache-flushing write")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (HBM counter calibration under rocprofv3)")
    return ap.parse_args()


# The sources the forward kernels (UT transform and recurrence) and their
# launches are built from.
FWD_SOURCES = ("api.hip", "common.h", "launchers.h", "lds_ring.h", "recurrence_roles.h", "chunk_bf16_roles.hip",
               "ut_wave.h", "ut_bf16.hip")


def kernel_source_hash() -> str:
    """Hash of the forward kernels' sources: the counter summary is only used
    while it matches the code it was taken on."""
    h = hashlib.sha256()
    for name in sorted(FWD_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_traffic(per_launch_units: dict):
    """HBM bytes per recurrence launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_trace_avg_us(kernel: str):
    """Average duration of `kernel` in the committed rocprofv3 kernel-trace
    summary of this benchmark, or None when missing or taken on different
    kernel sources.  Reported beside the live event timing, which also counts
    the launch latency each bracketing event pair adds."""
    if not os.path.exists(TRACE_FILE):
        return None
    lines = open(TRACE_FILE).read().splitlines()
    if not any(kernel_source_hash() in ln for ln in lines if ln.startswith("#")):
        return None
    for ln in lines:
        parts = ln.split()
        if parts and not ln.startswith("#") and parts[0].startswith("efla::" + kernel + "<"):
            try:
                return float(parts[-4])   # columns: name.. calls avg min max pct
            except ValueError:
                return None
    return None


def pct(xs, p):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the EFLA hot path "
              "shards over (batch, head) with no exchange between GPUs, so N GPUs each run this "
              "single-GPU workload on their share.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from delta_rule_sequence_efla_amd import efla
    from delta_rule_sequence_efla_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.get(args.workload)
    print(f"[bench] generating {w.name}: B={w.B} H={w.H} L={w.L} d={w.dk}/{w.dv} C={w.chunk}",
          file=sys.stderr, flush=True)
    inp = W.generate(w, device=dev)
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    o = torch.empty((w.B, w.L, w.H, w.dv), dtype=q.dtype, device=dev)
    s_final = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = efla.alloc_workspace(w.B, w.H, w.L, w.dk, w.dv, w.chunk, q.dtype, dev)
    ut, rec = efla.prepare_chunk_stages(q, k, v, beta, s0, o, s_final, ws, chunk=w.chunk)
    rec_kernel = efla.efla_chunk_recurrence_kernel(w.dk, w.dv, w.chunk, q.dtype)

    esz = q.element_size()
    n_ht = w.B * w.H * w.L
    nc = (w.L + w.chunk - 1) // w.chunk
    state_bytes = w.B * w.H * w.dk * w.dv * 4
    t_bytes = w.B * w.H * nc * w.chunk * w.chunk * esz
    # algorithmic bytes: what each stage must read and write once
    path_bytes = n_ht * ((2 * w.dk + 2 * w.dv) * esz + esz) + (state_bytes if s0 is not None else 0) \
        + state_bytes
    rec_bytes = n_ht * (2 * w.dk + 2 * w.dv) * esz + t_bytes + \
        (state_bytes if s0 is not None else 0) + state_bytes
    ut_bytes = n_ht * (w.dk + 1) * esz + t_bytes
    path_flops = n_ht * (6 * w.dk * w.dv + 5 * w.chunk * max(w.dk, w.dv) + w.chunk ** 2 // 3)

    for _ in range(args.warmup):
        ut()
        rec()
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps.  Every E-th step is bracketed by
    # HIP events around each kernel (on the launch stream), which gives the
    # per-kernel durations; an event between two launches keeps them from
    # overlapping, so only a sample of the steps carries them.
    K, E = args.steps, max(1, args.event_every)
    sampled = list(range(0, K, E))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if i in ev:
            ev[i][0].record()
            ut()
            ev[i][1].record()
            rec()
            ev[i][2].record()
        else:
            ut()
            rec()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    ut_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in sampled]
    rec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in sampled]
    path_ms = [ev[i][0].elapsed_time(ev[i][2]) for i in sampled]
    rec_avg = sum(rec_ms) / len(sampled)
    ut_avg = sum(ut_ms) / len(sampled)
    path_avg = sum(path_ms) / len(sampled)

    tokens = w.B * w.L
    value = tokens / (ms_per_step / 1e3)
    achieved = rec_bytes / (rec_avg / 1e3) / 1e9
    traffic = read_traffic({})

    # cold-cache iterations: a 1 GiB write evicts L2 and the Infinity Cache first
    cold = None
    if args.cold_iters > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cms = []
        for _ in range(args.cold_iters):
            flush.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ut()
            rec()
            b.record()
            torch.cuda.synchronize()
            cms.append(a.elapsed_time(b))
        del flush
        cold = {"median_us": round(pct(cms, 50) * 1e3, 2), "p10_us": round(pct(cms, 10) * 1e3, 2),
                "p90_us": round(pct(cms, 90) * 1e3, 2),
                "tokens_per_s": round(tokens / (pct(cms, 50) / 1e3), 1)}

    if args.copy_calibration:
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    euler = None
    if not args.no_euler:
        eut, erec = efla.prepare_chunk_stages(q, k, v, beta, s0, o, s_final, ws, chunk=w.chunk, rule="euler")
        for _ in range(args.warmup):
            eut()
            erec()
        torch.cuda.synchronize()

        def loop_us(stages):
            # K back-to-back passes between two events, no events in between
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(K):
                for f in stages:
                    f()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / K

        xus, eus = loop_us((ut, rec)), loop_us((eut, erec))
        euler = {"rule": "euler (alpha = beta)", "path_us": round(eus, 2),
                 "tokens_per_s": round(tokens / (eus / 1e6), 1),
                 "exact_path_us_same_loop": round(xus, 2),
                 "exact_over_euler_time": round(xus / eus, 4)}

    varlen = None
    if not args.no_varlen:
        wv = W.get("varlen_1p3b")
        lengths = W.length_mix(wv.B, wv.L, seed=wv.seed)
        pv = W.generate_packed(wv, lengths, device=dev)
        ov = torch.empty_like(pv["v"])
        sv = torch.empty((wv.B, wv.H, wv.dk, wv.dv), dtype=torch.float32, device=dev)
        wsv = torch.empty(max(1, efla.efla_chunk_fwd_varlen_workspace_size(wv.B, wv.H, wv.L, wv.dk, wv.dv,
                                                                           wv.chunk, pv["q"].dtype)),
                          dtype=torch.uint8, device=dev)
        fv = efla.prepare_chunk_fwd_varlen(pv["q"], pv["k"], pv["v"], pv["beta"], pv["cu_seqlens"], pv["s0"],
                                           ov, sv, wsv, chunk=wv.chunk)
        for _ in range(args.warmup):
            fv()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            fv()
        b.record()
        torch.cuda.synchronize()
        vus = a.elapsed_time(b) * 1e3 / K
        varlen = {"workload": wv.name, "sequences": wv.B, "tokens": wv.L, "H": wv.H,
                  "lengths_min_median_max": [min(lengths), sorted(lengths)[len(lengths) // 2], max(lengths)],
                  "path_us": round(vus, 2), "tokens_per_s": round(wv.L / (vus / 1e6), 1),
                  "note": "back-to-back calls; the longest sequence bounds the sequential pass"}
        del pv, ov, sv, wsv, fv

    backward = None
    if not args.no_backward:
        g = torch.Generator(device="cpu").manual_seed(7)
        d_o = torch.randn(o.shape, generator=g).to(q.dtype).to(dev)
        dsf = torch.randn(s_final.shape, generator=g).to(dev)
        gq, gk, gv, gb = (torch.empty_like(x) for x in (q, k, v, beta))
        gs0 = torch.empty_like(s_final)
        nb = efla.efla_chunk_bwd_workspace_size(w.B, w.H, w.L, w.dk, w.dv, w.chunk, q.dtype)
        wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        bwd = efla.prepare_chunk_bwd(q, k, v, beta, d_o, s0, dsf, gq, gk, gv, gb, gs0, wsb, chunk=w.chunk)
        bwd()
        torch.cuda.synchronize()
        KB = max(1, args.backward_steps)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(KB):
            bwd()
        b.record()
        torch.cuda.synchronize()
        bus = a.elapsed_time(b) * 1e3 / KB
        # bytes the backward must move: q, k, v, beta, d_o read; dq, dk, dv, dbeta written; states in/out
        bwd_bytes = n_ht * ((2 * w.dk + 2 * w.dv + 1) * esz + (2 * w.dk + w.dv + 1) * esz) + 3 * state_bytes
        backward = {"us": round(bus, 2), "tokens_per_s": round(tokens / (bus / 1e6), 1),
                    "algorithmic_bytes": bwd_bytes,
                    "hbm_frac": round(bwd_bytes / (bus / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                    "workspace_bytes": nb,
                    "fwd_plus_bwd_tokens_per_s": round(tokens / ((bus + ms_per_step * 1e3) / 1e6), 1)}
        del wsb, gq, gk, gv, gb, gs0, d_o, dsf, bwd

    segmented = None
    if not args.no_segmented:
        wl = W.get("stiff_64k")
        li = W.generate(wl, device=dev)
        ol = torch.empty_like(li["v"])
        sl = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
        segs = efla.default_segments(wl.B, wl.H, wl.L, wl.dv, wl.chunk)
        wsp = efla.alloc_workspace(wl.B, wl.H, wl.L, wl.dk, wl.dv, wl.chunk, li["q"].dtype, dev)
        nsg = efla.efla_chunk_fwd_segmented_workspace_size(wl.B, wl.H, wl.L, wl.dk, wl.dv, wl.chunk, segs,
                                                           li["q"].dtype)
        wss = torch.empty(max(nsg, 1), dtype=torch.uint8, device=dev)
        plain = efla.prepare_chunk_fwd(li["q"], li["k"], li["v"], li["beta"], li["s0"], ol, sl, wsp, chunk=wl.chunk)
        seg = efla.prepare_chunk_fwd_segmented(li["q"], li["k"], li["v"], li["beta"], li["s0"], ol, sl, wss,
                                               chunk=wl.chunk, segments=segs)

        def time_us(f, n=5):
            f()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                f()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / n

        pus, sus = time_us(plain), time_us(seg)
        segmented = {"workload": wl.name, "segments": segs, "plain_us": round(pus, 1), "segmented_us": round(sus, 1),
                     "plain_tokens_per_s": round(wl.tokens / (pus / 1e6), 1),
                     "segmented_tokens_per_s": round(wl.tokens / (sus / 1e6), 1),
                     "speedup": round(pus / sus, 3)}
        del li, ol, sl, wsp, wss, plain, seg

    decode = None
    if not args.no_decode:
        wd = W.get("decode_1p3b")
        dinp = W.generate_decode(wd, device=dev, steps=1)
        state = dinp["s0"].clone()
        od = torch.empty((wd.B, wd.H, wd.dv), dtype=q.dtype, device=dev)
        stp = efla.prepare_step(dinp["q"][0], dinp["k"][0], dinp["v"][0], dinp["beta"][0], state, od)
        for _ in range(3):
            stp()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.decode_steps):
            stp()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.decode_steps
        heads = wd.B * wd.H
        dbytes = heads * (2 * wd.dk * wd.dv * 4 + (2 * wd.dk + 2 * wd.dv + 1) * esz)
        decode = {"workload": "decode_1p3b", "N": wd.B, "H": wd.H, "d": wd.dk, "us_per_step": round(us, 2),
                  "tokens_per_s": round(wd.B / (us / 1e6), 1),
                  "roofline": {"bound": "hbm", "achieved": round(dbytes / (us / 1e6) / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(dbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                               "traffic": None},
                  "note": "back-to-back steps on the same resident state"}
        del state, dinp

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from delta_rule_sequence_efla_amd.workloads import to_f64
        cores = oracle.default_threads()
        threads = min(cores, w.B * w.H)
        qa, ka, va, ba, sa = (to_f64(x) for x in (q, k, v, beta, s0))
        # whole passes over the workload until about 15 s of CPU time (1 to 8 passes)
        passes, wall, cpu_s = 0, 0.0, 0.0
        while passes < 8 and (passes == 0 or cpu_s < 15.0):
            t, c = time.perf_counter(), time.process_time()
            oracle.forward(qa, ka, va, ba, sa, nthreads=threads)
            wall += time.perf_counter() - t
            cpu_s += time.process_time() - c
            passes += 1
        cpu = {"value": round(tokens * passes / wall, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole {w.name} workload ({w.B * w.H} sequences x {w.L} tokens), "
                         f"fp64 token-by-token recurrence, {passes} passes, {wall:.2f} s wall, "
                         f"{cpu_s:.1f} s of CPU time"}

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d_k": w.dk, "d_v": w.dv,
                   "chunk": w.chunk, "state": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": rec_kernel, "avg_us": round(rec_avg * 1e3, 2), "event_samples": len(sampled),
                     "algorithmic_bytes": rec_bytes, "trace_avg_us": read_trace_avg_us(rec_kernel)},
        "stages": {"ut_transform_us": round(ut_avg * 1e3, 2), "ut_transform_bytes": ut_bytes,
                   "recurrence_us": round(rec_avg * 1e3, 2),
                   "path_us_events": round(path_avg * 1e3, 2), "path_algorithmic_bytes": path_bytes,
                   "path_hbm_frac": round(path_bytes / (path_avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "path_mfma_frac": round(path_flops / (path_avg / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                   "head_tokens_per_s": round(n_ht / (ms_per_step / 1e3), 1)},
        "cold": cold,
        "decode": decode,
        "euler": euler,
        "varlen": varlen,
        "backward": backward,
        "segmented": segmented,
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
