#!/usr/bin/env python3
"""EFLA chunked-forward benchmark on one MI355X.

One step = one efla_chunk_fwd pass (coefficients + UT transform + sequential
recurrence with the fused output) over the 1.3B-model-shaped layer:
B=4, H=16, L=4096, d_k=d_v=128, chunk=64, bf16 q/k/v/beta/o, fp32 states.
Inputs are synthetic and seeded, resident in HBM before timing starts.

Timing protocol (the headline): every timed step is preceded by a cache
flush -- a 1 GiB write, then a 1 GiB read of another buffer, so that the L2s
and the 256 MB Infinity Cache hold clean lines of unrelated data and the
step's inputs come from HBM -- and is bracketed by HIP events on the launch
stream.  `value` and `ms_per_step` come from the median step; p10/p90 are
reported beside it.  The flush is enqueued before the step's events and
kernels, so the host's launch latency stays outside the timed interval.

Besides the contract fields the JSON line carries:
  roofline      the dominant kernel (the recurrence) against the HBM peak:
                its algorithmic bytes (q, k, v read, o written, states in and
                out, once) over its flushed event time
  path          the whole step (both kernels) against the same peak, and the
                bytes each stage moves beyond the algorithmic ones
  stream        flushed 1 GiB read + write passes (device copy, in-place
                scale): the measured bandwidth ceiling, with the recurrence's
                and the path's fractions of it
  warm          the same step back to back with no flush (caches warm)
  dirty_flush   the step after a write-only flush (dirty lines left in the
                caches, whose write-back then competes with the step)
  shapes        the flushed step on the other model-shaped workloads
  decode        efla_step at [256, 16, 128, 128] (fp32 state), flushed per step
  training      forward + backward per step under the exact rule and under
                the Euler (delta-rule) rule, the pages' throughput comparison;
                also the training pair (forward storing the chunk states, the
                backward reading them)
  euler         the forward alone under the Euler rule
  varlen        efla_chunk_fwd_varlen on the same heads packed as 16 sequences
  backward      efla_chunk_bwd on the benchmark workload
  segmented     the stiff long-context workload (B=1, H=16, L=65536): the
                plain chunked pass against efla_chunk_fwd_segmented
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
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "efla_fwd_shape_1p3b_traffic.txt")
TRACE_FILE = os.path.join(PROFILES, "efla_fwd_shape_1p3b_kernel_trace.txt")
FLUSH_BYTES = 1 << 30


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="flushed, timed steps (median reported)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="shape_1p3b")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--profile", choices=("fwd", "decode", "segmented", "training"), default=None,
                    help="only the flushed forward steps (or the decode, segment-scan or training leg), "
                         "for rocprofv3 runs of the same kernels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every leg after the headline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (HBM counter calibration under rocprofv3)")
    return ap.parse_args()


# The sources the profiled kernels (UT transform, split recurrence, decode
# step) and their launch functions are built from.  Declarations and the
# other entry points (api.hip, launchers.h) change no kernel code and are left
# out, so that a summary stays valid until one of these kernels changes.
FWD_SOURCES = ("common.h", "lds_ring.h", "recurrence_split.h", "chunk_bf16_split.hip",
               "ut_wave.h", "ut_bf16.hip", "step_kernels.hip")


def kernel_source_hash() -> str:
    """Hash of the forward kernels' sources: a counter summary is only used
    while it matches the code it was taken on."""
    h = hashlib.sha256()
    for name in sorted(FWD_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _kv(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    return kv


def read_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = _kv(TRAFFIC_FILE)
    if kv.get("source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(kv[f"{kernel}.hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_trace_avg_us(kernel: str):
    """Average duration of `kernel` in the committed rocprofv3 kernel-trace
    summary of `bench.py --profile`, or None when missing or taken on other
    sources.  Reported beside the live event timing."""
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


def stats_us(ms_list):
    return {"median_us": round(pct(ms_list, 50) * 1e3, 2), "p10_us": round(pct(ms_list, 10) * 1e3, 2),
            "p90_us": round(pct(ms_list, 90) * 1e3, 2), "samples": len(ms_list)}


class Flusher:
    """Leaves the L2s and the Infinity Cache holding clean, unrelated lines:
    a 1 GiB write, then a 1 GiB read of a second buffer (its lines evict the
    written ones, whose write-back happens here and not in the timed step)."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.w = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.r = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((), dtype=torch.float32, device=dev)

    def clean(self):
        self.w.fill_(1.0)
        self.torch.sum(self.r, dim=0, out=self.out)

    def dirty(self):
        self.w.fill_(2.0)


def flushed_steps(torch, fns, n, flush, marks=False):
    """n steps, each preceded by flush(); events around the whole step (and,
    with marks, between its calls).  Returns per-step lists of ms."""
    Ev = torch.cuda.Event
    evs = []
    torch.cuda.synchronize()
    for _ in range(n):
        flush()
        e = [Ev(enable_timing=True) for _ in range(len(fns) + 1 if marks else 2)]
        e[0].record()
        for i, f in enumerate(fns):
            f()
            if marks and i + 1 < len(fns):
                e[i + 1].record()
        e[-1].record()
        evs.append(e)
    torch.cuda.synchronize()
    whole = [e[0].elapsed_time(e[-1]) for e in evs]
    parts = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(len(fns))] if marks else None
    return whole, parts


def warm_us(torch, fns, n):
    """n steps back to back between two events: microseconds per step."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        for f in fns:
            f()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def decode_leg(torch, efla, W, fl, dev, dtype, args, esz):
    """efla_step at the 1.3B decode shape, a flush before every step."""
    wd = W.get("decode_1p3b")
    dinp = W.generate_decode(wd, device=dev, steps=1)
    state = dinp["s0"].clone()
    od = torch.empty((wd.B, wd.H, wd.dv), dtype=dtype, device=dev)
    stp = efla.prepare_step(dinp["q"][0], dinp["k"][0], dinp["v"][0], dinp["beta"][0], state, od)
    for _ in range(3):
        stp()
    dms, _ = flushed_steps(torch, (stp,), max(args.decode_steps, 20), fl.clean)
    dus = pct(dms, 50) * 1e3
    dw = warm_us(torch, (stp,), args.decode_steps)
    dbytes = wd.B * wd.H * (2 * wd.dk * wd.dv * 4 + (2 * wd.dk + 2 * wd.dv + 1) * esz)
    return {
        "workload": "decode_1p3b", "N": wd.B, "H": wd.H, "d": wd.dk, "flushed": stats_us(dms),
        "us_per_step": round(dus, 2), "tokens_per_s": round(wd.B / (dus / 1e6), 1),
        "roofline": {"bound": "hbm", "achieved": round(dbytes / (dus / 1e6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dbytes / (dus / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("step_kernel"), "kernel": "step_kernel",
                     "algorithmic_bytes": dbytes, "trace_avg_us": read_trace_avg_us("step_kernel")},
        "warm_us_per_step": round(dw, 2),
        "note": "flushed: a cache flush before every step; warm: back to back on the resident 256 MiB state"}


def training_leg(torch, efla, w, inp, o, s_final, ws, dev, K, args, rules=("exact", "euler")):
    """Forward + backward per step, back to back, under each rule."""
    q, k, v, beta, s0 = inp["q"], inp["k"], inp["v"], inp["beta"], inp["s0"]
    tokens = w.B * w.L
    g = torch.Generator(device="cpu").manual_seed(7)
    d_o = torch.randn(o.shape, generator=g).to(q.dtype).to(dev)
    dsf = torch.randn(s_final.shape, generator=g).to(dev)
    gq, gk, gv, gb = (torch.empty_like(x) for x in (q, k, v, beta))
    gs0 = torch.empty_like(s_final)
    nb = efla.efla_chunk_bwd_workspace_size(w.B, w.H, w.L, w.dk, w.dv, w.chunk, q.dtype)
    wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    train = {}
    for rule in rules:
        fwd = efla.prepare_chunk_fwd(q, k, v, beta, s0, o, s_final, ws, chunk=w.chunk, rule=rule)
        bwd = efla.prepare_chunk_bwd(q, k, v, beta, d_o, s0, dsf, gq, gk, gv, gb, gs0, wsb, chunk=w.chunk,
                                     rule=rule)
        fwd()
        bwd()
        KB = max(1, args.backward_steps)
        fus = warm_us(torch, (fwd,), K)
        bus = warm_us(torch, (bwd,), KB)
        tus = warm_us(torch, (fwd, bwd), KB)
        train[rule] = {"fwd_us": round(fus, 2), "bwd_us": round(bus, 2), "fwd_bwd_us": round(tus, 2),
                       "fwd_bwd_tokens_per_s": round(tokens / (tus / 1e6), 1)}
        # the training pair: the forward stores the chunk start states, the
        # backward reads them (its state pass skipped)
        tf, tb = efla.prepare_chunk_train(q, k, v, beta, d_o, s0, o, s_final, dsf, gq, gk, gv, gb, gs0, wsb,
                                          chunk=w.chunk, rule=rule)
        tf()
        tb()
        pfus = warm_us(torch, (tf,), K)
        pbus = warm_us(torch, (tb,), KB)
        ptus = warm_us(torch, (tf, tb), KB)
        train[rule]["pair"] = {"fwd_us": round(pfus, 2), "bwd_us": round(pbus, 2), "fwd_bwd_us": round(ptus, 2),
                               "fwd_bwd_tokens_per_s": round(tokens / (ptus / 1e6), 1),
                               "states_stored": efla.efla_chunk_train_saves_states(w.dk, w.dv, w.chunk, q.dtype)}
    if "exact" in train and "euler" in train:
        train["exact_over_euler_time"] = round(train["exact"]["fwd_bwd_us"] / train["euler"]["fwd_bwd_us"], 4)
        train["pair_exact_over_euler_time"] = round(train["exact"]["pair"]["fwd_bwd_us"] /
                                                    train["euler"]["pair"]["fwd_bwd_us"], 4)
    train["note"] = ("back-to-back steps; efla_chunk_fwd + efla_chunk_bwd, and under 'pair' "
                     "efla_chunk_fwd_train + efla_chunk_bwd_train; the pages report EFLA training throughput "
                     "matching DeltaNet's (Experimental Results), with no hardware or numbers given")
    return train, nb


def segmented_leg(torch, efla, W, fl, dev):
    """The stiff long-context workload: the plain chunked pass against the
    segment scan, flushed steps."""
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
    plain()
    seg()
    pms, _ = flushed_steps(torch, (plain,), 10, fl.clean)
    sms, _ = flushed_steps(torch, (seg,), 10, fl.clean)
    pus, sus = pct(pms, 50) * 1e3, pct(sms, 50) * 1e3
    return {"workload": wl.name, "segments": segs, "plain": stats_us(pms), "segmented": stats_us(sms),
            "plain_tokens_per_s": round(wl.tokens / (pus / 1e6), 1),
            "segmented_tokens_per_s": round(wl.tokens / (sus / 1e6), 1), "speedup": round(pus / sus, 3)}


def fwd_bytes(w, esz, with_s0=True):
    """Algorithmic bytes of one forward pass: q, k, v, beta read and o written
    once, plus the fp32 states in (if given) and out."""
    n_ht = w.B * w.H * w.L
    state = w.B * w.H * w.dk * w.dv * 4
    return n_ht * ((2 * w.dk + 2 * w.dv + 1) * esz) + (state if with_s0 else 0) + state


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
    fl = Flusher(torch, dev)

    esz = q.element_size()
    n_ht = w.B * w.H * w.L
    tokens = w.B * w.L
    nc = (w.L + w.chunk - 1) // w.chunk
    state_bytes = w.B * w.H * w.dk * w.dv * 4
    t_bytes = w.B * w.H * nc * w.chunk * w.chunk * esz
    path_bytes = fwd_bytes(w, esz, s0 is not None)
    # the recurrence's share of the algorithmic bytes: q, k, v, o and the states
    rec_bytes = n_ht * (2 * w.dk + 2 * w.dv) * esz + (state_bytes if s0 is not None else 0) + state_bytes
    path_flops = n_ht * (6 * w.dk * w.dv + 5 * w.chunk * max(w.dk, w.dv) + w.chunk ** 2 // 3)

    if args.copy_calibration:  # a device copy of known size, for the HBM counters under rocprofv3
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.profile == "decode":
        print(json.dumps({"decode": decode_leg(torch, efla, W, fl, dev, q.dtype, args, esz)}), flush=True)
        return
    if args.profile == "segmented":
        print(json.dumps({"segmented": segmented_leg(torch, efla, W, fl, dev)}), flush=True)
        return
    if args.profile == "training":
        train, _ = training_leg(torch, efla, w, inp, o, s_final, ws, dev, max(1, args.steps), args)
        print(json.dumps({"training": train}), flush=True)
        return
    for _ in range(args.warmup):
        ut()
        rec()
    torch.cuda.synchronize()

    # ---- headline: K flushed steps, median --------------------------------
    K = max(1, args.steps)
    t0 = time.perf_counter()
    path_ms, _ = flushed_steps(torch, (ut, rec), K, fl.clean)
    wall = time.perf_counter() - t0
    # the same steps with an event between the two kernels: per-kernel times
    _, parts = flushed_steps(torch, (ut, rec), K, fl.clean, marks=True)
    ut_ms, rec_ms = parts
    med_ms = pct(path_ms, 50)
    value = tokens / (med_ms / 1e3)
    rec_med_ms = pct(rec_ms, 50)
    achieved = rec_bytes / (rec_med_ms / 1e3) / 1e9

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d_k": w.dk, "d_v": w.dv,
                   "chunk": w.chunk, "state": "fp32", "parallelism": "single GPU",
                   "timing": "median of flushed steps (1 GiB write + 1 GiB read before each), HIP events"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(rec_kernel),
                     "kernel": rec_kernel, "avg_us": round(sum(rec_ms) / len(rec_ms) * 1e3, 2),
                     "median_us": round(rec_med_ms * 1e3, 2), "algorithmic_bytes": rec_bytes,
                     "trace_avg_us": read_trace_avg_us(rec_kernel)},
        "path": {"flushed": stats_us(path_ms), "algorithmic_bytes": path_bytes,
                 "hbm_frac": round(path_bytes / (med_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(path_flops / (med_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                 "ut_transform": stats_us(ut_ms), "recurrence": stats_us(rec_ms),
                 "overhead_bytes": {"T_workspace_write_and_read": 2 * t_bytes, "k_reread": n_ht * w.dk * esz},
                 "head_tokens_per_s": round(n_ht / (med_ms / 1e3), 1),
                 "wall_s_with_flushes": round(wall, 4)},
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if args.profile:
        print(json.dumps(line), flush=True)
        return
    extras = not args.no_extras

    # ---- the measured bandwidth: the secondary ceiling ----------------------
    # 1 GiB read and written once (the runtime's device copy; an in-place scale
    # by torch's elementwise kernel), flushed like the steps; the faster sets
    # the measured ceiling, the spec 8 TB/s stays the primary peak
    sa = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sb = torch.empty_like(sa)
    stream = {}
    for sname, sfn in (("copy", lambda: sb.copy_(sa)), ("scale_in_place", lambda: sa.mul_(1.0))):
        for _ in range(3):
            sfn()
        sms, _ = flushed_steps(torch, (sfn,), 10, fl.clean)
        stream[sname] = dict(stats_us(sms), GBps=round(2 * 4 * sa.numel() / (pct(sms, 50) / 1e3) / 1e9, 1))
    del sa, sb
    ceiling = max(s["GBps"] for s in stream.values())
    line["stream"] = dict(stream, bytes=2 * 4 * (1 << 28), ceiling_GBps=ceiling,
                          note="1 GiB read + 1 GiB written, a flush before each of ten; median")
    line["roofline"]["frac_of_measured"] = round(achieved / ceiling, 4)
    line["path"]["hbm_frac_of_measured"] = round(path_bytes / (med_ms / 1e3) / 1e9 / ceiling, 4)

    # ---- warm and dirty-flush references ----------------------------------
    wus = warm_us(torch, (ut, rec), K)
    line["warm"] = {"path_us": round(wus, 2), "tokens_per_s": round(tokens / (wus / 1e6), 1),
                    "hbm_frac": round(path_bytes / (wus / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                    "note": "back to back, caches warm (the 277 MB working set against a 256 MB Infinity Cache)"}
    dms, _ = flushed_steps(torch, (ut, rec), K, fl.dirty)
    line["dirty_flush"] = dict(stats_us(dms), note="write-only flush: the step competes with its write-back")

    if extras:
        # ---- the other model-shaped workloads ----------------------------
        shapes = {}
        for name in ("small_bf16", "shape_340m"):
            ws_ = W.get(name)
            li = W.generate(ws_, device=dev)
            ol = torch.empty_like(li["v"])
            sl = torch.empty((ws_.B, ws_.H, ws_.dk, ws_.dv), dtype=torch.float32, device=dev)
            wsp = efla.alloc_workspace(ws_.B, ws_.H, ws_.L, ws_.dk, ws_.dv, ws_.chunk, li["q"].dtype, dev)
            f = efla.prepare_chunk_fwd(li["q"], li["k"], li["v"], li["beta"], li["s0"], ol, sl, wsp,
                                       chunk=ws_.chunk)
            for _ in range(3):
                f()
            ms, _ = flushed_steps(torch, (f,), K, fl.clean)
            b = fwd_bytes(ws_, li["q"].element_size(), li["s0"] is not None)
            m = pct(ms, 50)
            shapes[name] = dict(stats_us(ms), B=ws_.B, H=ws_.H, L=ws_.L, d=ws_.dk,
                                tokens_per_s=round(ws_.tokens / (m / 1e3), 1), algorithmic_bytes=b,
                                hbm_frac=round(b / (m / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                warm_us=round(warm_us(torch, (f,), K), 2))
            # too few (b, h, value block) workgroups for the compute units: the
            # segment scan on the same inputs beside it
            G = efla.default_segments(ws_.B, ws_.H, ws_.L, ws_.dv, ws_.chunk)
            if G > 1:
                wsg = torch.empty(max(1, efla.efla_chunk_fwd_segmented_workspace_size(
                    ws_.B, ws_.H, ws_.L, ws_.dk, ws_.dv, ws_.chunk, G, li["q"].dtype)), dtype=torch.uint8, device=dev)
                fg = efla.prepare_chunk_fwd_segmented(li["q"], li["k"], li["v"], li["beta"], li["s0"], ol, sl, wsg,
                                                      chunk=ws_.chunk, segments=G)
                for _ in range(3):
                    fg()
                gms, _ = flushed_steps(torch, (fg,), K, fl.clean)
                gm = pct(gms, 50)
                shapes[name]["segmented"] = dict(stats_us(gms), segments=G,
                                                 tokens_per_s=round(ws_.tokens / (gm / 1e3), 1),
                                                 hbm_frac=round(b / (gm / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                                 note="efla_chunk_fwd_segmented, the same inputs")
                del wsg, fg
            del li, ol, sl, wsp, f
        line["shapes"] = shapes

        line["decode"] = decode_leg(torch, efla, W, fl, dev, q.dtype, args, esz)

        # ---- training step: forward + backward, exact and Euler ---------------
        train, nb = training_leg(torch, efla, w, inp, o, s_final, ws, dev, K, args)
        line["training"] = train
        # the forward under each rule, flushed steps alternating between the rules
        fx = efla.prepare_chunk_fwd(q, k, v, beta, s0, o, s_final, ws, chunk=w.chunk, rule="exact")
        fe = efla.prepare_chunk_fwd(q, k, v, beta, s0, o, s_final, ws, chunk=w.chunk, rule="euler")
        xs, es = [], []
        for _ in range(max(1, K // 10)):
            xs += flushed_steps(torch, (fx,), 10, fl.clean)[0]
            es += flushed_steps(torch, (fe,), 10, fl.clean)[0]
        xm, em = pct(xs, 50) * 1e3, pct(es, 50) * 1e3
        line["euler"] = {"rule": "euler (alpha = beta)", "flushed_fwd_us": round(em, 2),
                         "exact_flushed_fwd_us": round(xm, 2), "exact_over_euler_time": round(xm / em, 4),
                         "samples": len(es)}
        # backward: bytes it must move: q, k, v, beta, d_o read; dq, dk, dv, dbeta written; states
        bus = train["exact"]["bwd_us"]
        bwd_bytes = n_ht * ((2 * w.dk + 2 * w.dv + 1) * esz + (2 * w.dk + w.dv + 1) * esz) + 3 * state_bytes
        line["backward"] = {"us": bus, "tokens_per_s": round(tokens / (bus / 1e6), 1),
                            "algorithmic_bytes": bwd_bytes,
                            "hbm_frac": round(bwd_bytes / (bus / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                            "workspace_bytes": nb, "train_pair_bwd_us": train["exact"]["pair"]["bwd_us"]}

        # ---- packed variable-length batch -----------------------------------
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
        for _ in range(3):
            fv()
        vms, _ = flushed_steps(torch, (fv,), K, fl.clean)
        vus = pct(vms, 50) * 1e3
        line["varlen"] = {"workload": wv.name, "sequences": wv.B, "tokens": wv.L, "H": wv.H,
                          "lengths_min_median_max": [min(lengths), sorted(lengths)[len(lengths) // 2],
                                                     max(lengths)],
                          "flushed": stats_us(vms), "tokens_per_s": round(wv.L / (vus / 1e6), 1),
                          "warm_us": round(warm_us(torch, (fv,), K), 2)}
        del pv, ov, sv, wsv, fv

        line["segmented"] = segmented_leg(torch, efla, W, fl, dev)

    # ---- the oracle on the host cores -----------------------------------------
    if not args.no_cpu_baseline:
        import oracle
        from delta_rule_sequence_efla_amd.workloads import to_f64
        cores = oracle.default_threads()
        threads = min(cores, w.B * w.H)
        qa, ka, va, ba, sa = (to_f64(x) for x in (q, k, v, beta, s0))
        # whole passes over the workload until about 15 s of CPU time (1 to 8 passes)
        passes, wall_c, cpu_s = 0, 0.0, 0.0
        while passes < 8 and (passes == 0 or cpu_s < 15.0):
            t, c = time.perf_counter(), time.process_time()
            oracle.forward(qa, ka, va, ba, sa, nthreads=threads)
            wall_c += time.perf_counter() - t
            cpu_s += time.process_time() - c
            passes += 1
        line["cpu_baseline"] = {
            "value": round(tokens * passes / wall_c, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole {w.name} workload ({w.B * w.H} sequences x {w.L} tokens), "
                      f"fp64 token-by-token recurrence, {passes} passes, {wall_c:.2f} s wall, "
                      f"{cpu_s:.1f} s of CPU time"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
