#!/usr/bin/env python3
"""Benchmark of the context-lookup drafting hot path on one MI355X.

One step = lookup + fusion + greedy acceptance + scheduler update over a whole
batch (default: 64 requests of 25,000 tokens, 32 verbatim-restatement and 32
ordinary Zipf texts, vocabulary 40,960), through the fused lookup_decode_step
entry point (one kernel), or with --separate through the four entry points
lookup_propose, fuse_verify_block, greedy_accept, lookup_schedule_step.
Inputs are resident in HBM before timing.  The batch is copied into enough
distinct buffers (>= 320 MB) that consecutive steps never hit the 256 MB
Infinity Cache, and the steps are replayed from a HIP graph so the host does
not throttle the launches.

Printed: one JSON line with the throughput (history tokens scanned per second),
the roofline of the dominant kernel (the scan kernel that runs the whole step;
its duration is stamped by the GPU on each dispatch through the *_timed entry
point) and the CPU oracle timed on the host's cores as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c4|c5]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "history tokens scanned/s (HBM GB/s, % peak) + lookups/s at B=64, 25k ctx"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 320 << 20
COUNTERS_FILE = os.path.join(ROOT, "profiles", "lookup_scan_counters.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="c3", choices=["c3", "c4", "c5"])
    ap.add_argument("--cpu-work-seconds", type=float, default=20.0,
                    help="CPU work (seconds summed over threads) for the oracle baseline; 0 = skip")
    ap.add_argument("--scan-wgs", type=int, default=0, help="lookup launch tuning (0 = auto)")
    ap.add_argument("--separate", action="store_true",
                    help="time the four separate entry points instead of the fused step")
    ap.add_argument("--telemetry", action="store_true",
                    help="fused step with per-request acceptance telemetry on")
    ap.add_argument("--kernel-only", type=int, default=0, metavar="N",
                    help="profiling aid: only N eager lookup launches over the rotating sets")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="profiling aid: 5 plain device copies of MIB MiB (counter calibration)")
    return ap.parse_args()


def calibrate_copy(mib):
    """Plain device-to-device copies of known size, for scaling HBM counters."""
    import torch
    n = (mib << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 5}), flush=True)


def per_request_bytes(separate, telemetry=False):
    """Algorithmic bytes per request besides the history, for the timed kernel:
    the lookup alone reads row_off and len (12) and writes match_len, match_end
    and the draft (68); the whole step also reads the proposal, target tokens
    and scheduler state (104) and writes the block, block_len, accept, state
    and long_next (84); telemetry reads the request's 32-word row (128) and
    writes its 25 counters back (100)."""
    if separate:
        return 80
    return 80 + 104 + 84 + (228 if telemetry else 0)


KERNEL_SOURCES = ("context_lookup_drafting_amd/csrc/lcd_lookup.hip",
                  "context_lookup_drafting_amd/csrc/lcd_rules.h", "include/lcd.h")


def kernel_source_hash():
    """sha256[:16] over the sources the fused step kernel is compiled from."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload_name, launches_per_step=1):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source and this workload; otherwise None."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(workload_name)
    if not ent or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime the library is linked to."""

    def __init__(self, lib):
        self.h = lib
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.h.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        if self.h.hipEventSynchronize(ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        f = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, ev):
        self.h.hipEventDestroy(ctypes.c_void_p(ev))


def cpu_baseline(w, work_seconds):
    """The CPU oracle (as it is) over full steps of the same batch, threads over
    requests; bounded to about `work_seconds` of CPU time summed over threads."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liblcd_oracle.so")):
        oracle.build()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    op = oracle.default_params()
    q, tgt = w.step_inputs(np.zeros(w.B, np.int64), 0)
    hs = w.hists
    chunks = [list(range(i, w.B, cores)) for i in range(cores)]

    def run_chunk(idx):
        for r in idx:
            h = hs[r]
            m, e, d = oracle.lookup_propose(h, np.zeros(1, np.int64), np.array([len(h)], np.int32), op)
            blk, bl = oracle.fuse_verify_block(d, m, q[r:r + 1], np.zeros(1, np.int32), op)
            acc = oracle.greedy_accept(blk, bl, tgt[r:r + 1])
            st = np.zeros((1, 3), np.int32)
            oracle.lookup_schedule_step(st, m, acc, bl, op)
        return len(idx)

    tokens = int(sum(len(h) for h in hs))
    batches = 0
    cpu0 = time.process_time()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as pool:
        while True:
            list(pool.map(run_chunk, chunks))
            batches += 1
            if time.process_time() - cpu0 >= work_seconds or time.perf_counter() - t0 > 120:
                break
    wall = time.perf_counter() - t0
    return {
        "value": round(batches * tokens / wall, 1),
        "unit": "history tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{batches} full steps (lookup+fuse+accept+schedule) of the {w.B}-request "
                   f"batch, {tokens} history tokens each, threads over requests, "
                   f"{wall:.2f} s wall / {time.process_time() - cpu0:.1f} s CPU"),
        "lookups_per_s": round(batches * w.B / wall, 1),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the lookup path needs no "
              "cross-GPU exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np
    import torch

    import context_lookup_drafting_amd as lcd
    from context_lookup_drafting_amd import workloads as wl

    lib = lcd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "c3":
        w = wl.config3()
    elif args.workload == "c4":
        w = wl.config4()
    else:
        w = wl.config5()
    flat, ro, ln, cap = wl.pack_rows(w.hists)
    B = w.B
    tokens = int(ln.astype(np.int64).sum())
    max_len = int(ln.max())
    set_bytes = flat.nbytes
    R = max(2, -(-ROTATE_BYTES // set_bytes))
    R += R % 2                       # even, so the two long-mode buffers alternate cleanly
    p = lcd.default_params(scan_wgs=args.scan_wgs)

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    hist_sets = [t(flat) for _ in range(R)]
    ro_d, ln_d = t(ro), t(ln)
    q, tgt = w.step_inputs(np.zeros(B, np.int64), 0)
    q_d, tgt_d = t(q), t(tgt)
    ws = lcd.alloc_workspace(B, dev)
    dws = lcd.alloc_decode_workspace(B, max_len, dev, p)
    m = torch.empty(B, dtype=torch.int32, device=dev)
    e = torch.empty_like(m)
    d = torch.empty((B, 15), dtype=torch.int32, device=dev)
    blk = torch.empty((B, 15), dtype=torch.int32, device=dev)
    bl = torch.empty(B, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    ln_next = torch.empty(B, dtype=torch.int32, device=dev)
    state = torch.zeros((B, 3), dtype=torch.int32, device=dev)
    longs = [torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(2)]
    tele = lcd.alloc_telemetry(B, dev) if args.telemetry else None
    if args.telemetry and args.separate:
        print("bench.py: --telemetry applies to the fused step only", file=sys.stderr)
        sys.exit(2)

    if args.kernel_only:
        for i in range(args.kernel_only):
            if args.separate:
                lcd.lookup_propose(hist_sets[i % R], ro_d, ln_d, max_len, ws, m, e, d, p)
            else:
                lcd.lookup_decode_step(hist_sets[i % R], ro_d, ln_d, None, max_len, q_d, tgt_d,
                                       state, dws, m, e, d, blk, bl, acc, ln_next, False, p,
                                       telemetry=tele)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only_launches": args.kernel_only, "workload": w.name,
                          "tokens_per_launch": tokens,
                          "alg_bytes_per_launch": (4 * tokens
                                                   + per_request_bytes(args.separate, args.telemetry) * B),
                          "rotating_sets": R, "separate": args.separate}), flush=True)
        return

    def step(i):
        if args.separate:
            lcd.lookup_propose(hist_sets[i % R], ro_d, ln_d, max_len, ws, m, e, d, p)
            lcd.fuse_verify_block(d, m, q_d, longs[i % 2], blk, bl, p)
            lcd.greedy_accept(blk, bl, tgt_d, acc)
            lcd.lookup_schedule_step(state, m, acc, bl, longs[(i + 1) % 2], p)
        else:
            lcd.lookup_decode_step(hist_sets[i % R], ro_d, ln_d, None, max_len, q_d, tgt_d, state,
                                   dws, m, e, d, blk, bl, acc, ln_next, False, p, telemetry=tele)

    # eager reference of one step, then the graphs
    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (m, e, d)]

    def capture(nsteps):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(nsteps):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        return g

    K, W = args.steps, args.warmup
    g_full = capture(R)
    g_tail = capture(K % R) if K % R else None

    # warmup
    for _ in range(max(1, -(-W // R))):
        g_full.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ------------------------------------
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K // R):
        g_full.replay()
    if g_tail is not None:
        g_tail.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # every replay must reproduce the eager lookup (identical sets)
    for x, y in zip((m, e, d), ref):
        if not torch.equal(x, y):
            print("bench.py: graph replay disagrees with the eager step", file=sys.stderr)
            sys.exit(3)

    # ---- kernel duration of the lookup scan, stamped by the GPU -----------
    hev = HipEvents(lib)
    n_k = min(K, 400)
    evs = [(hev.create(), hev.create()) for _ in range(n_k)]
    for i in range(n_k):
        if args.separate:
            lcd.lookup_propose_timed(hist_sets[i % R], ro_d, ln_d, max_len, ws, m, e, d,
                                     evs[i][0], evs[i][1], p)
        else:
            lcd.lookup_decode_step_timed(hist_sets[i % R], ro_d, ln_d, None, max_len, q_d, tgt_d,
                                         state, dws, m, e, d, blk, bl, acc, evs[i][0], evs[i][1],
                                         ln_next, False, p, telemetry=tele)
    torch.cuda.synchronize()
    durs = np.array([hev.elapsed_ms(a, b) for a, b in evs]) * 1e-3
    for a, b in evs:
        hev.destroy(a)
        hev.destroy(b)
    k_avg = float(durs.mean())

    alg_bytes = 4 * tokens + per_request_bytes(args.separate, args.telemetry) * B
    achieved = alg_bytes / k_avg / 1e9
    traffic = None if (args.separate or args.telemetry) else load_traffic(w.name)
    value = K * tokens / elapsed
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "history tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed / K * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": B,
            "tokens_per_step": tokens,
            "max_len": max_len,
            "vocab": w.vocab,
            "rotating_sets": R,
            "rotating_bytes": R * set_bytes,
            "launch": (f"HIP graph of {R} steps, "
                       + ("4 entry points (4 kernels) per step" if args.separate
                          else "lookup_decode_step (1 kernel) per step")),
            "telemetry": args.telemetry,
        },
        "lookups_per_s": round(K * B / elapsed, 1),
        "step_hbm_gbps": round(value * 4 / 1e9, 2),
        "step_pct_peak": round(value * 4 / 1e9 / HBM_PEAK_GBPS * 100, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": ("lookup_scan_kernel<4,kPropose>" if args.separate
                       else "lookup_scan_kernel<4,kStep>"),
            "kernel_us_mean": round(k_avg * 1e6, 3),
            "kernel_us_p10_p50_p90": [round(float(np.percentile(durs, x)) * 1e6, 3)
                                      for x in (10, 50, 90)],
            "alg_bytes_per_launch": alg_bytes,
            "launches_timed": n_k,
        },
    }
    if args.cpu_work_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_work_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
