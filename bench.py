#!/usr/bin/env python3
"""Benchmark of the LatentIndex decode indexer on one MI355X.

One step = one decode step of a 4-layer group under hierarchical selection
(LatentIndex summary, "Methodology", Hierarchical Selection): append the new
token's latent, absorb the anchor's queries, scan and score the whole shared
cache, select the anchor's top-B candidates and top-k, then for each of the
three followers absorb, rescore the candidates and select top-k.  Workload:
batch 4, 128K context, H = 64, r = 256, bf16 latent, B = 8192, k = 2048
(synthetic, seeded).

Printed: one JSON line with the throughput in scored tokens per second
(L + 3*min(B, L) positions per query per step), the group-step time, the
dominant kernel's roofline fraction (the anchor's latent scan, timed with HIP
events on its stream), the same workload's full-scan step for the HS speedup,
and the CPU oracle timed on a bounded sample of the same step.

A second leg measures the prefill chunk on the matrix cores: 2,048 causal
query positions (62K-64K) against a 64K-token bf16 latent, four layers of
li_score (bf16 absorbed queries, H = 64, r = 256) each followed by li_topk
(k = 2048 per row), reported as MFMA utilisation against the bf16 dense peak.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12  # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15  # flop/s, MI355X dense bf16 matrix cores


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extra", action="store_true", help="skip full-scan and cold-MALL legs")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run warmup + this many steps (for profilers); prints nothing else")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --profile-steps: also run a plain device copy of this many MiB "
                         "three times (calibrates hardware byte counters)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk leg")
    ap.add_argument("--prefill-iters", type=int, default=10)
    ap.add_argument("--path", choices=["hs", "prefill"], default="hs",
                    help="with --profile-steps: which path to run")
    ap.add_argument("--graphs", action="store_true",
                    help="replay the step as two HIP graphs around a direct scan launch instead of "
                         "launching every kernel from the host (on this stack a graph's end costs "
                         "~8 us before the next launch starts, more than the host needs per launch)")
    return ap.parse_args()


def scored_positions(wl, hs: bool) -> int:
    tot = 0
    for s in range(wl.n_q):
        L = int(wl.q_len[s])
        tot += L + (wl.G - 1) * min(wl.B, L) if hs else wl.G * L
    return tot


def latent_bytes_per_token(wl) -> int:
    return {"bf16": 2, "fp8": 1, "fp32": 4}[wl.cache_dtype] * wl.r + (4 if wl.cache_dtype == "fp8" else 0)


ROOT = os.path.dirname(os.path.abspath(__file__))
EV_EVERY = 5  # timed steps per event-timed anchor scan


class ScanEvent:
    """A HIP timing event without the system-scope fence a default event
    performs when it completes (hipEventDisableSystemFence): that fence's
    cache writeback and invalidation would otherwise sit inside the timed
    interval (+2 us on the scan here) and slow the following kernels.
    Recorded on torch's current stream, read like torch.cuda.Event."""
    _hip = None

    def __init__(self):
        import ctypes
        import torch
        self._torch = torch
        if ScanEvent._hip is None:
            ScanEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._c = ctypes
        self.e = ctypes.c_void_p()
        r = self._hip.hipEventCreateWithFlags(ctypes.byref(self.e), ctypes.c_uint(0x20000000))
        if r != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({r})")

    def record(self):
        r = self._hip.hipEventRecord(self.e,
                                     self._c.c_void_p(self._torch.cuda.current_stream().cuda_stream))
        if r != 0:
            raise RuntimeError(f"hipEventRecord failed ({r})")

    def elapsed_time(self, end) -> float:
        ms = self._c.c_float()
        r = self._hip.hipEventElapsedTime(self._c.byref(ms), self.e, end.e)
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return ms.value

    def __del__(self):
        if getattr(self, "e", None) and ScanEvent._hip is not None:
            ScanEvent._hip.hipEventDestroy(self.e)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "anchor_scan_128k_b4_hbm_traffic.md")
SCAN_SOURCES = ["sparse_attention_indexer_latent_amd/csrc/score_scan.hip",
                "sparse_attention_indexer_latent_amd/csrc/li_device.h"]
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_score_2048x64k_mfma_counters.md")
PREFILL_SOURCES = ["sparse_attention_indexer_latent_amd/csrc/score_prefill.hip",
                   "sparse_attention_indexer_latent_amd/csrc/li_device.h"]


def profile_fields(path, sources):
    """The machine-read `key: value` lines of a committed counter summary, or
    None when it is missing or the kernel sources changed since it was taken
    (the summary records their SHA-256)."""
    import hashlib
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "-", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return fields if fields.get("kernel_source_sha256") == h.hexdigest() else None


def measured_traffic(wl):
    """HBM bytes per anchor-scan launch from the committed counter summary
    (calibrated FETCH_SIZE + WRITE_SIZE), or None when that summary covers
    another workload or the scan kernel's source changed since it was taken."""
    f = profile_fields(TRAFFIC_FILE, SCAN_SOURCES) if wl.name == "hs-128k-b4" else None
    try:
        return int(f["traffic_bytes_per_launch"]) if f else None
    except (KeyError, ValueError):
        return None


def measured_mfma_busy():
    """Fraction of cycles the matrix pipes were busy in the prefill scorer,
    from the committed counter summary (None when stale)."""
    f = profile_fields(MFMA_FILE, PREFILL_SOURCES)
    try:
        return float(f["mfma_busy_frac"]) if f else None
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, seconds: float):
    """The oracle's HS group step, query by query, until `seconds` elapse."""
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    done_pos, n_steps = 0, 0
    s = 0
    lat = {}
    el = 0.0
    while True:
        seq = int(wl.q_seq[s])
        if seq not in lat:   # exact decode of the stored cache, outside the timing
            lat[seq] = O.sequence_latent(wl, seq)
        t_a = time.perf_counter()
        O.decode_group(wl, s, C=lat[seq], layers=[0], hs=True)
        el += time.perf_counter() - t_a
        n_steps += 1
        L = int(wl.q_len[s])
        done_pos += L + (wl.G - 1) * min(wl.B, L)
        if el >= seconds:
            break
        s = (s + 1) % wl.n_q
    return {"value": done_pos / el, "unit": "scored tokens/s", "cores": min(cores, blas_threads),
            "kind": "oracle",
            "sample": f"{n_steps} single-query HS group steps of this workload (L={int(wl.q_len[0])}, "
                      f"anchor full scan + top-B + 3 follower rescores, float64 key "
                      f"reconstruction and stable sort), {el:.1f} s of oracle time (the exact "
                      f"decode of the stored cache is done once, untimed); host affinity "
                      f"{cores} cores, BLAS threads {blas_threads}"}


def prefill_setup(torch, W, DeviceWorkload):
    """Device operands of the prefill chunk: the 64K-token latent, every
    layer's bf16 absorbed queries and head weights, score and index buffers."""
    wl = W.config(4)
    dw = DeviceWorkload(wl, hold_last=False)
    qts, ws = [], []
    for layer in range(wl.G):
        bits, w = wl.prefill_queries(layer)
        qts.append(torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16))
        ws.append(torch.from_numpy(w).cuda())
    L = int(wl.lens[0])
    u = torch.empty((wl.n_q, L), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.G, wl.n_q, wl.k), dtype=torch.int32, device="cuda")
    return wl, dw, qts, ws, u, idx


def prefill_chunk(ops, wl, dw, qts, ws, u, idx, ev=None):
    """One prefill chunk: per layer, score every causal (query, token) pair,
    then select each row's top-k.  ev (optional): per layer, a pair of events
    bracketing li_score."""
    L = int(wl.lens[0])
    for layer in range(wl.G):
        if ev is not None:
            ev[layer][0].record()
        ops.score(qts[layer], ws[layer], None, dw.q_seq, dw.q_len, L, dw.cache, scores=u)
        if ev is not None:
            ev[layer][1].record()
        ops.topk(u, dw.q_len, L, wl.k, out_idx=idx[layer])


def prefill_leg(torch, ops, W, DeviceWorkload, iters: int) -> dict:
    wl, dw, qts, ws, u, idx = prefill_setup(torch, W, DeviceWorkload)
    for _ in range(2):
        prefill_chunk(ops, wl, dw, qts, ws, u, idx)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(wl.G)] for _ in range(iters)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        prefill_chunk(ops, wl, dw, qts, ws, u, idx, ev[i])
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / iters
    score_s = float(np.mean([a.elapsed_time(b) for it in ev for a, b in it])) * 1e-3
    pairs = int(wl.q_len.astype(np.int64).sum())       # valid (query, token) pairs per layer
    flop = 2 * wl.H * wl.r * pairs                        # one MAC per head and latent dim
    return {"workload": f"{wl.name}: {wl.G} layers x (li_score of {wl.n_q} causal bf16 queries "
                        f"(positions {int(wl.q_len[0]) - 1}..{int(wl.q_len[-1]) - 1}) over "
                        f"{int(wl.lens[0])} bf16 latents, H={wl.H}, r={wl.r}; li_topk k={wl.k} "
                        f"per row)",
            "ms_per_chunk": el * 1e3,
            "score_ms_per_layer": score_s * 1e3,
            "topk_ms_per_layer": (el - wl.G * score_s) / wl.G * 1e3,
            "valid_pairs_per_layer": pairs,
            "flop_per_layer": flop,
            "roofline": {"bound": "mfma", "kernel": "score_prefill_kernel",
                         "achieved": flop / score_s / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                         "unit": "TFLOP/s", "frac": flop / score_s / MFMA_BF16_PEAK,
                         "traffic": None, "avg_kernel_us": score_s * 1e6,
                         "flop_per_launch": flop,
                         "mfma_busy_frac_counters": measured_mfma_busy()},
            "tokens_scored_per_s": wl.G * pairs / el}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the indexer runs and is measured on one GPU (sharding across "
                                   "GPUs is a design only), so --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch

    from sparse_attention_indexer_latent_amd import ops
    from sparse_attention_indexer_latent_amd import workloads as W
    from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload

    torch.cuda.set_device(0)
    if ops.lib().li_check_device() != ops.LI_OK:
        raise SystemExit(ops.lib().li_last_error().decode())
    if args.profile_steps and args.path == "prefill":
        pf = prefill_setup(torch, W, DeviceWorkload)
        for _ in range(args.warmup + args.profile_steps):
            prefill_chunk(ops, *pf)
        torch.cuda.synchronize()
        return
    wl = W.config(args.config)
    hs = wl.B is not None
    dw = DeviceWorkload(wl, hold_last=True)
    if args.graphs:
        graphs = dw.capture(hs)
        step = graphs.replay
    else:
        step = dw.hs_step if hs else dw.full_step

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        if args.copy_mib:
            x = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
            y = torch.empty_like(x)
            for _ in range(3):
                torch.neg(x, out=y)  # reads and writes copy_mib MiB
        torch.cuda.synchronize()
        return

    K = args.steps
    # Events bracket the anchor scan on every EV_EVERY-th timed step: even a
    # fence-free pair of event records costs ~3 us of a ~115 us step, so
    # timing every step would slow the very loop whose throughput is reported.
    evs = {i: (ScanEvent(), ScanEvent()) for i in range(0, K, EV_EVERY)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events=evs.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    el = t1 - t0
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in evs.values()]))

    pos = scored_positions(wl, hs)
    bpt = latent_bytes_per_token(wl)
    scan_tokens = int(wl.q_len.sum())
    scan_bytes = scan_tokens * (bpt + 4)            # latent read + fp32 score write
    step_bytes = scan_tokens * bpt + (sum(min(wl.B, int(L)) for L in wl.q_len) * (wl.G - 1) * bpt
                                      if hs else scan_tokens * bpt * (wl.G - 1))
    us_step = el / K * 1e6

    out = {
        "metric": "indexer scored tokens/s and us/decode step per 4-layer group at 128K; % HBM BW",
        "value": pos * K / el,
        "unit": "scored tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": el / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cache_dtype == "bf16" else wl.cache_dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: HS decode step of a 4-layer group, batch {wl.n_q}, "
                               f"L={wl.max_len}, H={wl.H}, r={wl.r}, {wl.cache_dtype} latent, "
                               f"B={wl.B}, k={wl.k}, 64-token pages, random block table",
                   "global_batch": wl.n_q, "seq_len": wl.max_len, "parallelism": "none (1 GPU)",
                   "launch": "hipGraph pre | direct anchor scan | hipGraph post" if args.graphs
                   else "direct launches from the host on one stream"},
        "us_per_group_step": us_step,
        "scored_positions_per_step": pos,
        "hbm_frac_step": step_bytes / (el / K) / HBM_PEAK,
        "roofline": {"bound": "hbm", "kernel": "score_scan_kernel (anchor full scan)",
                     "achieved": scan_bytes / (scan_ms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": scan_bytes / (scan_ms * 1e-3) / HBM_PEAK,
                     "traffic": measured_traffic(wl), "avg_kernel_us": scan_ms * 1e3,
                     "bytes_per_launch": scan_bytes},
    }

    if not args.no_extra:
        # Full scan of the same group (every layer scans everything).
        Kf = max(5, K // 2)
        fstep = dw.capture(False).replay if args.graphs else dw.full_step
        for _ in range(2):
            fstep()
        fevs = {i: (ScanEvent(), ScanEvent()) for i in range(0, Kf, EV_EVERY)}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(Kf):
            fstep(events=fevs.get(i))
        torch.cuda.synchronize()
        elf = time.perf_counter() - t0
        fscan = float(np.mean([a.elapsed_time(b) for a, b in fevs.values()]))
        fpos = scored_positions(wl, False)
        out["full_scan"] = {"us_per_group_step": elf / Kf * 1e6,
                            "scored_tokens_per_s": fpos * Kf / elf,
                            "hbm_frac_step": scan_tokens * bpt * wl.G / (elf / Kf) / HBM_PEAK,
                            "scan_kernel_us": fscan * 1e3}
        out["hs_speedup_vs_full_scan"] = (elf / Kf) / (el / K)
        # Cold MALL: stream 1 GiB through the memory system before each step.
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        Kc = 10
        cold = []
        for i in range(Kc):
            flush.fill_(float(i))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        out["cold_mall_us_per_group_step"] = float(np.median(cold)) * 1e3
        del flush

    if not args.no_prefill:
        out["prefill"] = prefill_leg(torch, ops, W, DeviceWorkload, args.prefill_iters)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        out["gpu_over_cpu"] = out["value"] / out["cpu_baseline"]["value"]

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
