#!/usr/bin/env python3
"""Benchmark of the LatentIndex decode indexer on one MI355X.

One step = one decode step of a 4-layer group under hierarchical selection
(LatentIndex summary, "Methodology", Hierarchical Selection): append the new
token's latent, absorb every layer's queries, scan and score the whole shared
cache with the anchor, select its top-B candidates and top-k, then rescore the
candidates with the three followers and select their top-k.  Workload: batch
4, 128K context, H = 64, r = 256, bf16 latent, B = 8192, k = 2048 (synthetic,
seeded).

Printed: one JSON line with the throughput in scored tokens per second
(L + 3*min(B, L) positions per query per step), the group-step time, the
dominant kernel's roofline fraction (the anchor's latent scan, timed with HIP
events on its stream inside the timed loop), and the CPU oracle timed on a
bounded sample of the same step.  Beside them:
  cold      the same step and scan after the 256 MB last-level cache (MALL)
            was flushed (a 1 GiB write, then a 1 GiB read of another buffer,
            so no dirty line is left to write back inside the timing);
  legs      the full-scan group step of the same workload (HS speedup); the
            128K batch-1 group (full scan and HS); the 32K batch-1 bf16 and
            16 ragged fp8 sequences full-scan steps -- each with its scan's
            warm (back-to-back launches) and cold time and HBM fraction;
  ceiling   a plain device copy of the anchor scan's byte count, warm and
            cold, as the practical bandwidth ceiling of this part;
  prefill   2,048 causal query positions against a 64K-token bf16 latent,
            four layers of li_score + li_topk (k = 2048 per row), as matrix-
            core utilisation against the bf16 dense peak.
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
MFMA_FP32_PEAK = 157.3e12  # flop/s, MI355X dense fp32 matrix cores


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hs-128k-b4",
                    help="headline workload (a name from workloads.WORKLOADS)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extra", action="store_true", help="skip the cold, legs and ceiling parts")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run warmup + this many steps (for profilers); prints nothing else")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --profile-steps: also run a plain device copy of this many MiB "
                         "three times (calibrates hardware byte counters)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk leg")
    ap.add_argument("--prefill-iters", type=int, default=10)
    ap.add_argument("--path", choices=["hs", "full", "b1", "dsv32-32k", "ragged-fp8", "prefill",
                                       "calib"],
                    default="hs",
                    help="with --profile-steps: which step to run (hs / full: the 4 x 128K HS or "
                         "full-scan step; b1: the 128K batch-1 full-scan step; dsv32-32k: 32K batch 1; "
                         "ragged-fp8: 16 ragged fp8 sequences; prefill: the prefill chunk)")
    ap.add_argument("--no-legs", action="store_true", help="skip the legs beside the headline")
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
    wl = W.named("prefill-2048x64k")
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


class Flusher:
    """Empties the last-level cache between timed runs without leaving dirty
    lines behind: a 1 GiB write of one buffer, then a 1 GiB read of another
    (the read evicts the written lines, whose write-back happens during the
    flush).  Enqueued without a host synchronisation, it keeps the GPU busy
    for about 0.5 ms while the host enqueues the timed work behind it, so the
    events that follow time the device only."""

    def __init__(self, torch):
        self.a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        self.b = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.acc = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
        self.torch = torch

    def __call__(self):
        self.a.fill_(1.0)
        self.torch.sum(self.b.view(1 << 16, -1), dim=1, out=self.acc)


def timed_pair(torch, fn, flush=None, scan=False):
    """(step us, scan us) of one run of fn, device-timed with events; flush
    first when given.  fn takes events= for its scoring launch when scan."""
    a, b = ScanEvent(), ScanEvent()
    sev = (ScanEvent(), ScanEvent()) if scan else None
    if flush is not None:
        flush()
    a.record()
    if scan:
        fn(events=sev)
    else:
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3, (sev[0].elapsed_time(sev[1]) * 1e3 if scan else None)


def scan_b2b_us(torch, scan, n=20):
    """Average time of n back-to-back launches of one scan (warm), between
    two events: no per-launch event overhead, the launch gaps included."""
    for _ in range(3):
        scan()
    a, b = ScanEvent(), ScanEvent()
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        scan()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def loop_us(torch, step, K, warm=3):
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / K * 1e6


def leg(torch, flush, dw, hs, K=20, Kc=8):
    """Warm and cold figures of one decode workload: the group step (warm:
    wall clock of K back-to-back steps; cold: device time after a flush), and
    the layer-0 scan (warm: back-to-back launches; cold: after a flush)."""
    wl = dw.wl
    step = dw.hs_step if hs else dw.full_step
    us = loop_us(torch, step, K)
    dw.absorb()
    from sparse_attention_indexer_latent_amd import ops
    # pre-marshalled, so that back-to-back launches are not host-bound
    scan = ops.prepared_score(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len,
                              dw.max_len, dw.cache, dw.scores)
    warm_scan = scan_b2b_us(torch, scan)
    cold = [timed_pair(torch, step, flush, scan=True) for _ in range(Kc)]
    cold_scan = [timed_pair(torch, scan, flush)[0] for _ in range(Kc)]
    bpt = latent_bytes_per_token(wl)
    scan_tokens = int(wl.q_len.sum())
    sbytes = scan_tokens * (bpt + 4)
    cs = float(np.median(cold_scan))
    pos = scored_positions(wl, hs)
    return {"us_per_group_step": us,
            "cold_us_per_group_step": float(np.median([c[0] for c in cold])),
            "scored_tokens_per_s": pos / (us * 1e-6),
            "scan_bytes_per_launch": sbytes,
            "scan_us_warm": warm_scan, "scan_frac_warm": sbytes / (warm_scan * 1e-6) / HBM_PEAK,
            "scan_us_cold": cs, "scan_frac_cold": sbytes / (cs * 1e-6) / HBM_PEAK,
            "scan_us_cold_in_step": float(np.median([c[1] for c in cold]))}


def copy_ceiling(torch, flush, nbytes):
    """A plain device copy of nbytes (read nbytes, write nbytes), warm and
    cold, in TB/s of bytes moved."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    warm = scan_b2b_us(torch, lambda: y.copy_(x), n=10)
    cold = float(np.median([timed_pair(torch, lambda: y.copy_(x), flush)[0] for _ in range(6)]))
    del x, y
    return {"bytes_moved": 2 * nbytes, "warm_us": warm, "warm_TBps": 2 * nbytes / warm / 1e6,
            "cold_us": cold, "cold_TBps": 2 * nbytes / cold / 1e6}


def dsa_leg(torch, flush, W, DsaGroup, batch, K=20, Kc=6):
    """The native DSA indexer over the group's four layers at 128K: warm
    (back-to-back steps) and cold step times, and its layer-0 key scan."""
    from sparse_attention_indexer_latent_amd import ops
    g = DsaGroup([W.dsa_layer(l, [131072] * batch) for l in range(4)])
    us = loop_us(torch, g.step, K)
    cold = [timed_pair(torch, g.step, flush, scan=True) for _ in range(Kc)]
    d = g.layers[0]
    scan = ops.prepared_score(d.q[0], d.w[0], None, d.q_seq, d.q_len, d.max_len, d.cache, d.scores)
    warm_scan = scan_b2b_us(torch, scan)
    cold_scan = float(np.median([timed_pair(torch, scan, flush)[0] for _ in range(Kc)]))
    sbytes = batch * 131072 * (d.cache.bytes_per_token + 4)
    out = {"workload": f"native DSA indexer, 4 layers x own fp8 key cache ({d.cache.bytes_per_token} "
                       f"B/token: 128 values + 1 fp32 scale), H=64, batch {batch} x 131072, "
                       f"k=2048; per layer: append the new key, li_score_topk",
           "us_per_group_step": us,
           "cold_us_per_group_step": float(np.median([c[0] for c in cold])),
           "scan_bytes_per_launch": sbytes,
           "scan_us_warm": warm_scan, "scan_frac_warm": sbytes / (warm_scan * 1e-6) / HBM_PEAK,
           "scan_us_cold": cold_scan, "scan_frac_cold": sbytes / (cold_scan * 1e-6) / HBM_PEAK,
           "scored_tokens_per_s": 4 * batch * 131072 / (us * 1e-6)}
    del g
    torch.cuda.empty_cache()
    return out


def context_sweep(torch, W, DeviceWorkload, DsaGroup, Ls, K=20):
    """HS step of the pages' geometry (192-value fp8 latent, 200-byte record,
    B = 8192) against the native DSA indexer of the same four layers (132 B
    per token per layer), batch 1, at each context length of the pages'
    Table 4; warm step times (back-to-back steps)."""
    rows = []
    for L in Ls:
        wl = W.hs_128k(1, r=192, cache_dtype="fp8", scale_block=128, L=L)
        d = DeviceWorkload(wl, hold_last=True)
        hs_us = loop_us(torch, d.hs_step, K)
        full_us = loop_us(torch, d.full_step, K)
        del d
        g = DsaGroup([W.dsa_layer(l, [L]) for l in range(4)])
        dsa_us = loop_us(torch, g.step, K)
        del g
        torch.cuda.empty_cache()
        rows.append({"L": L, "hs_us_per_group_step": hs_us, "full_scan_us_per_group_step": full_us,
                     "dsa_us_per_group_step": dsa_us, "hs_speedup_vs_dsa": dsa_us / hs_us,
                     "hs_latent_bytes": 200 * (L + 3 * min(8192, L)), "dsa_key_bytes": 4 * 132 * L})
    return {"workload": "batch 1, H=64, k=2048; HS: 200 B/token latent (192 fp8 values + 2 fp32 "
                        "block scales), B=8192, 3 followers; DSA: 4 layers x own fp8 key cache "
                        "(128 values + 1 fp32 scale = 132 B/token)",
            "pages_table4_context": "HS over DSA 2.30-2.72x at 8K-128K (ms per decode token, all "
                                    "61 indexers, batch 1, eight unnamed GPUs)",
            "points": rows}


def budget_sweep(torch, W, DeviceWorkload, Bs, r=192, dtype="fp8", sb=128, K=20, layer_corr=0.0):
    """Candidate budget B against HS step time and the followers' recall of
    their own full-scan selections (|S_HS ∩ S_full| / k, mean over followers
    and queries) on the synthetic 128K batch-1 workload of the pages'
    geometry.  Synthetic decoders share a common part (D_l = (G0 + 0.3 G_l) /
    sqrt(r)); the layers' queries and head weights are independent, or
    correlated at layer_corr.  These recalls describe the generator, not a
    trained model."""
    from sparse_attention_indexer_latent_amd import ops
    wl = W.hs_128k(1, r=r, cache_dtype=dtype, scale_block=sb, B=max(Bs), layer_corr=layer_corr)
    dw = DeviceWorkload(wl, hold_last=True)
    dw.full_step()
    torch.cuda.synchronize()
    full = dw.sel.cpu().numpy()
    rows = []
    for B in Bs:
        cand = torch.empty((wl.n_q, B), dtype=torch.int32, device="cuda")
        hs = torch.empty((wl.G, wl.n_q, wl.k), dtype=torch.int32, device="cuda")
        aws = ops.hs_anchor_workspace(wl.n_q, dw.max_len)
        fws = ops.hs_workspace(wl.n_q, B, wl.k, n_f=wl.G - 1)

        def step(B=B, cand=cand, hs=hs, aws=aws, fws=fws):
            dw._pre(True)
            ops.hs_anchor(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, dw.max_len,
                          dw.cache, B, wl.k, scores=dw.scores, cand=cand, sel=hs[0], ws=aws)
            ops.hs_select(cand, dw.q_tilde[1:], dw.w[1:], dw.beta[1:], dw.q_seq, dw.cache, wl.k,
                          out_idx=hs[1:], ws=fws)
        us = loop_us(torch, step, K)
        h = hs.cpu().numpy()
        rec = [len(set(h[l, s].tolist()) & set(full[l, s].tolist())) / wl.k
               for l in range(1, wl.G) for s in range(wl.n_q)]
        rows.append({"B": B, "us_per_group_step": us, "follower_recall": float(np.mean(rec)),
                     "scored_positions": 131072 + (wl.G - 1) * min(B, 131072)})
    del dw
    torch.cuda.empty_cache()
    return {"workload": f"{wl.name} with B varied (HS step: anchor scan + nested top-B/top-k, "
                        f"3 followers rescore B candidates)", "points": rows}


def calibration_leg(torch, n=16384, d=7168, m=4, d_R=64, d_N=64, reps=3):
    """The calibration's normal equations at DeepSeek-V3.2's hidden size: one
    li_calib_gram over n bf16 hidden-state rows X [n, d] and the group's keys
    Y [n, m (d_R + d_N)] (random draws: timing only), against the dense fp32
    matrix-core peak (the kernel multiplies on v_mfma_f32_16x16x4f32).
    Algorithmic flop: 2 n per distinct output, i.e. n d (d + 1) for the
    symmetric X^T X plus 2 n d e for X^T Y.  Then the host's closed form
    (float64) from those normal equations, timed apart."""
    from sparse_attention_indexer_latent_amd import calibrate, ops
    e = m * (d_R + d_N)
    g = torch.Generator(device="cuda").manual_seed(7)
    X = torch.randn((n, d), generator=g, device="cuda").to(torch.bfloat16)
    Y = torch.randn((n, e), generator=g, device="cuda").to(torch.bfloat16)
    G = torch.empty((d, d), dtype=torch.float32, device="cuda")
    H = torch.empty((d, e), dtype=torch.float32, device="cuda")
    xs = torch.empty(d, dtype=torch.float32, device="cuda")
    ys = torch.empty(e, dtype=torch.float32, device="cuda")
    ops.calib_gram(X, Y, G, H, xs, ys)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ops.calib_gram(X, Y, G, H, xs, ys)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flop = n * d * (d + 1) + 2 * n * d * e
    ne = (G.double().cpu().numpy(), H.double().cpu().numpy(), xs.double().cpu().numpy(),
          ys.double().cpu().numpy(), n)
    del X, Y, G, H
    torch.cuda.empty_cache()
    theta = 10000.0 ** (-np.arange(d_R // 2) * 2.0 / d_R)
    t0 = time.perf_counter()
    cal = calibrate.fit_from_normal_equations(ne, m, d_R, theta, 128, 1, 1.0)
    host_s = time.perf_counter() - t0
    return {"workload": f"calibration normal equations: n={n} bf16 rows, d_model={d}, "
                        f"{m} layers x (d_R={d_R} + d_N={d_N}) keys; closed form r = "
                        f"{cal.P.shape[1]} (r_R={cal.r_R}, r_N=128), lam=1",
            "gram_ms": ms, "roofline": {"bound": "mfma", "achieved": flop / (ms * 1e-3) / 1e12,
                                        "peak": MFMA_FP32_PEAK / 1e12, "unit": "TFLOP/s",
                                        "frac": flop / (ms * 1e-3) / MFMA_FP32_PEAK,
                                        "flop_per_launch": flop},
            "host_closed_form_s": host_s}


def batch1_128k(W):
    """The 128K batch-1 group: the batch-4 workload's generator for one
    sequence."""
    return W.make_decode("hs-128k-b1", 3, 0, G=4, H=64, r=256, d_I=128, k=2048, B=8192,
                         cache_dtype="bf16", lens=[131072], plant_frac=0.01, plant_factor=3.0,
                         permute_blocks=True)


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
    if args.path == "calib":  # the calibration's normal equations alone (for profiling)
        print(json.dumps(calibration_leg(torch)), flush=True)
        return
    if args.profile_steps and args.path == "prefill":
        pf = prefill_setup(torch, W, DeviceWorkload)
        for _ in range(args.warmup + args.profile_steps):
            prefill_chunk(ops, *pf)
        torch.cuda.synchronize()
        return
    if args.profile_steps and args.path in ("b1", "dsv32-32k", "ragged-fp8"):
        wl = {"b1": batch1_128k(W), "dsv32-32k": W.named("dsv32-decode-32k"),
              "ragged-fp8": W.named("ragged-16x8k-128k-fp8")}[args.path]
        dw = DeviceWorkload(wl, hold_last=True)
        for _ in range(args.warmup + args.profile_steps):
            dw.full_step()
        torch.cuda.synchronize()
        return
    wl = W.named(args.workload)
    hs = wl.B is not None and args.path != "full"
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
    # fence-free pair of event records costs ~3 us of the step, so timing
    # every step would slow the very loop whose throughput is reported.
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
        "config": {"workload": f"{wl.name}: {'HS' if hs else 'full-scan'} decode step of a "
                               f"4-layer group, batch {wl.n_q}, L={wl.max_len}, H={wl.H}, "
                               f"r={wl.r}, {wl.cache_dtype} latent, B={wl.B}, k={wl.k}, "
                               f"64-token pages, random block table",
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
                     "bytes_per_launch": scan_bytes,
                     "timing": "warm: inside the timed loop of back-to-back steps (the 256 MB "
                               "MALL may hold part of the 268 MB the scan reads); the cold "
                               "figure is under roofline.cold"},
    }

    if not args.no_extra:
        flush = Flusher(torch)
        Kc = 10
        cold = [timed_pair(torch, step, flush, scan=True) for _ in range(Kc)]
        cscan = float(np.median([c[1] for c in cold]))
        out["roofline"]["cold"] = {"avg_kernel_us": cscan,
                                   "achieved": scan_bytes / (cscan * 1e-6) / 1e9,
                                   "frac": scan_bytes / (cscan * 1e-6) / HBM_PEAK,
                                   "timing": f"median of {Kc} steps, each after a flush of the "
                                             "last-level cache (1 GiB written, then 1 GiB of "
                                             "another buffer read)"}
        out["cold_us_per_group_step"] = float(np.median([c[0] for c in cold]))
        out["ceiling"] = copy_ceiling(torch, flush, scan_bytes)
        if not args.no_legs:
            legs = {}
            full = leg(torch, flush, dw, False, K=max(5, K // 2))
            legs["full_scan_128k_b4"] = full
            out["hs_speedup_vs_full_scan"] = full["us_per_group_step"] / us_step
            out["hs_speedup_vs_full_scan_cold"] = (full["cold_us_per_group_step"]
                                                  / out["cold_us_per_group_step"])
            del dw
            torch.cuda.empty_cache()
            for name, wlf, with_hs in (("128k_b1", batch1_128k(W), True),
                                       ("32k_b1_bf16", W.named("dsv32-decode-32k"), False),
                                       ("ragged16_fp8", W.named("ragged-16x8k-128k-fp8"), False)):
                d = DeviceWorkload(wlf, hold_last=True)
                lf = leg(torch, flush, d, False)
                lf["workload"] = (f"{wlf.name}: full-scan step, {wlf.n_q} x L "
                                  f"{int(wlf.q_len.min())}..{int(wlf.q_len.max())}, "
                                  f"{wlf.cache_dtype} latent, r={wlf.r}, H={wlf.H}, k={wlf.k}")
                legs["full_scan_" + name] = lf
                if with_hs:
                    lh = leg(torch, flush, d, True)
                    lh["workload"] = f"{wlf.name}: HS step, B={wlf.B}"
                    legs["hs_" + name] = lh
                del d
                torch.cuda.empty_cache()
            # the pages' geometry (192-value fp8 latent, 200-byte record) and
            # the native DSA indexer of the same group, batch 1 and 4
            from sparse_attention_indexer_latent_amd.runtime import DsaGroup
            for batch in (1, 4):
                wlp = W.hs_128k(batch, r=192, cache_dtype="fp8", scale_block=128)
                d = DeviceWorkload(wlp, hold_last=True)
                for hs_mode in (True, False):
                    lp = leg(torch, flush, d, hs_mode)
                    lp["workload"] = (f"{wlp.name}: {'HS' if hs_mode else 'full-scan'} step, "
                                      f"{d.cache.bytes_per_token} B/token (192 fp8 values + 2 "
                                      f"fp32 block scales), B={wlp.B}, k={wlp.k}")
                    legs[f"{'hs' if hs_mode else 'full_scan'}_128k_b{batch}_fp8r192"] = lp
                del d
                torch.cuda.empty_cache()
                legs[f"dsa_128k_b{batch}"] = dsa_leg(torch, flush, W, DsaGroup, batch)
                dsa = legs[f"dsa_128k_b{batch}"]
                hsp = legs[f"hs_128k_b{batch}_fp8r192"]
                out[f"hs_speedup_vs_dsa_128k_b{batch}"] = {
                    "fp8r192_200B": dsa["us_per_group_step"] / hsp["us_per_group_step"],
                    "fp8r192_200B_cold": dsa["cold_us_per_group_step"] / hsp["cold_us_per_group_step"],
                    "bf16r256": dsa["us_per_group_step"] / (
                        legs["hs_128k_b1"]["us_per_group_step"] if batch == 1 else us_step),
                    "pages_table4_context": "2.30-2.72x (ms per decode token, all 61 indexers, "
                                            "batch 1, eight unnamed GPUs)"}
            out["context_sweep"] = context_sweep(torch, W, DeviceWorkload, DsaGroup,
                                                 [8192, 16384, 32768, 65536, 131072])
            out["b_sweep"] = budget_sweep(torch, W, DeviceWorkload, [2048, 4096, 8192, 16384, 32768])
            out["b_sweep_correlated_layers"] = budget_sweep(
                torch, W, DeviceWorkload, [2048, 4096, 8192, 16384, 32768], layer_corr=0.9)
            wl8 = W.hs_128k(1, G=8, name="hs-128k-b1-bf16-r256-G8")
            d8 = DeviceWorkload(wl8, hold_last=True)
            for hs_mode in (True, False):
                l8 = leg(torch, flush, d8, hs_mode)
                l8["workload"] = (f"{wl8.name}: {'HS' if hs_mode else 'full-scan'} step of an "
                                  f"8-layer group (7 followers), B={wl8.B}")
                legs[f"{'hs' if hs_mode else 'full_scan'}_128k_b1_G8"] = l8
            del d8
            torch.cuda.empty_cache()
            out["legs"] = legs
        del flush

    if not args.no_prefill:
        out["prefill"] = prefill_leg(torch, ops, W, DeviceWorkload, args.prefill_iters)
    if not args.no_legs and not args.no_extra:
        out["calibration"] = calibration_leg(torch)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        out["gpu_over_cpu"] = out["value"] / out["cpu_baseline"]["value"]

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
