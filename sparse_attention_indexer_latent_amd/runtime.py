"""Device-side driver of one layer group's decode step.

Uploads a synthetic workload, fills its paged latent cache through
li_append_latent, and runs the two decode variants of the LatentIndex
summary ("Methodology"):

* full scan: every layer absorbs its queries (eq. 6), scores the whole shared
  cache (eq. 8) and keeps its own top-k;
* hierarchical selection: the anchor scores everything and proposes its
  top-B candidates; each follower rescores and refines only those.

Every buffer a step touches is allocated up front, so a step allocates
nothing (and can be captured in a HIP graph).  All arithmetic runs in the
library's kernels; torch only owns memory and the stream.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import ops
from .workloads import BLOCK, Workload


def _t(a, dtype=None, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


class DeviceWorkload:
    def __init__(self, wl: Workload, device="cuda", hold_last: bool = True):
        """Upload wl.  With hold_last the cache receives positions 0..L-2 of
        each sequence; the decode step appends position L-1 (then scores L)."""
        self.wl = wl
        self.device = device
        bt = _t(wl.block_table, torch.int32, device)
        self.cache = ops.Cache.empty(wl.n_phys_blocks, wl.r, wl.cache_dtype, bt, device,
                                     scale_block=wl.scale_block)
        self.q_seq = _t(wl.q_seq, torch.int32, device)
        self.q_len = _t(wl.q_len, torch.int32, device)
        self.max_len = int(wl.q_len.max())
        G, H = wl.G, wl.H
        # every per-layer operand is stacked layer-major (index [l] is layer l)
        self.Dt = _t(wl.Dt, torch.float32, device)
        self.b = _t(wl.b, torch.float32, device) if wl.b.shape[1] else None
        self.w = _t(wl.w, torch.float32, device)
        self.q = _t(wl.q, torch.float32, device) if wl.q is not None else None
        self.fill_cache(hold_last)
        n_q = wl.n_q
        # last token of every sequence: appended by each decode step
        last = np.stack([wl.latent(s)[int(wl.lens[s]) - 1] for s in range(wl.n_seq)])
        self.x_new = _t(last, torch.float32, device)
        self.new_seq = torch.arange(wl.n_seq, dtype=torch.int32, device=device)
        self.new_pos = _t((wl.lens - 1).astype(np.int32), torch.int32, device)
        # per-step buffers
        r = wl.r
        self.q_tilde = torch.empty((G, n_q, H, r), dtype=torch.float32, device=device)
        self.beta = torch.empty((G, n_q, H), dtype=torch.float32, device=device)
        self.scores = torch.empty((n_q, self.max_len), dtype=torch.float32, device=device)
        self.sel = torch.empty((G, n_q, wl.k), dtype=torch.int32, device=device)
        self.topk_ws = self._ws(ops.lib().li_topk_workspace_bytes(n_q, self.max_len, max(wl.k, wl.B or 0)))
        if wl.B:
            self.cand = torch.empty((n_q, wl.B), dtype=torch.int32, device=device)
            self.hs_sel = torch.empty((G, n_q, wl.k), dtype=torch.int32, device=device)
            self.cand_scores = torch.empty((G, n_q, wl.B), dtype=torch.float32, device=device)
            self.hs_ws = ops.hs_workspace(n_q, wl.B, wl.k, device, n_f=max(G - 1, 1))
            self.anchor_ws = ops.hs_anchor_workspace(n_q, self.max_len, device)
        # the full-scan step's selections (li_score_topk; zeroed once)
        self.full_ws = ops.hs_anchor_workspace(n_q, self.max_len, device)

    def _ws(self, n):
        return torch.empty(n, dtype=torch.uint8, device=self.device) if n else None

    def fill_cache(self, hold_last: bool = True, chunk: int = 1 << 16) -> None:
        wl = self.wl
        for s in range(wl.n_seq):
            lat = wl.latent(s)
            L = int(wl.lens[s]) - (1 if hold_last else 0)
            for a in range(0, L, chunk):
                b = min(L, a + chunk)
                x = _t(lat[a:b], torch.float32, self.device)
                seq = torch.full((b - a,), s, dtype=torch.int32, device=self.device)
                pos = torch.arange(a, b, dtype=torch.int32, device=self.device)
                ops.append_latent(x, self.cache, seq, pos)
        torch.cuda.synchronize()

    # ---- steps -------------------------------------------------------------
    def append(self) -> None:
        ops.append_latent(self.x_new, self.cache, self.new_seq, self.new_pos)

    def absorb(self, layer: Optional[int] = None) -> None:
        """Absorb one layer's queries, or (layer None) all layers in one call."""
        if layer is None:
            ops.absorb_queries(self.q, self.Dt, self.b, self.wl.nope_off,
                               q_tilde=self.q_tilde, beta=self.beta)
        else:
            ops.absorb_queries(self.q[layer], self.Dt[layer],
                               None if self.b is None else self.b[layer], self.wl.nope_off,
                               q_tilde=self.q_tilde[layer], beta=self.beta[layer])

    def score(self, layer: int, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
        return ops.score(self.q_tilde[layer], self.w[layer], self.beta[layer], self.q_seq,
                         self.q_len, self.max_len, self.cache,
                         scores=self.scores if scores is None else scores)

    # A decode step is split into three parts so that a scan of the whole
    # cache (the dominant kernel) can be timed with events on its stream:
    # pre (append + every layer's absorb), scan (layer-0 score), post (the rest).
    def _pre(self, append: bool) -> None:
        if append:  # both in one launch
            ops.append_absorb(self.x_new, self.cache, self.new_seq, self.new_pos, self.q, self.Dt,
                              self.b, self.wl.nope_off, self.q_tilde, self.beta)
        else:
            self.absorb()

    def _full_post(self, keep_scores: bool = False) -> None:
        """Graph-capturable remainder of the two-call full-scan step: layer
        0's top-k (its scores are in place), then li_score + li_topk for the
        other layers."""
        wl = self.wl
        if keep_scores:
            self.full_scores[0].copy_(self.scores)
        ops.topk(self.scores, self.q_len, self.max_len, wl.k, out_idx=self.sel[0], ws=self.topk_ws)
        for l in range(1, wl.G):
            self.score(l)
            if keep_scores:
                self.full_scores[l].copy_(self.scores)
            ops.topk(self.scores, self.q_len, self.max_len, wl.k, out_idx=self.sel[l],
                     ws=self.topk_ws)

    def score_topk(self, layer: int, events=None) -> None:
        """One layer's full-scan step (li_score_topk): scores into
        self.scores, selection into self.sel[layer]."""
        raw = None if events is None else (events[0].e, events[1].e)
        ops.score_topk(self.q_tilde[layer], self.w[layer], self.beta[layer], self.q_seq,
                       self.q_len, self.max_len, self.cache, self.wl.k, scores=self.scores,
                       out_idx=self.sel[layer], ws=self.full_ws, scan_events=raw)

    def _hs_post(self, keep_scores: bool = False) -> None:
        wl = self.wl
        ops.hs_anchor_select(self.scores, self.q_len, self.max_len, wl.B, wl.k, cand=self.cand,
                             sel=self.hs_sel[0], ws=self.anchor_ws)
        self._hs_followers(keep_scores)

    def _hs_followers(self, keep_scores: bool = False) -> None:
        wl = self.wl
        if wl.G > 1:  # every follower at once: they share the candidate set
            ops.hs_select(self.cand, self.q_tilde[1:], self.w[1:],
                          self.beta[1:], self.q_seq, self.cache, wl.k, out_idx=self.hs_sel[1:],
                          cand_scores=self.cand_scores[1:] if keep_scores else None,
                          ws=self.hs_ws)

    def full_step(self, append: bool = True, events=None, keep_scores: bool = False,
                  two_call: bool = False) -> None:
        """Full-scan decode step of the group: every layer's queries absorbed,
        then per layer one li_score_topk call (scores and top-k).
        events: optional (start, end) events around layer 0's scoring launch
        (raw HIP events with an `e` handle, or torch events, which make layer
        0 run as li_score + li_topk around them).
        keep_scores (tests): also copy every layer's scores to full_scores
        [G, n_q, L] (allocated on first use).
        two_call: li_score + li_topk per layer instead (the graph-captured
        form of the step)."""
        self._pre(append)
        if keep_scores and getattr(self, "full_scores", None) is None:
            self.full_scores = torch.empty((self.wl.G,) + tuple(self.scores.shape),
                                           dtype=torch.float32, device=self.device)
        raw_ev = events is not None and getattr(events[0], "e", None) is not None
        if two_call or (events is not None and not raw_ev):
            if events is not None:
                events[0].record()
            self.score(0)
            if events is not None:
                events[1].record()
            self._full_post(keep_scores)
            return
        for l in range(self.wl.G):
            self.score_topk(l, events if l == 0 else None)
            if keep_scores:
                self.full_scores[l].copy_(self.scores)

    def hs_step(self, append: bool = True, keep_scores: bool = False, events=None) -> None:
        """Hierarchical-selection decode step: the anchor scans and proposes
        its top-B (one li_hs_anchor call), followers rescore and refine within
        the candidates.  events: optional (start, end) events around the
        anchor's scoring launch: raw HIP events (an `e` handle) go into the
        call; torch events make the anchor run as two calls around them."""
        self._pre(append)
        raw = None if events is None else (getattr(events[0], "e", None), getattr(events[1], "e", None))
        if raw is not None and (raw[0] is None or raw[1] is None):  # torch events: separate calls
            events[0].record()
            self.score(0)
            events[1].record()
            self._hs_post(keep_scores)
            return
        wl = self.wl
        ops.hs_anchor(self.q_tilde[0], self.w[0], self.beta[0], self.q_seq, self.q_len,
                      self.max_len, self.cache, wl.B, wl.k, scores=self.scores, cand=self.cand,
                      sel=self.hs_sel[0], ws=self.anchor_ws, scan_events=raw)
        self._hs_followers(keep_scores)

    def capture(self, hs: bool, append: bool = True, keep_scores: bool = False) -> "StepGraphs":
        """Capture one decode step as graphs around the scan (see StepGraphs)."""
        return StepGraphs(self, hs, append, keep_scores)


class StepGraphs:
    """A decode step as two HIP graphs around one direct launch of the scan.

    pre (append + every layer's absorb) and post (selections and the other layers)
    are captured graphs; the layer-0 scan between them is launched directly
    through a pre-marshalled call, so events recorded around it time exactly
    that kernel on its stream.  The library allocates nothing, so every replay
    reuses the same buffers and reproduces an eager step."""

    def __init__(self, dw: DeviceWorkload, hs: bool, append: bool = True,
                 keep_scores: bool = False):
        post = (lambda: dw._hs_post(keep_scores)) if hs else dw._full_post
        self.scan = ops.prepared_score(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len,
                                       dw.max_len, dw.cache, dw.scores)
        parts = [lambda: dw._pre(append), post]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside capture (one-time attributes)
            for f in parts:
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graphs = []
        for f in parts:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                f()
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self, events=None) -> None:
        pre, post = self.graphs
        pre.replay()
        if events is not None:
            events[0].record()
        self.scan()
        if events is not None:
            events[1].record()
        post.replay()


class DsaGroup:
    """The native DSA indexer over the same G layers, for comparison: each
    layer appends its new token's key to its own fp8 key cache and scores
    that cache with its own queries (no shared latent, no absorption: the
    query itself takes the absorbed query's place), then keeps its top-k,
    all through the same library calls (li_append_latent, li_score_topk)."""

    def __init__(self, layers, device="cuda"):
        self.layers = [DeviceWorkload(wl, device=device, hold_last=True) for wl in layers]

    def step(self, events=None) -> None:
        for i, d in enumerate(self.layers):
            d.append()
            raw = None if (events is None or i) else (events[0].e, events[1].e)
            ops.score_topk(d.q[0], d.w[0], None, d.q_seq, d.q_len, d.max_len, d.cache, d.wl.k,
                           scores=d.scores, out_idx=d.sel[0], ws=d.full_ws, scan_events=raw)

    def scan0(self) -> None:
        d = self.layers[0]
        ops.score(d.q[0], d.w[0], None, d.q_seq, d.q_len, d.max_len, d.cache, scores=d.scores)


def read_cache_rows(cache: ops.Cache, block_table: np.ndarray, s: int, L: int):
    """Host copy of sequence s's first L stored rows (and scales) in token order."""
    nblk = (L + BLOCK - 1) // BLOCK
    blocks = torch.as_tensor(block_table[s, :nblk].astype(np.int64), device=cache.data.device)
    src = cache.data.view(torch.int16) if cache.data.dtype == torch.bfloat16 else cache.data
    data = src.index_select(0, blocks).reshape(nblk * BLOCK, -1)[:L].cpu().numpy()
    if cache.data.dtype == torch.bfloat16:
        data = data.view(np.uint16)
    scale = None
    if cache.scale is not None:
        sc = cache.scale.index_select(0, blocks)
        ns = sc.numel() // (nblk * BLOCK)
        scale = sc.reshape(nblk * BLOCK, ns)[:L].cpu().numpy()
        if cache.scale_block == 0:
            scale = scale[:, 0].copy()
    return data, scale
