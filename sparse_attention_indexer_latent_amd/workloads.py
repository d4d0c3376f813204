"""Seeded synthetic workloads for the LatentIndex decode indexer.

This module only draws random inputs and arranges them into shapes: it holds
none of the method's arithmetic (no absorption, scoring, selection or
quantisation).  Both the CPU oracle (through the tests and the bench's CPU leg)
and the HIP path consume exactly the arrays produced here.

Shapes follow the LatentIndex paper summary (picx.dev, "Methodology"): one
shared latent c_t of width d_C (= r here) per token per layer group, per-layer
decoders D^(l) that map it to d_I-wide indexer keys (eq. 3), per-head queries
q_{s,h} of width d_I and head weights w_{s,h} (eq. 8), groups of four layers
(explainer page, storage paragraph), k = 2048 and a candidate budget B = 8192
(Table 4 caption text).

Every array comes from its own counter-seeded NumPy PCG64 stream,
``default_rng([seed, cfg_id, stream])``, so any part (one sequence's latent,
one layer's queries) can be regenerated alone, identically on every machine.

Stream ids:
  1            context lengths (ragged configurations)
  1000 + s     latent rows of sequence s, then its planted-token choice
  2000         decoders: the shared matrix G0, then one noise matrix per layer
  3000 + l     queries, then head weights, of layer l
  4000         physical block permutation (block table)
  5000 + l     prefill absorbed queries and head weights of layer l

Readings taken where the configuration text is terse:
  * D_l = (G0 + 0.3 * G_l) / sqrt(r), G0 and G_l i.i.d. N(0, 1), stored
    transposed as Dt_l of shape [r, d_I] and shared by all heads of the layer.
  * Planted tokens are drawn uniformly without replacement; their latent rows
    are multiplied by the planting factor before any quantisation.
  * Ragged lengths are round(exp(U[ln 8192, ln 131072])).
  * Queries q ~ N(0, 1) and head weights w ~ N(0, 1)/sqrt(H) per (layer,
    query, head), independent across layers unless a layer correlation rho
    is asked for: then each layer's draw is rho x a group-shared draw +
    sqrt(1 - rho^2) x its own.
  * The prefill chunk's absorbed queries are drawn directly on the bf16 grid
    (an N(0, d_I*(1+0.3^2)/r) fp32 draw rounded to bf16, nearest-even), which
    matches the variance of Dt_l @ q without this module doing the absorption
    itself.
  * The decode step appends the last token of each sequence: the cache holds
    positions 0..L-2 before the step and 0..L-1 after it; layer queries score
    all L positions (causal set inclusive of the current token).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK = 64  # tokens per paged latent block


@dataclasses.dataclass
class Workload:
    """One synthetic configuration.  All arrays are host NumPy arrays."""

    name: str
    cfg_id: int
    seed: int
    G: int                       # layers per group (layer 0 is the anchor)
    H: int                       # indexer heads
    r: int                       # latent width d_C
    d_I: int                     # indexer key width
    k: int                       # per-layer top-k
    B: Optional[int]             # HS candidate budget (None: full scan only)
    cache_dtype: str             # "fp32" | "bf16" | "fp8"
    lens: np.ndarray             # int64 [n_seq] context lengths L_s
    block_table: np.ndarray      # int32 [n_seq, max_blocks], -1 = unused
    n_phys_blocks: int
    nope_off: int                # key coordinates [nope_off, d_I) carry the bias b
    Dt: np.ndarray               # fp32 [G, r, d_I]  (D_l transposed)
    b: np.ndarray                # fp32 [G, d_I - nope_off]
    q: Optional[np.ndarray]      # fp32 [G, n_q, H, d_I]   (decode)
    w: np.ndarray                # fp32 [G, n_q, H]
    q_seq: np.ndarray            # int32 [n_q] sequence of each query
    q_len: np.ndarray            # int32 [n_q] causal prefix length of each query
    planted: list                # per sequence: int64 array of planted token ids
    plant_factor: float
    _latent: Optional[list] = None   # per-sequence fp32 [L_s, r], drawn lazily
    prefill_positions: Optional[np.ndarray] = None  # int64 [n_q] (prefill only)
    scale_block: int = 0             # fp8 cache: 0 (one scale per token) or 128

    @property
    def n_seq(self) -> int:
        return int(self.lens.shape[0])

    @property
    def n_q(self) -> int:
        return int(self.q_seq.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_len(self) -> int:
        return int(self.lens.max())

    def latent(self, s: int) -> np.ndarray:
        """fp32 [L_s, r] latent rows of sequence s (planted rows scaled)."""
        if self._latent is None:
            self._latent = [None] * self.n_seq
        if self._latent[s] is None:
            self._latent[s] = _draw_latent(self, s)[0]
        return self._latent[s]

    def drop_latents(self) -> None:
        self._latent = None

    def prefill_queries(self, layer: int) -> tuple[np.ndarray, np.ndarray]:
        """(q_tilde bf16 bit patterns uint16 [n_q, H, r], w fp32 [n_q, H])."""
        assert self.prefill_positions is not None
        rng = _rng(self.seed, self.cfg_id, 5000 + layer)
        std = math.sqrt(self.d_I * (1.0 + 0.3 ** 2) / self.r)
        qt = rng.standard_normal((self.n_q, self.H, self.r), dtype=np.float32)
        qt *= np.float32(std)
        u = qt.view(np.uint32).astype(np.uint64)
        bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # nearest, ties to even
        w = rng.standard_normal((self.n_q, self.H), dtype=np.float32)
        w *= np.float32(1.0 / math.sqrt(self.H))
        return bits, w


def _rng(seed: int, cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg_id), int(stream)])


def _draw_latent(wl: Workload, s: int):
    rng = _rng(wl.seed, wl.cfg_id, 1000 + s)
    L = int(wl.lens[s])
    lat = rng.standard_normal((L, wl.r), dtype=np.float32)
    n_plant = len(wl.planted[s])
    idx = rng.choice(L, size=n_plant, replace=False) if n_plant else np.zeros(0, np.int64)
    idx = np.sort(idx.astype(np.int64))
    lat[idx] *= np.float32(wl.plant_factor)
    return lat, idx


def _planted_ids(seed, cfg_id, s, L, n_plant, r):
    # The planted choice is drawn from the latent stream after the latent rows.
    rng = _rng(seed, cfg_id, 1000 + s)
    rng.standard_normal((L, r), dtype=np.float32)
    idx = rng.choice(L, size=n_plant, replace=False) if n_plant else np.zeros(0, np.int64)
    return np.sort(idx.astype(np.int64))


def _block_table(seed, cfg_id, lens, permute):
    nblk = [(int(L) + BLOCK - 1) // BLOCK for L in lens]
    total = sum(nblk)
    max_blocks = max(nblk)
    if permute:
        perm = _rng(seed, cfg_id, 4000).permutation(total).astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    bt = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblk):
        bt[s, :n] = perm[off:off + n]
        off += n
    return bt, total


def _decoders(seed, cfg_id, G, r, d_I):
    rng = _rng(seed, cfg_id, 2000)
    g0 = rng.standard_normal((r, d_I), dtype=np.float32)
    Dt = np.empty((G, r, d_I), dtype=np.float32)
    inv = np.float32(1.0 / math.sqrt(r))
    for l in range(G):
        gl = rng.standard_normal((r, d_I), dtype=np.float32)
        Dt[l] = (g0 + np.float32(0.3) * gl) * inv
    return Dt


def _queries(seed, cfg_id, G, n_q, H, d_I, layer_corr=0.0):
    """Per-layer queries and head weights; with layer_corr = rho > 0 every
    layer's draw is rho x a draw shared by the group + sqrt(1 - rho^2) x its
    own (same marginal distribution, correlation rho between layers)."""
    q = np.empty((G, n_q, H, d_I), dtype=np.float32)
    w = np.empty((G, n_q, H), dtype=np.float32)
    sw = np.float32(1.0 / math.sqrt(H))
    if layer_corr:
        rng0 = _rng(seed, cfg_id, 3100)
        q0 = rng0.standard_normal((n_q, H, d_I), dtype=np.float32)
        w0 = rng0.standard_normal((n_q, H), dtype=np.float32)
        a = np.float32(layer_corr)
        c = np.float32(math.sqrt(1.0 - layer_corr ** 2))
    for l in range(G):
        rng = _rng(seed, cfg_id, 3000 + l)
        q[l] = rng.standard_normal((n_q, H, d_I), dtype=np.float32)
        w[l] = rng.standard_normal((n_q, H), dtype=np.float32)
        if layer_corr:
            q[l] = a * q0 + c * q[l]
            w[l] = a * w0 + c * w[l]
        w[l] *= sw
    return q, w


def make_decode(name, cfg_id, seed, *, G, H, r, d_I, k, B, cache_dtype, lens,
                plant_frac=None, n_plant=None, plant_factor, permute_blocks,
                nope_off=None, bias=False, scale_block=0, layer_corr=0.0) -> Workload:
    lens = np.asarray(lens, dtype=np.int64)
    n_seq = len(lens)
    planted = []
    for s in range(n_seq):
        L = int(lens[s])
        n = n_plant if n_plant is not None else int(round(plant_frac * L))
        n = min(n, L)
        planted.append(_planted_ids(seed, cfg_id, s, L, n, r))
    bt, nphys = _block_table(seed, cfg_id, lens, permute_blocks)
    Dt = _decoders(seed, cfg_id, G, r, d_I)
    q, w = _queries(seed, cfg_id, G, n_seq, H, d_I, layer_corr)
    no = d_I if nope_off is None else nope_off
    b = np.zeros((G, d_I - no), dtype=np.float32)
    if bias and d_I - no > 0:
        b = _rng(seed, cfg_id, 2001).standard_normal((G, d_I - no), dtype=np.float32)
    return Workload(
        name=name, cfg_id=cfg_id, seed=seed, G=G, H=H, r=r, d_I=d_I, k=k, B=B,
        cache_dtype=cache_dtype, lens=lens, block_table=bt, n_phys_blocks=nphys,
        nope_off=no, Dt=Dt, b=b, q=q, w=w,
        q_seq=np.arange(n_seq, dtype=np.int32), q_len=lens.astype(np.int32),
        planted=planted, plant_factor=plant_factor, scale_block=scale_block)


def ragged_lens(seed, cfg_id, n, lo=8192, hi=131072):
    u = _rng(seed, cfg_id, 1).uniform(math.log(lo), math.log(hi), size=n)
    return np.rint(np.exp(u)).astype(np.int64)


WORKLOADS = ("tiny-4k", "dsv32-decode-32k", "ragged-16x8k-128k-fp8", "hs-128k-b4",
             "prefill-2048x64k")


def named(name: str, seed: int = 0) -> Workload:
    """The five synthetic workloads, by name.

    tiny-4k                 1 sequence, L=4096, H=8, r=32, d_I=64, fp32 cache,
                            k=256, 16 planted tokens x4 (CPU-seconds parity case).
    dsv32-decode-32k        DeepSeek-V3.2-shaped decode at 32K: H=64, r=256,
                            d_I=128, bf16 cache, batch 1, k=2048, 1% planted x3.
    ragged-16x8k-128k-fp8   batched long decode: 16 sequences, ragged
                            log-uniform 8K-128K, fp8 e4m3 cache with per-token
                            fp32 scale, 64-token pages behind a random block
                            table, k=2048.
    hs-128k-b4              HS at 128K: batch 4, L=131072 each, bf16, paged as
                            the ragged workload, B=8192, k=2048.
    prefill-2048x64k        prefill chunk: 2048 queries at positions
                            63488..65535 against a 65536-token bf16 latent,
                            H=64, r=256, causal, k=2048.
    """
    if name == "tiny-4k":
        return make_decode("tiny-4k", 0, seed, G=4, H=8, r=32, d_I=64, k=256, B=None,
                           cache_dtype="fp32", lens=[4096], n_plant=16, plant_factor=4.0,
                           permute_blocks=False)
    if name == "dsv32-decode-32k":
        return make_decode("dsv32-decode-32k", 1, seed, G=4, H=64, r=256, d_I=128, k=2048,
                           B=None, cache_dtype="bf16", lens=[32768], plant_frac=0.01,
                           plant_factor=3.0, permute_blocks=False)
    if name == "ragged-16x8k-128k-fp8":
        return make_decode("ragged-16x8k-128k-fp8", 2, seed, G=4, H=64, r=256, d_I=128,
                           k=2048, B=None, cache_dtype="fp8", lens=ragged_lens(seed, 2, 16),
                           plant_frac=0.01, plant_factor=3.0, permute_blocks=True)
    if name == "hs-128k-b4":
        return make_decode("hs-128k-b4", 3, seed, G=4, H=64, r=256, d_I=128, k=2048, B=8192,
                           cache_dtype="bf16", lens=[131072] * 4, plant_frac=0.01,
                           plant_factor=3.0, permute_blocks=True)
    if name == "prefill-2048x64k":
        return make_prefill(seed)
    raise ValueError(f"no workload {name!r}; known: {', '.join(WORKLOADS)}")


def hs_128k(batch: int, seed: int = 0, r: int = 256, cache_dtype: str = "bf16",
            scale_block: int = 0, B: int = 8192, G: int = 4, name: str = None,
            layer_corr: float = 0.0, L: int = 131072) -> Workload:
    """The 128K hierarchical-selection workload (hs-128k-b4's generator) at
    any batch, latent width, cache type, candidate budget and
    group size (and, for a sweep over context lengths, any length L).
    r = 192 with an fp8 cache and scale_block = 128 is the
    DeepSeek-V3.2 geometry of the LatentIndex explainer's storage paragraph
    (192 values, a 200-byte record)."""
    name = name or (f"hs-{L // 1024}k-b{batch}-{cache_dtype}-r{r}"
                    + (f"-sb{scale_block}" if scale_block else "")
                    + (f"-rho{layer_corr:g}" if layer_corr else ""))
    return make_decode(name, 3 if r == 256 else 5, seed, G=G, H=64, r=r, d_I=128, k=2048, B=B,
                       cache_dtype=cache_dtype, lens=[L] * batch, plant_frac=0.01,
                       plant_factor=3.0, permute_blocks=True, scale_block=scale_block,
                       layer_corr=layer_corr)


def dsa_layer(layer: int, lens, seed: int = 0, H: int = 64, d_I: int = 128,
              k: int = 2048) -> Workload:
    """One layer of a native DSA indexer, the comparator of the pages' Table 4:
    the layer's own key cache of d_I fp8 values and one fp32 scale per token
    (132 bytes at d_I = 128), queries [n_q, H, d_I] and head weights, no
    shared latent.  Its keys are seeded draws of their own (1 % of tokens
    planted x3); the queries score them directly (the absorbed-query slot
    holds the raw query)."""
    return make_decode(f"dsa-key-layer{layer}", 30 + layer, seed, G=1, H=H, r=d_I, d_I=d_I, k=k,
                       B=None, cache_dtype="fp8", lens=list(lens), plant_frac=0.01,
                       plant_factor=3.0, permute_blocks=True)


def calibration_set(seed: int = 0, n: int = 4096, d_model: int = 96, m: int = 4, d_R: int = 16,
                    d_N: int = 32, noise: float = 0.1):
    """Synthetic calibration inputs for one group: anchor hidden states X
    [n, d_model] (per-feature scales log-uniform in [0.3, 3]), and per layer
    the draws of a native indexer's key projections W_R[l] [d_model, d_R] and
    W_N[l] [d_model, d_N], each a shared part plus 0.3x a layer part over
    sqrt(d_model) (the layers' keys are then X W, which the caller forms),
    key-noise draws E[l] [n, d_R + d_N] scaled by `noise`, NoPE key offsets
    [m, d_N], and the keys' rotary frequencies [d_R / 2] (10000^(-2j/d_R))."""
    rng = _rng(seed, 70, 1)
    X = rng.standard_normal((n, d_model), dtype=np.float32)
    X *= np.exp(rng.uniform(np.log(0.3), np.log(3.0), d_model)).astype(np.float32)
    inv = np.float32(1.0 / math.sqrt(d_model))
    w0R = rng.standard_normal((d_model, d_R), dtype=np.float32)
    w0N = rng.standard_normal((d_model, d_N), dtype=np.float32)
    WR = np.stack([(w0R + np.float32(0.3) * rng.standard_normal((d_model, d_R), dtype=np.float32)) * inv
                   for _ in range(m)])
    WN = np.stack([(w0N + np.float32(0.3) * rng.standard_normal((d_model, d_N), dtype=np.float32)) * inv
                   for _ in range(m)])
    E = rng.standard_normal((m, n, d_R + d_N), dtype=np.float32) * np.float32(noise)
    off = rng.standard_normal((m, d_N), dtype=np.float32)
    theta = (10000.0 ** (-np.arange(d_R // 2) * 2.0 / d_R)).astype(np.float32)
    return X, WR, WN, E, off, theta


def make_prefill(seed: int = 0, n_q: int = 2048, L: int = 65536, H: int = 64, r: int = 256,
                 d_I: int = 128, k: int = 2048, G: int = 4, cfg_id: int = 4) -> Workload:
    lens = np.array([L], dtype=np.int64)
    planted = [_planted_ids(seed, cfg_id, 0, L, int(round(0.01 * L)), r)]
    bt, nphys = _block_table(seed, cfg_id, lens, False)
    pos = np.arange(L - n_q, L, dtype=np.int64)
    w = np.empty((G, n_q, H), dtype=np.float32)
    wl = Workload(
        name=f"prefill-{n_q}x{L // 1024}k", cfg_id=cfg_id, seed=seed, G=G, H=H, r=r, d_I=d_I,
        k=k, B=None, cache_dtype="bf16", lens=lens, block_table=bt, n_phys_blocks=nphys,
        nope_off=d_I, Dt=np.zeros((G, r, d_I), np.float32), b=np.zeros((G, 0), np.float32),
        q=None, w=w, q_seq=np.zeros(n_q, dtype=np.int32), q_len=(pos + 1).astype(np.int32),
        planted=planted, plant_factor=3.0, prefill_positions=pos)
    for l in range(G):
        w[l] = wl.prefill_queries(l)[1]
    return wl


def small_decode(seed: int, *, n_seq=2, lens=None, H=8, r=32, d_I=16, G=2, k=16, B=None,
                 cache_dtype="fp32", nope_off=None, bias=False, plant=0, factor=4.0,
                 permute=True, cfg_id=90, scale_block=0) -> Workload:
    """A tiny decode workload for fast tests (ragged lengths allowed)."""
    if lens is None:
        lens = [100 + 37 * s for s in range(n_seq)]
    return make_decode(f"small-{cfg_id}", cfg_id, seed, G=G, H=H, r=r, d_I=d_I, k=k, B=B,
                       cache_dtype=cache_dtype, lens=lens, n_plant=plant, plant_factor=factor,
                       permute_blocks=permute, nope_off=nope_off, bias=bias,
                       scale_block=scale_block)
