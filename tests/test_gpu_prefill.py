"""GPU parity of the prefill path: many bf16 absorbed queries per sequence
scored on the matrix cores (li_score's prefill scorer), then each row's
top-k (li_topk over many long rows)."""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload

from parity_util import RTOL_BF16, assert_scores_close, assert_selection_band, say

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _bf16_queries(rng, n_q, H=64, r=256, scale=0.5):
    x = (rng.standard_normal((n_q, H, r)) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def _score(bits, w, beta, q_seq, q_len, max_len, cache, ld):
    out = torch.full((len(q_seq), ld), SENTINEL, dtype=torch.float32, device="cuda")
    ops.score(_dev_bf16(bits), torch.from_numpy(w).cuda(),
              None if beta is None else torch.from_numpy(beta).cuda(),
              torch.from_numpy(q_seq).cuda(), torch.from_numpy(q_len).cuda(), max_len, cache,
              scores=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_rows(u, bits, w, beta, q_seq, q_len, lat, rows, what):
    qt = O.bf16_decode(bits)
    for i in rows:
        n = int(q_len[i])
        o = O.absorbed_scores(lat[int(q_seq[i])][:n], qt[i],
                              None if beta is None else beta[i].astype(np.float64), w[i])
        assert_scores_close(u[i, :n], o, RTOL_BF16, f"{what} query {i}")
        assert np.all(u[i, n:] == SENTINEL), f"{what} query {i}: wrote past its causal prefix"


@pytest.mark.parametrize("with_beta", [False, True])
def test_prefill_chunk_small_every_score(with_beta):
    """One sequence, a causal chunk of 200 queries (a ragged last group of
    eight) at the end of a 2,500-token context (a ragged last page, pages in
    every one of the eight token ranges); every score is checked."""
    L, n_q = 2500, 200
    say(f"prefill scorer: {n_q} queries x {L} tokens, beta={with_beta}")
    wl = W.small_decode(21, n_seq=1, lens=[L], H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(8)
    bits = _bf16_queries(rng, n_q)
    w = rng.standard_normal((n_q, 64)).astype(np.float32) / 8
    beta = (rng.standard_normal((n_q, 64)) * 0.5).astype(np.float32) if with_beta else None
    q_seq = np.zeros(n_q, np.int32)
    q_len = np.arange(L - n_q + 1, L + 1, dtype=np.int32)
    u = _score(bits, w, beta, q_seq, q_len, L, dw.cache, L + 5)
    lat = [O.sequence_latent(wl, 0)]
    _check_rows(u, bits, w, beta, q_seq, q_len, lat, range(n_q), "small chunk")


def test_prefill_queries_over_several_sequences():
    """Queries of one workgroup that read different sequences (served in
    rounds), random causal lengths including 1 and a full context."""
    lens = [700, 1500, 130]
    n_q = 96
    say(f"prefill scorer: {n_q} queries over sequences of {lens}")
    wl = W.small_decode(22, n_seq=3, lens=lens, H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(9)
    bits = _bf16_queries(rng, n_q)
    w = rng.standard_normal((n_q, 64)).astype(np.float32) / 8
    beta = (rng.standard_normal((n_q, 64)) * 0.5).astype(np.float32)
    q_seq = rng.integers(0, 3, n_q).astype(np.int32)
    q_len = np.array([rng.integers(1, lens[s] + 1) for s in q_seq], dtype=np.int32)
    q_len[0], q_len[5] = 1, lens[q_seq[5]]
    max_len = int(q_len.max())
    u = _score(bits, w, beta, q_seq, q_len, max_len, dw.cache, max_len)
    lat = [O.sequence_latent(wl, s) for s in range(3)]
    _check_rows(u, bits, w, beta, q_seq, q_len, lat, range(n_q), "3 sequences")


def _prefill_rows(n_q, rng):
    """64 rows checked in full (the first and last rows, the edges of the
    first and last eight-query workgroups, the middle, random rows) and every
    eight-query workgroup boundary pair (8j - 1, 8j) checked on sampled
    tokens."""
    fixed = [0, 1, 7, 8, 15, 16, 1023, 1024, n_q - 8, n_q - 2, n_q - 1]
    rest = rng.choice(np.setdiff1d(np.arange(n_q), fixed), 64 - len(fixed), replace=False)
    full = sorted(set(fixed) | set(int(x) for x in rest))
    bound = sorted(set(j for b in range(8, n_q, 8) for j in (b - 1, b)) - set(full))
    return full, bound


def test_prefill_config4_all_layers_scores_and_topk():
    """2,048 queries at positions 63,488..65,535 over a 64K-token bf16
    latent, per-row top-2,048, all four layers: 64 full rows per layer
    against the oracle, their selections bit-exact against the oracle's
    selection over the same (GPU) scores and within the threshold band of the
    oracle's own scores; every workgroup-boundary row on sampled tokens (the
    first and last 64 positions of its prefix and 512 random ones)."""
    wl = W.named("prefill-2048x64k")
    say(f"prefill config: {wl.name}")
    dw = DeviceWorkload(wl, hold_last=False)
    lat = O.sequence_latent(wl, 0)
    n_q, L, k = wl.n_q, int(wl.lens[0]), wl.k
    rng = np.random.default_rng(44)
    full, bound = _prefill_rows(n_q, rng)
    assert len(full) == 64 and 0 in full and n_q - 1 in full
    for layer in range(wl.G):
        bits, w = wl.prefill_queries(layer)
        say(f"  layer {layer}: score")
        u_dev = torch.full((n_q, L), SENTINEL, dtype=torch.float32, device="cuda")
        ops.score(_dev_bf16(bits), torch.from_numpy(w).cuda(), None, dw.q_seq, dw.q_len, L,
                  dw.cache, scores=u_dev)
        say(f"  layer {layer}: top-{k}")
        idx = ops.topk(u_dev, dw.q_len, L, k)
        torch.cuda.synchronize()
        u = u_dev[full].cpu().numpy()
        sel = idx[full].cpu().numpy()
        qt = O.bf16_decode(bits[full])
        for j, i in enumerate(full):
            n = int(wl.q_len[i])
            assert n == 63489 + i
            o = O.absorbed_scores(lat[:n], qt[j], None, w[i])
            assert_scores_close(u[j, :n], o, RTOL_BF16, f"prefill layer {layer} full row {i}")
            assert np.all(u[j, n:] == SENTINEL)
            ref = O.pad(O.topk(u[j, :n].astype(np.float64), k), k)
            assert np.array_equal(sel[j], ref), f"layer {layer} row {i}: top-k differs"
            assert_selection_band(sel[j], o, k, RTOL_BF16, f"prefill layer {layer} full row {i}")
        ub = u_dev[bound].cpu().numpy()
        qb = O.bf16_decode(bits[bound])
        for j, i in enumerate(bound):
            n = int(wl.q_len[i])
            t = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                          rng.integers(0, n, 512)]))
            o = O.absorbed_scores(lat[t], qb[j], None, w[i])
            assert_scores_close(ub[j, t], o, RTOL_BF16, f"prefill layer {layer} boundary row {i}")
            assert np.all(ub[j, n:] == SENTINEL)
