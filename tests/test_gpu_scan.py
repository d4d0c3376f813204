"""GPU parity of the full-scan decode scorer (li_score over a bf16 cache with
H = 64, r = 256 and at most 64 queries): many ragged queries on remapped
sequences with both q~ dtypes, every score against the oracle, nothing
written past a query's length; the batch-4 x 128K workload, sampled and
bit-identical across launches; and the whole HS decode step at that shape
(anchor, then three followers on 8192 candidates each)."""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload

from parity_util import RTOL_BF16, assert_scores_close, say

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


@pytest.mark.parametrize("qdt", ["fp32", "bf16"])
@pytest.mark.parametrize("with_beta", [False, True])
def test_scan_64_ragged_queries_every_score(qdt, with_beta):
    """64 queries over 64 sequences of 1 .. 3,000 tokens (one page, a page
    plus one token, ragged last pages), queries mapped to sequences by a
    permutation with repeats and cut to random prefixes, so the workgroup
    plan cannot be guessed and is computed from the lengths."""
    rng = np.random.default_rng(40)
    lens = [int(x) for x in rng.integers(1, 3001, 64)]
    lens[:6] = [1, 63, 64, 65, 128, 3000]
    say(f"scan: 64 ragged queries, q~ {qdt}, beta={with_beta}")
    wl = W.small_decode(41, n_seq=64, lens=lens, H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    n_q = 64
    q_seq = rng.permutation(64).astype(np.int32)
    q_seq[10:14] = q_seq[0]  # a few queries share a sequence
    q_len = np.array([rng.integers(1, lens[s] + 1) for s in q_seq], dtype=np.int32)
    q_len[:6] = [lens[s] for s in q_seq[:6]]
    qt = (rng.standard_normal((n_q, 64, 256)) * 0.1).astype(np.float32)
    if qdt == "bf16":
        bits = (qt.view(np.uint32) >> 16).astype(np.uint16)
        qt_dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        qt64 = O.bf16_decode(bits)
    else:
        qt_dev = torch.from_numpy(qt).cuda()
        qt64 = qt.astype(np.float64)
    w = (rng.standard_normal((n_q, 64)) / 8).astype(np.float32)
    beta = (rng.standard_normal((n_q, 64)) * 0.3).astype(np.float32) if with_beta else None
    max_len = int(q_len.max())
    out = torch.full((n_q, max_len + 3), SENTINEL, dtype=torch.float32, device="cuda")
    ops.score(qt_dev, torch.from_numpy(w).cuda(),
              None if beta is None else torch.from_numpy(beta).cuda(),
              torch.from_numpy(q_seq).cuda(), torch.from_numpy(q_len).cuda(), max_len, dw.cache,
              scores=out)
    torch.cuda.synchronize()
    u = out.cpu().numpy()
    lat = {}
    for i in range(n_q):
        s, n = int(q_seq[i]), int(q_len[i])
        if s not in lat:
            lat[s] = O.sequence_latent(wl, s)
        o = O.absorbed_scores(lat[s][:n], qt64[i],
                              None if beta is None else beta[i].astype(np.float64), w[i])
        assert_scores_close(u[i, :n], o, RTOL_BF16, f"query {i} (sequence {s}, {n} tokens)")
        assert np.all(u[i, n:] == SENTINEL), f"query {i}: wrote past its length"


def test_scan_batch4_128k_sampled_and_deterministic():
    """Four 128K-token sequences behind a random block table, absorbed fp32
    queries of layers 0 and 3: sampled tokens (first and last pages, planted
    tokens, 1,500 random) against the oracle, and a second launch
    bit-identical to the first."""
    wl = W.named("hs-128k-b4")
    say(f"scan: {wl.name}")
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(3)
    for l in (0, 3):
        dw.absorb(l)
        u1 = dw.score(l).clone()
        u2 = dw.score(l).clone()
        torch.cuda.synchronize()
        assert torch.equal(u1, u2), f"layer {l}: two launches differ"
        u = u1.cpu().numpy()
        for s in range(wl.n_q):
            seq, L = int(wl.q_seq[s]), int(wl.q_len[s])
            rows = np.unique(np.concatenate([rng.integers(0, L, 1500), np.arange(64),
                                             np.arange(L - 64, L),
                                             wl.planted[seq][wl.planted[seq] < L]]))
            C = O.store_latent(wl.latent(seq)[rows], wl.cache_dtype)[2]
            o = O.layer_scores(C, wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            assert_scores_close(u[s, rows], o, RTOL_BF16, f"layer {l} query {s}")


def test_hs_step_batch4_128k_followers():
    """The whole HS decode step at the benchmark's shape (four 128K-token
    queries, B = 8192, k = 2048, three followers): the anchor's candidates
    and selection exact on its dumped scores, every follower's candidate
    scores against the oracle, and every follower's selection exact on its
    dumped candidate scores."""
    wl = W.named("hs-128k-b4")
    say(f"HS step followers: {wl.name}")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.hs_step(append=False, keep_scores=True)
    torch.cuda.synchronize()
    u0 = dw.scores.cpu().numpy()
    cand = dw.cand.cpu().numpy()
    sel = dw.hs_sel.cpu().numpy()
    cs_all = dw.cand_scores.cpu().numpy()
    for s in range(wl.n_q):
        seq, L = int(wl.q_seq[s]), int(wl.q_len[s])
        row = u0[s, :L].astype(np.float64)
        assert np.array_equal(cand[s], O.pad(O.hs_candidates(row, wl.B), wl.B)), s
        assert np.array_equal(sel[0, s], O.pad(O.topk(row, wl.k), wl.k)), s
        C = O.store_latent(wl.latent(seq)[cand[s]], wl.cache_dtype)[2]
        for l in range(1, wl.G):
            cs = cs_all[l, s]
            o = O.layer_scores(C, wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            assert_scores_close(cs, o, RTOL_BF16, f"follower {l} query {s}")
            ref = O.pad(O.hs_follower(cand[s], cs.astype(np.float64), wl.k), wl.k)
            assert np.array_equal(sel[l, s], ref), (l, s)
