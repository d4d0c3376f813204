"""GPU parity of the issuer/compute scan for every cache shape it serves:
bf16 with r = 192 and 256, fp8 E4M3FN with r = 128, 192 and 256 and one
scale per token or one per 128-value block (r = 192 with two scales is the
pages' 200-byte record).  Page mode (many ragged queries on remapped
sequences, every score), candidate mode (HS followers), the fused anchor
(in-scan key histograms) and the quantiser's per-block scales."""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload, read_cache_rows

from parity_util import RTOL_BF16, RTOL_FP8, assert_scores_close, say

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0
SHAPES = [("bf16", 192, 0), ("fp8", 256, 0), ("fp8", 256, 128), ("fp8", 192, 0),
          ("fp8", 192, 128), ("fp8", 128, 0)]
RT = {"bf16": RTOL_BF16, "fp8": RTOL_FP8}


def _id(s):
    return f"{s[0]}-r{s[1]}-sb{s[2]}"


@pytest.mark.parametrize("shape", [("fp8", 192, 128), ("fp8", 256, 128), ("fp8", 128, 0)], ids=_id)
def test_append_per_block_scales_bit_exact(shape):
    dt, r, sb = shape
    say(f"append {_id(shape)}")
    wl = W.small_decode(81, n_seq=3, lens=[1, 130, 777], H=64, r=r, d_I=128, cache_dtype=dt,
                        plant=4, factor=4.0, scale_block=sb)
    dw = DeviceWorkload(wl, hold_last=False)
    assert dw.cache.bytes_per_token == r + 4 * (1 if sb == 0 else -(-r // sb))
    for s in range(wl.n_seq):
        L = int(wl.lens[s])
        data, scale = read_cache_rows(dw.cache, wl.block_table, s, L)
        stored, oscale, _ = O.store_latent(wl.latent(s), dt, sb)
        assert np.array_equal(np.asarray(data).reshape(stored.shape), stored), s
        assert np.array_equal(scale.view(np.uint32), oscale.view(np.uint32)), s


@pytest.mark.parametrize("qdt", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_scan_shapes_ragged_queries_every_score(shape, qdt):
    """64 queries over 64 sequences of 1 .. 3,000 tokens (unit edges at 64 and
    128), remapped to sequences with repeats and cut to random prefixes, with
    beta: every score against the oracle, nothing written past a length."""
    dt, r, sb = shape
    rng = np.random.default_rng(r + sb + (1 if qdt == "bf16" else 0))
    lens = [int(x) for x in rng.integers(1, 3001, 64)]
    lens[:9] = [1, 63, 64, 65, 127, 128, 129, 256, 3000]
    say(f"scan shape {_id(shape)}: 64 ragged queries, q~ {qdt}")
    wl = W.small_decode(82, n_seq=64, lens=lens, H=64, r=r, d_I=128, G=1, k=16, cache_dtype=dt,
                        scale_block=sb, plant=3, factor=3.0)
    dw = DeviceWorkload(wl, hold_last=False)
    n_q = 64
    q_seq = rng.permutation(64).astype(np.int32)
    q_seq[10:14] = q_seq[0]
    q_len = np.array([rng.integers(1, lens[s] + 1) for s in q_seq], dtype=np.int32)
    q_len[:9] = [lens[s] for s in q_seq[:9]]
    qt = (rng.standard_normal((n_q, 64, r)) * 0.1).astype(np.float32)
    qt[:, 7] *= 1e-3          # heads of very different magnitudes
    qt[:, 9] *= 1e3
    if qdt == "bf16":
        bits = (qt.view(np.uint32) >> 16).astype(np.uint16)
        qt_dev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        qt64 = O.bf16_decode(bits)
    else:
        qt_dev = torch.from_numpy(qt).cuda()
        qt64 = qt.astype(np.float64)
    w = (rng.standard_normal((n_q, 64)) / 8).astype(np.float32)
    beta = (rng.standard_normal((n_q, 64)) * 0.3).astype(np.float32)
    max_len = int(q_len.max())
    out = torch.full((n_q, max_len + 3), SENTINEL, dtype=torch.float32, device="cuda")
    ops.score(qt_dev, torch.from_numpy(w).cuda(), torch.from_numpy(beta).cuda(),
              torch.from_numpy(q_seq).cuda(), torch.from_numpy(q_len).cuda(), max_len, dw.cache,
              scores=out)
    torch.cuda.synchronize()
    u = out.cpu().numpy()
    lat = {}
    for i in range(n_q):
        s, n = int(q_seq[i]), int(q_len[i])
        if s not in lat:
            lat[s] = O.sequence_latent(wl, s)
        o = O.absorbed_scores(lat[s][:n], qt64[i], beta[i].astype(np.float64), w[i])
        assert_scores_close(u[i, :n], o, RT[dt], f"scan {_id(shape)} q~ {qdt} query {i}")
        assert np.all(u[i, n:] == SENTINEL), f"query {i}: wrote past its length"


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_scan_shapes_hs_followers(shape):
    """The followers' candidate rescoring on each shape: candidate scores
    against the oracle (-inf on padding), selections exact on them, and the
    anchor's fused scan + selection equal to li_score + li_hs_anchor_select."""
    dt, r, sb = shape
    say(f"HS on shape {_id(shape)}")
    wl = W.small_decode(83, n_seq=3, lens=[50, 1500, 4000], H=64, r=r, d_I=128, G=4, k=64, B=700,
                        cache_dtype=dt, scale_block=sb, plant=20, factor=3.0, nope_off=64,
                        bias=True)
    dw = DeviceWorkload(wl, hold_last=False)
    dw.hs_step(append=False, keep_scores=True)
    torch.cuda.synchronize()
    u_fused = dw.scores.cpu().numpy()
    cand = dw.cand.cpu().numpy()
    sel = dw.hs_sel.cpu().numpy()
    cs_all = dw.cand_scores.cpu().numpy()
    ref = ops.score(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, dw.max_len, dw.cache)
    rc, rs = ops.hs_anchor_select(ref, dw.q_len, dw.max_len, wl.B, wl.k)
    torch.cuda.synchronize()
    assert np.array_equal(cand, rc.cpu().numpy()) and np.array_equal(sel[0], rs.cpu().numpy())
    ur = ref.cpu().numpy()
    for s in range(wl.n_q):
        L = int(wl.q_len[s])
        assert np.array_equal(u_fused[s, :L].view(np.uint32), ur[s, :L].view(np.uint32)), s
        C = O.sequence_latent(wl, s)
        o0 = O.layer_scores(C[:L], wl.q[0, s], wl.Dt[0], wl.b[0], wl.nope_off, wl.w[0, s])
        assert_scores_close(u_fused[s, :L], o0, RT[dt], f"HS {_id(shape)} anchor query {s}")
        assert np.array_equal(cand[s], O.pad(O.hs_candidates(u_fused[s, :L].astype(np.float64),
                                                             wl.B), wl.B))
        nc = min(wl.B, L)
        for l in range(1, wl.G):
            cs = cs_all[l, s]
            assert np.all(np.isneginf(cs[nc:]))
            o = O.layer_scores(C[cand[s, :nc]], wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off,
                               wl.w[l, s])
            assert_scores_close(cs[:nc], o, RT[dt], f"HS {_id(shape)} follower {l} query {s}")
            refsel = O.pad(O.hs_follower(cand[s, :nc], cs[:nc].astype(np.float64), wl.k), wl.k)
            assert np.array_equal(sel[l, s], refsel), (l, s)


def test_dsa_comparator_group_step():
    """The native DSA comparator: four layers, each with its own fp8 key
    cache (128 values + one scale, 132 B per token), append then
    li_score_topk per layer.  Scores against the oracle (the raw query
    against each stored key), selections exact on the dumped scores and in
    the threshold band of the oracle's own scores."""
    from sparse_attention_indexer_latent_amd.runtime import DsaGroup
    from parity_util import assert_selection_band
    lens = [9000, 4100, 300]
    say(f"DSA comparator group step, lens {lens}")
    layers = [W.dsa_layer(l, lens, k=512) for l in range(4)]
    g = DsaGroup(layers)
    g.step()
    torch.cuda.synchronize()
    for l, d in enumerate(g.layers):
        wl = d.wl
        assert d.cache.bytes_per_token == 132
        u = d.scores.cpu().numpy()
        sel = d.sel[0].cpu().numpy()
        for s in range(wl.n_q):
            L = int(wl.q_len[s])
            K = O.sequence_latent(wl, s)[:L]
            o = O.absorbed_scores(K, wl.q[0, s].astype(np.float64), None, wl.w[0, s])
            assert_scores_close(u[s, :L], o, RTOL_FP8, f"DSA layer {l} query {s}")
            assert np.array_equal(sel[s], O.pad(O.topk(u[s, :L].astype(np.float64), wl.k), wl.k))
            assert_selection_band(sel[s], o, wl.k, RTOL_FP8, f"DSA layer {l} top-k query {s}")


@pytest.mark.parametrize("L", [8192, 16384])
def test_pages_geometry_hs_and_full_step(L):
    """The context sweep's batch-1 workload of the pages' geometry (192 fp8
    values + two block scales, B = 8192, k = 2048) at 8K (B covers the row:
    the candidate set is every position and the selections must equal the
    full-scan step's) and at 16K: every anchor and follower score against the
    oracle, every selection exact on the dumped scores."""
    say(f"pages' geometry HS and full step, L={L}")
    wl = W.hs_128k(1, r=192, cache_dtype="fp8", scale_block=128, L=L)
    dw = DeviceWorkload(wl, hold_last=False)
    dw.hs_step(append=False, keep_scores=True)
    torch.cuda.synchronize()
    u = dw.scores.cpu().numpy()[0, :L]
    cand = dw.cand.cpu().numpy()[0]
    hs_sel = dw.hs_sel.cpu().numpy()[:, 0]
    cs_all = dw.cand_scores.cpu().numpy()[:, 0]
    C = O.sequence_latent(wl, 0)[:L]
    o0 = O.layer_scores(C, wl.q[0, 0], wl.Dt[0], wl.b[0], wl.nope_off, wl.w[0, 0])
    assert_scores_close(u, o0, RTOL_FP8, f"pages' geometry L={L} anchor")
    assert np.array_equal(cand, O.pad(O.hs_candidates(u.astype(np.float64), wl.B), wl.B))
    assert np.array_equal(hs_sel[0], O.pad(O.topk(u.astype(np.float64), wl.k), wl.k))
    nc = min(wl.B, L)
    if L <= wl.B:
        assert np.array_equal(cand[:L], np.arange(L)) and np.all(cand[L:] == -1)
    for l in range(1, wl.G):
        cs = cs_all[l]
        o = O.layer_scores(C[cand[:nc]], wl.q[l, 0], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, 0])
        assert_scores_close(cs[:nc], o, RTOL_FP8, f"pages' geometry L={L} follower {l}")
        assert np.array_equal(hs_sel[l], O.pad(O.hs_follower(cand[:nc], cs[:nc].astype(np.float64),
                                                             wl.k), wl.k)), l
    if L <= wl.B:  # HS scores every position of every layer: it is the full scan
        dw.full_step(append=False)
        torch.cuda.synchronize()
        assert np.array_equal(dw.sel.cpu().numpy()[:, 0], hs_sel)
