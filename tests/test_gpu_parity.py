"""GPU parity of every C-ABI call against the CPU oracle (MI355X only)."""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload, read_cache_rows

from parity_util import (RTOL_BF16, RTOL_FP8, RTOL_FP32, assert_scores_close,
                         assert_selection_band, say)

pytestmark = pytest.mark.gpu


def test_device_is_gfx950():
    assert ops.lib().li_check_device() == ops.LI_OK


# ------------------------------------------------------------------ append ---

@pytest.mark.parametrize("dtype,r", [("fp32", 32), ("bf16", 256), ("fp8", 256), ("fp8", 64)])
def test_append_matches_oracle_quantiser_bit_exact(dtype, r):
    say(f"append exact dtype={dtype} r={r}")
    wl = W.small_decode(1, n_seq=3, lens=[1, 130, 777], r=r, H=8, d_I=16, cache_dtype=dtype,
                        plant=4, factor=4.0)
    dw = DeviceWorkload(wl, hold_last=False)
    for s in range(wl.n_seq):
        L = int(wl.lens[s])
        data, scale = read_cache_rows(dw.cache, wl.block_table, s, L)
        stored, oscale, _ = O.store_latent(wl.latent(s), dtype)
        assert np.array_equal(np.asarray(data).view(stored.dtype).reshape(stored.shape), stored), s
        if dtype == "fp8":
            assert np.array_equal(scale.view(np.uint32), oscale.view(np.uint32)), s


def test_append_zero_row_and_extremes_fp8():
    say("append fp8 zero row and extremes")
    r = 64
    rows = np.zeros((5, r), np.float32)
    rows[1, 3] = 1e-30
    rows[2] = np.linspace(-1000, 1000, r, dtype=np.float32)
    rows[3, :] = -2.5
    rows[4] = np.random.default_rng(0).standard_normal(r).astype(np.float32) * 1e-5
    bt = torch.arange(1, dtype=torch.int32, device="cuda").reshape(1, 1)
    cache = ops.Cache.empty(1, r, "fp8", bt)
    ops.append_latent(torch.from_numpy(rows).cuda(), cache, torch.zeros(5, dtype=torch.int32, device="cuda"),
                      torch.arange(5, dtype=torch.int32, device="cuda"))
    codes, oscale = O.quantize_fp8(rows)
    got = cache.data[0, :5].cpu().numpy()
    assert np.array_equal(got, codes)
    assert np.array_equal(cache.scale[0, :5].cpu().numpy().view(np.uint32), oscale.view(np.uint32))


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp8"])
@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_append_projection_and_rope(dtype, xdt):
    say(f"append with P and rope dtype={dtype} x={xdt}")
    rng = np.random.default_rng(5)
    n_tok, d_model, r, r_R = 37, 300, 64, 16
    x = rng.standard_normal((n_tok, d_model)).astype(np.float32)
    P = (rng.standard_normal((d_model, r)) / np.sqrt(d_model)).astype(np.float32)
    theta = (10000.0 ** (-np.arange(r_R // 2) * 2.0 / r_R)).astype(np.float32)
    pos = rng.permutation(200)[:n_tok].astype(np.int32)
    xt = torch.from_numpy(x).cuda().to(xdt)
    Pt = torch.from_numpy(P).cuda().to(xdt)
    xe = xt.float().cpu().numpy()
    Pe = Pt.float().cpu().numpy()
    bt = torch.arange(4, dtype=torch.int32, device="cuda").reshape(1, 4)
    cache = ops.Cache.empty(4, r, dtype, bt)
    ops.append_latent(xt, cache, torch.zeros(n_tok, dtype=torch.int32, device="cuda"),
                      torch.from_numpy(pos).cuda(), P=Pt, rope_theta=torch.from_numpy(theta).cuda())
    ref = O.project_latent(xe, Pe, theta, pos)              # float64, eqs. 1-2
    data = cache.data.reshape(256, r)[pos.astype(np.int64)].cpu()
    if dtype == "fp32":
        got = data.numpy().astype(np.float64)
        tol = 1e-5 * np.abs(ref).max()
    elif dtype == "bf16":
        got = data.float().numpy().astype(np.float64)
        tol = np.abs(ref) * 2.0 ** -7 + 1e-6               # one bf16 rounding
    else:
        sc = cache.scale.reshape(256)[pos.astype(np.int64)].cpu().numpy()
        got = O.dequantize_fp8(data.numpy(), sc)
        tol = np.abs(ref) * 2.0 ** -3 + sc[:, None] * 2.0 ** -9 * 1.01
    assert np.all(np.abs(got - ref) <= tol)
    # the rotation preserves each pair's norm and leaves the N branch alone
    if dtype == "fp32":
        nr = np.hypot(got[:, 0:r_R:2], got[:, 1:r_R:2])
        y = xe.astype(np.float64) @ Pe.astype(np.float64)
        assert np.allclose(nr, np.hypot(y[:, 0:r_R:2], y[:, 1:r_R:2]), rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------ absorb ---

@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("qdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n_layers", [1, 3])
def test_absorb_matches_oracle(per_head, qdt, n_layers):
    """One layer, or several layers (each with its own decoder and bias)
    stacked into one call."""
    say(f"absorb per_head={per_head} q={qdt} layers={n_layers}")
    rng = np.random.default_rng(9 + n_layers)
    n_q, H, d_I, r, no = 3, 64, 128, 256, 64
    q = rng.standard_normal((n_layers, n_q, H, d_I)).astype(np.float32)
    Dt = (rng.standard_normal((n_layers, H, r, d_I) if per_head else (n_layers, r, d_I)) / 16
          ).astype(np.float32)
    b = rng.standard_normal((n_layers, d_I - no)).astype(np.float32)
    q_dev = torch.from_numpy(q).cuda().to(qdt)
    qe = q_dev.float().cpu().numpy()
    if n_layers == 1:
        qt, beta = ops.absorb_queries(q_dev[0], torch.from_numpy(Dt[0]).cuda(),
                                      torch.from_numpy(b[0]).cuda(), no, per_head=per_head)
        qt, beta = qt[None], beta[None]
    else:
        qt, beta = ops.absorb_queries(q_dev, torch.from_numpy(Dt).cuda(), torch.from_numpy(b).cuda(),
                                      no, per_head=per_head)
    qt, beta = qt.cpu().numpy(), beta.cpu().numpy()
    for l in range(n_layers):
        for s in range(n_q):
            oq, ob = O.absorb(qe[l, s], Dt[l], b[l], no)
            assert np.max(np.abs(qt[l, s] - oq)) <= 1e-5 * np.abs(oq).max(), (l, s)
            assert np.max(np.abs(beta[l, s] - ob)) <= 1e-5 * (np.abs(ob).max() + 1), (l, s)


@pytest.mark.parametrize("dtype,per_head,xdt,qdt,n_tok,n_q", [
    ("bf16", False, torch.float32, torch.float32, 37, 4),
    ("fp8", True, torch.bfloat16, torch.bfloat16, 61, 3),
    ("fp32", False, torch.float32, torch.bfloat16, 0, 2),
    ("bf16", True, torch.bfloat16, torch.float32, 5, 0),
])
def test_append_absorb_equals_the_two_calls(dtype, per_head, xdt, qdt, n_tok, n_q):
    """The one-launch prelude writes exactly what li_append_latent (no
    projection, with rope) and li_absorb_queries write, bit for bit; both of
    those are checked against the oracle above."""
    say(f"append_absorb dtype={dtype} per_head={per_head} x={xdt} q={qdt} n_tok={n_tok} n_q={n_q}")
    rng = np.random.default_rng(17 + n_tok + n_q)
    r, r_R, L, H, d_I, no = 256, 64, 3, 64, 128, 64
    x = torch.from_numpy(rng.standard_normal((n_tok, r)).astype(np.float32)).cuda().to(xdt)
    theta = torch.from_numpy((10000.0 ** (-np.arange(r_R // 2) * 2.0 / r_R)).astype(np.float32)).cuda()
    seq = torch.from_numpy(rng.integers(0, 2, n_tok).astype(np.int32)).cuda()
    pos = torch.from_numpy(rng.permutation(256)[:n_tok].astype(np.int32)).cuda()
    q = torch.from_numpy(rng.standard_normal((L, n_q, H, d_I)).astype(np.float32)).cuda().to(qdt)
    Dt = torch.from_numpy((rng.standard_normal((L, H, r, d_I) if per_head else (L, r, d_I)) / 16
                           ).astype(np.float32)).cuda()
    b = torch.from_numpy(rng.standard_normal((L, d_I - no)).astype(np.float32)).cuda()
    bt = torch.arange(8, dtype=torch.int32, device="cuda").reshape(2, 4)
    caches, outs = [], []
    for fused in (False, True):
        cache = ops.Cache.empty(8, r, dtype, bt)
        cache.data.view(torch.uint8).fill_(0x5a)  # same prior contents for both
        if cache.scale is not None:
            cache.scale.fill_(3.0)
        qt = torch.full((L, n_q, H, r), 7.0, device="cuda")
        beta = torch.full((L, n_q, H), 7.0, device="cuda")
        if fused:
            ops.append_absorb(x, cache, seq, pos, q, Dt, b, no, qt, beta, rope_theta=theta,
                              per_head=per_head)
        else:
            if n_tok:
                ops.append_latent(x, cache, seq, pos, rope_theta=theta)
            if n_q:
                ops.absorb_queries(q, Dt, b, no, q_tilde=qt, beta=beta, per_head=per_head)
        caches.append(cache)
        outs.append((qt, beta))
    torch.cuda.synchronize()
    assert torch.equal(caches[0].data.view(torch.uint8), caches[1].data.view(torch.uint8))
    if dtype == "fp8":
        assert torch.equal(caches[0].scale, caches[1].scale)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ------------------------------------------------------------------- score ---

def _scores_vs_oracle(wl, dw, rtol, layers=None, sample=None):
    layers = range(wl.G) if layers is None else layers
    for l in layers:
        say(f"  score layer {l}")
        dw.absorb(l)
        dw.score(l)
        torch.cuda.synchronize()
        u = dw.scores.cpu().numpy()
        for s in range(wl.n_q):
            seq = int(wl.q_seq[s])
            L = int(wl.q_len[s])
            C = O.sequence_latent(wl, seq)[:L]
            rows = np.arange(L) if sample is None else np.unique(
                np.concatenate([sample(L), wl.planted[seq][wl.planted[seq] < L]]))
            o = O.layer_scores(C[rows], wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            assert_scores_close(u[s, rows], o, rtol, f"layer {l} query {s}")


def test_score_valu_tiny_config_fp32():
    say("score VALU, tiny workload (L 4096, H 8, r 32, fp32)")
    wl = W.named("tiny-4k")
    dw = DeviceWorkload(wl, hold_last=False)
    _scores_vs_oracle(wl, dw, RTOL_FP32)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp8"])
def test_score_small_ragged_with_bias(dtype):
    say(f"score small ragged with bias dtype={dtype} (H=64, r=256)")
    wl = W.small_decode(2, n_seq=3, lens=[1, 95, 700], H=64, r=256, d_I=128, G=2, k=16,
                        cache_dtype=dtype, nope_off=64, bias=True, plant=3, factor=3.0)
    dw = DeviceWorkload(wl, hold_last=False)
    _scores_vs_oracle(wl, dw, {"fp32": RTOL_FP32, "bf16": RTOL_BF16, "fp8": RTOL_FP8}[dtype])


def test_score_bf16_queries_single_pass():
    """A stored bf16 q~ (prefill form) is scored exactly as given."""
    say("score with bf16 q~ input (H=64, r=256)")
    wl = W.small_decode(3, n_seq=2, lens=[300, 129], H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(1)
    bits = (rng.standard_normal((2, 64, 256)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qt = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    u = ops.score(qt, dw.w[0], None, dw.q_seq, dw.q_len, dw.max_len, dw.cache)
    torch.cuda.synchronize()
    qt64 = O.bf16_decode(bits)
    for s in range(2):
        C = O.sequence_latent(wl, s)
        o = O.absorbed_scores(C, qt64[s], None, wl.w[0, s])
        assert_scores_close(u[s, :len(o)].cpu().numpy(), o, 1e-5, f"bf16 q~ query {s}")


@pytest.mark.parametrize("dtype,H", [("bf16", 8), ("fp8", 8), ("bf16", 64), ("fp8", 64)])
def test_score_valu_r192(dtype, H):
    """A latent of 192 values (the pages' DeepSeek-V3.2 width) takes the
    vector-ALU scorer for every cache type: ragged lengths, a bias on half
    of the key, every score against the oracle."""
    say(f"score r=192 dtype={dtype} H={H} (VALU path)")
    wl = W.small_decode(31, n_seq=3, lens=[1, 200, 1500], H=H, r=192, d_I=128, G=2, k=16,
                        cache_dtype=dtype, nope_off=64, bias=True, plant=5, factor=3.0)
    dw = DeviceWorkload(wl, hold_last=False)
    _scores_vs_oracle(wl, dw, {"bf16": RTOL_BF16, "fp8": RTOL_FP8}[dtype])


def test_score_config1_32k_bf16():
    say("score 32K batch-1 workload (H=64, r=256, bf16): all 4 layers")
    wl = W.named("dsv32-decode-32k")
    dw = DeviceWorkload(wl, hold_last=False)
    _scores_vs_oracle(wl, dw, RTOL_BF16)


def test_score_plan_guess_holds_and_falls_back():
    """The matrix-core scorer guesses the common decode plan (every query
    ceil(max_len/64) pages long, query q on sequence q).  Scores must match
    the oracle whether the guess holds or not: remapped sequences, a larger
    max_len, and lengths that differ only inside the last page."""
    say("score plan guess: holds / wrong sequence map / wrong page count / last-page raggedness")
    L = 1000  # 16 pages; sequence 3 is longer, so the block table has room for 18
    wl = W.small_decode(11, n_seq=4, lens=[L, L, L, L + 100], H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16", nope_off=64, bias=True)
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb(0)
    lat = [O.sequence_latent(wl, s) for s in range(4)]

    def run(q_seq, q_len, max_len, case):
        qs = torch.tensor(q_seq, dtype=torch.int32, device="cuda")
        ql = torch.tensor(q_len, dtype=torch.int32, device="cuda")
        u = ops.score(dw.q_tilde[0], dw.w[0], dw.beta[0], qs, ql, max_len, dw.cache).cpu().numpy()
        for s in range(len(q_seq)):
            n = q_len[s]
            o = O.layer_scores(lat[q_seq[s]][:n], wl.q[0, s], wl.Dt[0], wl.b[0], wl.nope_off,
                               wl.w[0, s])
            assert_scores_close(u[s, :n], o, RTOL_BF16, f"{case}: query {s}")

    run([0, 1, 2, 3], [L, L, L, L], L, "guess holds")
    run([3, 0, 1, 2], [L, L, L, L], L, "sequences remapped")
    run([0, 1, 2, 3], [L, L, L, L], L + 64, "max_len one page larger")
    run([0, 1, 2, 3], [L, L - 7, L - 30, L - 1], L, "lengths differ inside the last page")
    run([1, 1, 1, 3], [L - 500, L, 64, L + 100], L + 100, "ragged, shared sequence")


def test_score_config2_fp8_sampled():
    """The ragged fp8 workload at full size (16 sequences, 8K-128K, fp8 cache behind a
    random block table) on the matrix-core path: sampled tokens of every
    query, first and last pages included, against the oracle."""
    say("score ragged workload (16 sequences, fp8 E4M3 + per-token scale): layers 0 and 3, sampled")
    wl = W.named("ragged-16x8k-128k-fp8")
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(2)
    for l in (0, 3):
        dw.absorb(l)
        u = dw.score(l).cpu().numpy()
        for s in range(wl.n_q):
            seq, L = int(wl.q_seq[s]), int(wl.q_len[s])
            rows = np.unique(np.concatenate([rng.integers(0, L, 1500), np.arange(64),
                                             np.arange(L - 64, L),
                                             wl.planted[seq][wl.planted[seq] < L]]))
            C = O.store_latent(wl.latent(seq)[rows], wl.cache_dtype)[2]  # per-token quantiser
            o = O.layer_scores(C, wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            assert_scores_close(u[s, rows], o, RTOL_FP8, f"layer {l} query {s} (L={L})")


@pytest.mark.parametrize("qdt", ["fp32", "bf16"])
def test_score_fp8_wide_head_range(qdt):
    """fp8 cache with q~ whose heads span 2^-20 .. 2^20 in magnitude, one head
    all zero and one holding a single non-zero: each head's fp8 split is scaled
    on its own."""
    say(f"score fp8 cache, q~ {qdt} with heads of very different magnitudes")
    wl = W.small_decode(12, n_seq=2, lens=[777, 130], H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="fp8")
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(3)
    qt = rng.standard_normal((2, 64, 256)) * np.exp2(rng.integers(-20, 21, (2, 64, 1)))
    qt[:, 5] = 0.0
    qt[:, 9] = 0.0
    qt[:, 9, 17] = 3.0
    if qdt == "bf16":
        bits = (qt.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        qt64 = O.bf16_decode(bits)
        qdev = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        qt64 = qt.astype(np.float32).astype(np.float64)
        qdev = torch.from_numpy(qt.astype(np.float32)).cuda()
    w = rng.standard_normal((2, 64)).astype(np.float32)
    beta = rng.standard_normal((2, 64)).astype(np.float32) * 1e-3
    u = ops.score(qdev, torch.from_numpy(w).cuda(), torch.from_numpy(beta).cuda(), dw.q_seq,
                  dw.q_len, dw.max_len, dw.cache).cpu().numpy()
    for s in range(2):
        C = O.sequence_latent(wl, s)
        o = O.absorbed_scores(C, qt64[s], beta[s].astype(np.float64), w[s])
        assert_scores_close(u[s, :len(o)], o, RTOL_FP8, f"query {s}")


def test_score_more_than_64_queries():
    """Batches above 64 queries take the workgroup scorer; both paths agree
    with the oracle."""
    say("score with 70 queries over 3 sequences (bf16, H=64)")
    lens = [300, 1000, 64]
    wl = W.small_decode(13, n_seq=3, lens=lens, H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16", nope_off=64, bias=True)
    dw = DeviceWorkload(wl, hold_last=False)
    rng = np.random.default_rng(5)
    n_q = 70
    qs = rng.integers(0, 3, n_q).astype(np.int32)
    ql = np.array([rng.integers(1, lens[s] + 1) for s in qs], dtype=np.int32)
    qt = rng.standard_normal((n_q, 64, 256)).astype(np.float32) * 0.1
    w = rng.standard_normal((n_q, 64)).astype(np.float32)
    beta = rng.standard_normal((n_q, 64)).astype(np.float32) * 0.1
    for nq in (n_q, 64):
        u = ops.score(torch.from_numpy(qt[:nq]).cuda(), torch.from_numpy(w[:nq]).cuda(),
                      torch.from_numpy(beta[:nq]).cuda(), torch.from_numpy(qs[:nq]).cuda(),
                      torch.from_numpy(ql[:nq]).cuda(), int(ql[:nq].max()), dw.cache).cpu().numpy()
        lat = [O.sequence_latent(wl, s) for s in range(3)]
        for i in range(nq):
            n = int(ql[i])
            o = O.absorbed_scores(lat[qs[i]][:n], qt[i].astype(np.float64),
                                  beta[i].astype(np.float64), w[i])
            assert_scores_close(u[i, :n], o, RTOL_BF16, f"n_q={nq} query {i}")


# ------------------------------------------------------------------- top-k ---

def _topk_gpu(u, lens, k):
    ut = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).cuda()
    vl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    idx, val = ops.topk(ut, vl, u.shape[1], k, want_val=True)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def _check_topk_exact(u, lens, k):
    idx, val = _topk_gpu(u, lens, k)
    for i in range(u.shape[0]):
        n = int(lens[i])
        ref = O.pad(O.topk(u[i, :n].astype(np.float64), k), k)
        assert np.array_equal(idx[i], ref), f"row {i}: n={n} k={k}"
        m = min(k, n)
        assert np.array_equal(val[i, :m].view(np.uint32), u[i, ref[:m]].astype(np.float32).view(np.uint32))
        assert np.all(np.isneginf(val[i, m:]))


@pytest.mark.parametrize("k", [1, 7, 256, 2048, 8192])
def test_topk_exact_random_rows(k):
    say(f"topk exact random k={k}")
    rng = np.random.default_rng(k)
    lens = [0, 1, 5, 1000, 4096, 33333, 70000]
    u = rng.standard_normal((len(lens), 70000)).astype(np.float32)
    _check_topk_exact(u, lens, k)


def test_topk_exact_ties_and_signed_zero():
    say("topk exact with heavy ties, signed zeros, all-equal rows")
    rng = np.random.default_rng(3)
    n = 20000
    rows = [np.round(rng.standard_normal(n), 1),
            np.zeros(n),
            np.where(rng.random(n) < 0.5, -0.0, 0.0),
            np.full(n, 3.25),
            np.concatenate([np.full(n // 2, 1.0), np.full(n - n // 2, 2.0)]),
            rng.choice([-np.inf, 0.0, 1.0], n)]
    u = np.stack(rows).astype(np.float32)
    for k in [1, 100, 2048, 9999, 20000, 30000]:
        _check_topk_exact(u, [n] * len(rows), k)


def _check_topk_exact_sample(u, lens, k, rows):
    """As _check_topk_exact, with every row selected on the GPU and the
    listed rows compared."""
    idx, val = _topk_gpu(u, lens, k)
    for i in rows:
        n = int(lens[i])
        ref = O.pad(O.topk(u[i, :n].astype(np.float64), k), k)
        assert np.array_equal(idx[i], ref), f"row {i}: n={n} k={k}"
        m = min(k, n)
        assert np.array_equal(val[i, :m].view(np.uint32), u[i, ref[:m]].astype(np.float32).view(np.uint32))
        assert np.all(np.isneginf(val[i, m:]))


@pytest.mark.parametrize("k", [1, 2048, 8192])
def test_topk_many_long_rows_exact(k):
    """More than 64 rows longer than 16K (one workgroup per row, the row held
    in registers), an odd row stride (unaligned rows), ragged lengths around
    the 4,096-position load blocks and k."""
    say(f"topk many long rows k={k}")
    rng = np.random.default_rng(100 + k)
    n_rows, ld = 80, 65537
    u = rng.standard_normal((n_rows, ld)).astype(np.float32)
    edge = [0, 1, k - 1, k, k + 1, 4095, 4096, 4097, 16385, 32767, 32768, 32769, 65535, 65536]
    lens = np.array(edge + list(rng.integers(16385, 65537, n_rows - len(edge))), dtype=np.int32)
    lens = np.clip(lens, 0, 65536)
    rows = list(range(len(edge))) + list(rng.choice(np.arange(len(edge), n_rows), 6, replace=False))
    _check_topk_exact_sample(u, lens, k, rows)


def test_topk_many_rows_ties_and_signed_zero():
    say("topk many long rows: heavy ties, signed zeros, all-equal rows")
    rng = np.random.default_rng(4)
    n = 40000
    base = [np.round(rng.standard_normal(n), 1),
            np.zeros(n),
            np.where(rng.random(n) < 0.5, -0.0, 0.0),
            np.full(n, 3.25),
            np.concatenate([np.full(n // 2, 1.0), np.full(n - n // 2, 2.0)]),
            rng.choice([-np.inf, 0.0, 1.0], n),
            rng.integers(0, 4, n) * 0.5]
    u = np.stack([base[i % len(base)] for i in range(70)]).astype(np.float32)
    for k in [1, 100, 2048, 9999, 39999]:
        _check_topk_exact_sample(u, [n] * len(u), k, range(len(base)))


@pytest.mark.parametrize("B,k", [(8192, 2048), (300, 300), (5000, 1)])
def test_hs_anchor_select_nested_exact(B, k):
    say(f"hs_anchor_select B={B} k={k}")
    rng = np.random.default_rng(B + k)
    lens = [0, 17, 4096, 60000, 131072]
    u = np.round(rng.standard_normal((len(lens), 131072)), 2).astype(np.float32)  # ties
    ut = torch.from_numpy(u).cuda()
    vl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    cand, sel = ops.hs_anchor_select(ut, vl, 131072, B, k)
    torch.cuda.synchronize()
    cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
    for i, n in enumerate(lens):
        row = u[i, :n].astype(np.float64)
        assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, B), B)), i
        assert np.array_equal(sel[i], O.pad(O.topk(row, k), k)), i


@pytest.mark.parametrize("B,k", [(8192, 2048), (3000, 2048), (5000, 1)])
def test_hs_anchor_select_short_rows_exact(B, k):
    """Rows of at most 8192 positions take one single-workgroup launch per
    selection; both outputs exact against the oracle (ties included), and a
    long-row call on the same workspace afterwards is still exact."""
    say(f"hs_anchor_select short rows B={B} k={k}")
    rng = np.random.default_rng(3 * B + k)
    lens = [0, 1, 17, 2048, 5000, 8191, 8192]
    u = np.round(rng.standard_normal((len(lens), 8192)), 2).astype(np.float32)
    ws = ops.hs_anchor_workspace(len(lens), 131072)
    cand, sel = ops.hs_anchor_select(torch.from_numpy(u).cuda(),
                                     torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(),
                                     8192, B, k, ws=ws)
    torch.cuda.synchronize()
    cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
    for i, n in enumerate(lens):
        row = u[i, :n].astype(np.float64)
        assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, B), B)), i
        assert np.array_equal(sel[i], O.pad(O.topk(row, k), k)), i
    ul = np.round(rng.standard_normal((2, 40000)), 2).astype(np.float32)
    ll = np.asarray([40000, 31000], dtype=np.int32)
    cand, sel = ops.hs_anchor_select(torch.from_numpy(ul).cuda(), torch.from_numpy(ll).cuda(),
                                     40000, B, k, ws=ws)
    torch.cuda.synchronize()
    cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
    for i, n in enumerate(ll):
        row = ul[i, :n].astype(np.float64)
        assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, B), B)), ("long", i)
        assert np.array_equal(sel[i], O.pad(O.topk(row, k), k)), ("long", i)


def test_hs_anchor_select_reuses_one_workspace():
    """One workspace across calls of different row counts and lengths (each
    call leaves its counting arrays zeroed for the next), every result exact."""
    say("hs_anchor_select: one workspace, several calls")
    rng = np.random.default_rng(77)
    ws = ops.hs_anchor_workspace(6, 131072)
    for n_rows, L, B, k in [(5, 131072, 8192, 2048), (3, 40000, 4000, 100), (6, 131072, 8192, 2048),
                            (1, 5000, 300, 7), (5, 131072, 8192, 2048)]:
        u = np.round(rng.standard_normal((n_rows, L)), 3).astype(np.float32)
        lens = rng.integers(1, L + 1, n_rows).astype(np.int32)
        lens[0] = L
        cand, sel = ops.hs_anchor_select(torch.from_numpy(u).cuda(), torch.from_numpy(lens).cuda(),
                                         L, B, k, ws=ws)
        torch.cuda.synchronize()
        cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
        for i in range(n_rows):
            row = u[i, :lens[i]].astype(np.float64)
            assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, B), B)), (n_rows, L, i)
            assert np.array_equal(sel[i], O.pad(O.topk(row, k), k)), (n_rows, L, i)


@pytest.mark.parametrize("case", ["ragged", "batch4_128k", "fp32_cache", "bf16_q_beta"])
def test_hs_anchor_fused_equals_two_calls(case):
    """li_hs_anchor (scores with the key histograms built by the scorer, then
    the selection) gives the bits of li_score followed by
    li_hs_anchor_select, call after call on one workspace, and the oracle's
    selection of the dumped scores; fp32_cache takes the unfused route."""
    say(f"hs_anchor fused: {case}")
    if case == "ragged":
        wl = W.small_decode(12, n_seq=5, lens=[1, 63, 700, 4000, 9000], H=64, r=256, d_I=128, G=1,
                            k=64, B=512, cache_dtype="bf16")
    elif case == "fp32_cache":
        wl = W.small_decode(13, n_seq=3, lens=[40, 900, 5000], H=8, r=32, d_I=16, G=1, k=16, B=100,
                            cache_dtype="fp32")
    elif case == "bf16_q_beta":  # stored bf16 absorbed queries, a bias on half the dims
        wl = W.small_decode(14, n_seq=4, lens=[3000, 70, 12000, 6500], H=64, r=256, d_I=128, G=1,
                            k=100, B=1000, cache_dtype="bf16", nope_off=64, bias=True)
    else:
        wl = W.named("hs-128k-b4")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb(0)
    n_q, L = wl.n_q, dw.max_len
    qt = dw.q_tilde[0].to(torch.bfloat16) if case == "bf16_q_beta" else dw.q_tilde[0]
    if case == "bf16_q_beta":
        assert float(dw.beta[0].abs().max()) > 0
    ws = ops.hs_anchor_workspace(n_q, L)
    for rep in range(2):
        sc, cand, sel = ops.hs_anchor(qt, dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, L,
                                      dw.cache, wl.B, wl.k, ws=ws)
        ref = ops.score(qt, dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, L, dw.cache)
        rc, rs = ops.hs_anchor_select(ref, dw.q_len, L, wl.B, wl.k)
        torch.cuda.synchronize()
        u, ur = sc.cpu().numpy(), ref.cpu().numpy()
        cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
        for i in range(n_q):
            n = int(wl.q_len[i])
            assert np.array_equal(u[i, :n].view(np.uint32), ur[i, :n].view(np.uint32)), (rep, i)
        assert np.array_equal(cand, rc.cpu().numpy()) and np.array_equal(sel, rs.cpu().numpy()), rep
        for i in range(n_q):
            row = u[i, :int(wl.q_len[i])].astype(np.float64)
            assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, wl.B), wl.B)), (rep, i)
            assert np.array_equal(sel[i], O.pad(O.topk(row, wl.k), wl.k)), (rep, i)


@pytest.mark.parametrize("case", ["bf16_fused", "fp8", "fp32_tiny", "65_queries"])
def test_score_topk_equals_score_then_topk(case):
    """li_score_topk (one call; the scorer builds the key histograms for a
    bf16 cache with H = 64, r = 256 and <= 64 queries) gives the bits of
    li_score followed by li_topk, call after call on one workspace."""
    say(f"score_topk: {case}")
    if case == "bf16_fused":
        wl = W.small_decode(70, n_seq=4, lens=[9000, 40, 4100, 13000], H=64, r=256, d_I=128, G=1,
                            k=2048, cache_dtype="bf16", nope_off=64, bias=True)
    elif case == "fp8":
        wl = W.small_decode(71, n_seq=3, lens=[5000, 12000, 700], H=64, r=256, d_I=128, G=1,
                            k=512, cache_dtype="fp8")
    elif case == "fp32_tiny":
        wl = W.small_decode(72, n_seq=2, lens=[4096, 300], H=8, r=32, d_I=16, G=1, k=256,
                            cache_dtype="fp32")
    else:
        rng = np.random.default_rng(73)
        wl = W.small_decode(73, n_seq=65, lens=[int(x) for x in rng.integers(100, 6000, 65)],
                            H=64, r=256, d_I=128, G=1, k=64, cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb(0)
    L = dw.max_len
    ws = ops.hs_anchor_workspace(wl.n_q, L)
    for rep in range(2):
        sc, idx = ops.score_topk(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, L,
                                 dw.cache, wl.k, ws=ws)
        ref = ops.score(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, L, dw.cache)
        ridx = ops.topk(ref, dw.q_len, L, wl.k)
        torch.cuda.synchronize()
        u, ur = sc.cpu().numpy(), ref.cpu().numpy()
        for i in range(wl.n_q):
            n = int(wl.q_len[i])
            assert np.array_equal(u[i, :n].view(np.uint32), ur[i, :n].view(np.uint32)), (rep, i)
        assert torch.equal(idx, ridx), rep
        got = idx.cpu().numpy()
        for i in range(wl.n_q):
            n = int(wl.q_len[i])
            assert np.array_equal(got[i], O.pad(O.topk(u[i, :n].astype(np.float64), wl.k), wl.k))


@pytest.mark.parametrize("n_seq", [64, 65])
def test_hs_anchor_many_queries(n_seq):
    """64 queries (the most whose key histograms the scorer builds) and 65
    (the two-call route), ragged lengths from one page to 9,000 tokens:
    li_hs_anchor equals li_score + li_hs_anchor_select bit for bit, and the
    selections are the oracle's on the dumped scores."""
    say(f"hs_anchor with {n_seq} queries")
    rng = np.random.default_rng(n_seq)
    lens = [int(x) for x in rng.integers(40, 9001, n_seq)]
    lens[:3] = [40, 4096, 9000]
    wl = W.small_decode(16, n_seq=n_seq, lens=lens, H=64, r=256, d_I=128, G=1, k=32, B=300,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb(0)
    L = dw.max_len
    sc, cand, sel = ops.hs_anchor(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, L,
                                  dw.cache, wl.B, wl.k)
    ref = ops.score(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, L, dw.cache)
    rc, rs = ops.hs_anchor_select(ref, dw.q_len, L, wl.B, wl.k)
    torch.cuda.synchronize()
    u, ur = sc.cpu().numpy(), ref.cpu().numpy()
    cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
    assert np.array_equal(cand, rc.cpu().numpy()) and np.array_equal(sel, rs.cpu().numpy())
    for i in range(wl.n_q):
        n = int(wl.q_len[i])
        assert np.array_equal(u[i, :n].view(np.uint32), ur[i, :n].view(np.uint32)), i
        row = u[i, :n].astype(np.float64)
        assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, wl.B), wl.B)), i
        assert np.array_equal(sel[i], O.pad(O.topk(row, wl.k), wl.k)), i


def test_hs_anchor_candidates_only_and_scan_events():
    """li_hs_anchor with sel = NULL returns the candidate set alone, and its
    two timing events bracket the scoring launch (recorded, ordered)."""
    import ctypes
    say("hs_anchor: candidates only, scan events")
    wl = W.small_decode(15, n_seq=2, lens=[5000, 9000], H=64, r=256, d_I=128, G=1, k=50, B=700,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb(0)
    hip = ctypes.CDLL("libamdhip64.so")
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        sc, cand, sel = ops.hs_anchor(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len,
                                      dw.max_len, dw.cache, wl.B, wl.k, want_sel=False,
                                      scan_events=ev)
        torch.cuda.synchronize()
        assert sel is None
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 1000.0
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
    u, cand = sc.cpu().numpy(), cand.cpu().numpy()
    for i in range(wl.n_q):
        row = u[i, :int(wl.q_len[i])].astype(np.float64)
        assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, wl.B), wl.B)), i


@pytest.mark.parametrize("n", [16384, 9000, 8192, 5001])
def test_topk_exact_short_rows_in_lds(n):
    """Rows of at most 16K elements take the LDS-resident path, rows of at
    most 8,192 the register-resident one (5,001: an odd row stride, so rows
    are not 16-byte aligned)."""
    say(f"topk exact, LDS-resident rows n={n}")
    rng = np.random.default_rng(n)
    rows = [rng.standard_normal(n), np.round(rng.standard_normal(n), 1), np.zeros(n),
            np.where(rng.random(n) < 0.5, -0.0, 0.0), rng.choice([-np.inf, 0.0, 1.0], n),
            np.full(n, 7.0)]
    u = np.stack(rows).astype(np.float32)
    lens = [n, n - 1, n, 1, n // 2, 0]
    for k in [1, 64, 2048, n - 3, n + 5]:
        _check_topk_exact(u, lens, k)


def test_topk_bucket_overflow_path():
    """More than the LDS candidate capacity share the threshold bucket."""
    say("topk with a crowded threshold bucket")
    rng = np.random.default_rng(4)
    n = 100000
    u = (1.0 + rng.random(n) * 1e-3).astype(np.float32)      # one 12-bit bucket
    _check_topk_exact(u[None, :], [n], 2048)
    rows = np.stack([u, np.full(n, 2.0, np.float32)])        # many rows: single-workgroup path
    _check_topk_exact(np.repeat(rows, 40, axis=0), [n] * 80, 2048)


# --------------------------------------------------------------------- HS ---

@pytest.mark.parametrize("dtype,H,r,B", [("bf16", 64, 256, 512), ("fp32", 8, 32, 301),
                                         ("fp8", 64, 256, 512)])
def test_hs_select_matches_oracle(dtype, H, r, B):
    """B = 301: candidate lists at an odd stride (unaligned id rows)."""
    say(f"hs_select dtype={dtype} H={H} r={r} B={B}")
    wl = W.small_decode(6, n_seq=3, lens=[50, 1500, 4000], H=H, r=r, d_I=128 if H == 64 else 16,
                        G=4, k=64, B=B, cache_dtype=dtype, plant=20, factor=3.0)
    dw = DeviceWorkload(wl, hold_last=False)
    dw.hs_step(append=False, keep_scores=True)
    torch.cuda.synchronize()
    rtol = {"fp32": RTOL_FP32, "bf16": RTOL_BF16, "fp8": RTOL_FP8}[dtype]
    cand = dw.cand.cpu().numpy()
    dw.absorb(0)
    u0 = dw.score(0).cpu().numpy()
    for s in range(wl.n_q):
        L = int(wl.q_len[s])
        # anchor candidates: bit-exact on the dumped anchor scores
        ref_c = O.pad(O.hs_candidates(u0[s, :L].astype(np.float64), wl.B), wl.B)
        assert np.array_equal(cand[s], ref_c)
        assert np.array_equal(dw.hs_sel[0, s].cpu().numpy(), O.pad(O.topk(u0[s, :L].astype(np.float64), wl.k), wl.k))
        nc = min(wl.B, L)
        C = O.sequence_latent(wl, s)
        for l in range(1, wl.G):
            cs = dw.cand_scores[l, s].cpu().numpy()
            assert np.all(np.isneginf(cs[nc:]))
            o = O.layer_scores(C[cand[s, :nc]], wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            assert_scores_close(cs[:nc], o, rtol, f"follower {l} query {s}")
            sel = dw.hs_sel[l, s].cpu().numpy()
            ref = O.pad(O.hs_follower(cand[s, :nc], cs[:nc].astype(np.float64), wl.k), wl.k)
            assert np.array_equal(sel, ref)                      # bit-exact on dumped scores
            assert set(sel[sel >= 0]) <= set(cand[s, :nc])        # follower picks inside C
            full = O.layer_scores(C[:L], wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            if L <= wl.B:                                         # C = everything: HS = full
                assert_selection_band(sel, full, wl.k, rtol, f"HS=full follower {l} q {s}")
    # one follower per call gives the same bits as all followers in one call
    for l in range(1, wl.G):
        one, one_cs = ops.hs_select(dw.cand, dw.q_tilde[l], dw.w[l], dw.beta[l], dw.q_seq,
                                    dw.cache, wl.k, want_scores=True)
        assert torch.equal(one, dw.hs_sel[l]), l
        assert torch.equal(one_cs, dw.cand_scores[l]), l


# ------------------------------------------------------------ metamorphic ---

def test_determinism_permutation_and_homogeneity():
    say("metamorphic: determinism, block permutation, x4 homogeneity (bf16, H=64)")
    wl = W.small_decode(8, n_seq=1, lens=[2000], H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16", permute=True)
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb(0)
    a = dw.score(0).clone()
    b = dw.score(0).clone()
    assert torch.equal(a, b)
    wl2 = W.small_decode(8, n_seq=1, lens=[2000], H=64, r=256, d_I=128, G=1, k=16,
                         cache_dtype="bf16", permute=False)
    dw2 = DeviceWorkload(wl2, hold_last=False)
    dw2.absorb(0)
    c = dw2.score(0).clone()
    assert torch.equal(a, c)                     # physical layout does not change results
    # token 5 replaced by 4x token 3 (exact in bf16): its score is exactly 4x
    lat = wl.latent(0)
    x = torch.from_numpy(4.0 * lat[3:4]).cuda()
    ops.append_latent(x, dw.cache, torch.zeros(1, dtype=torch.int32, device="cuda"),
                      torch.full((1,), 5, dtype=torch.int32, device="cuda"))
    d = dw.score(0)
    torch.cuda.synchronize()
    assert d[0, 5].item() == 4.0 * d[0, 3].item()


def test_graph_replays_match_eager():
    """The captured HS and full-scan steps reproduce the eager results on
    every replay, with eager work and synchronisations in between."""
    say("graph capture of the HS and full-scan steps vs eager")
    wl = W.small_decode(12, n_seq=3, lens=[900, 3000, 5000], H=64, r=256, d_I=128, G=4, k=64,
                        B=512, cache_dtype="bf16", plant=20, factor=3.0)
    dw = DeviceWorkload(wl, hold_last=True)
    dw.hs_step(append=True, keep_scores=True)
    dw.full_step(append=False)
    torch.cuda.synchronize()
    ref_hs = dw.hs_sel.clone()
    ref_cs = dw.cand_scores.clone()
    ref_full = dw.sel.clone()
    g_hs = dw.capture(hs=True, keep_scores=True)
    g_full = dw.capture(hs=False, append=False)
    for rep in range(3):
        dw.hs_sel.fill_(-7)
        dw.sel.fill_(-7)
        dw.cand_scores.fill_(0.5)
        torch.cuda.synchronize()
        g_hs.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.hs_sel, ref_hs), rep
        assert torch.equal(dw.cand_scores[1:], ref_cs[1:]), rep
        _ = (dw.scores * 2).sum().item()          # eager work between replays
        g_full.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.sel, ref_full), rep


def test_hs_group_of_eight_layers():
    """A group of eight layers (seven followers share the anchor's
    candidates): every follower's candidate scores against the oracle and
    its selection exact on them; the one-call follower step equals one call
    per follower."""
    say("HS with G = 8 (seven followers)")
    wl = W.small_decode(19, n_seq=2, lens=[6000, 2500], H=64, r=256, d_I=128, G=8, k=128, B=1024,
                        cache_dtype="bf16", plant=20, factor=3.0)
    dw = DeviceWorkload(wl, hold_last=False)
    dw.hs_step(append=False, keep_scores=True)
    torch.cuda.synchronize()
    cand = dw.cand.cpu().numpy()
    sel = dw.hs_sel.cpu().numpy()
    cs_all = dw.cand_scores.cpu().numpy()
    for s in range(wl.n_q):
        L = int(wl.q_len[s])
        nc = min(wl.B, L)
        C = O.sequence_latent(wl, s)
        for l in range(1, wl.G):
            o = O.layer_scores(C[cand[s, :nc]], wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            assert_scores_close(cs_all[l, s, :nc], o, RTOL_BF16, f"G=8 follower {l} query {s}")
            ref = O.pad(O.hs_follower(cand[s, :nc], cs_all[l, s, :nc].astype(np.float64), wl.k), wl.k)
            assert np.array_equal(sel[l, s], ref), (l, s)
    for l in (1, 7):
        one = ops.hs_select(dw.cand, dw.q_tilde[l], dw.w[l], dw.beta[l], dw.q_seq, dw.cache, wl.k)
        assert torch.equal(one, dw.hs_sel[l]), l
