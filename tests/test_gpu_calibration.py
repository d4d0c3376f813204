"""GPU parity of the training-free calibration (LatentIndex summary,
"Methodology", Training-free Calibration): the normal equations on the
matrix cores against float64, the whole fit (GPU normal equations + closed
form) against the oracle's float64 ridge reduced-rank regression, and a
calibrated group run through the library end to end (projection and rotary
map at append, absorption, scoring) against the oracle."""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_indexer_latent_amd import calibrate, ops
from sparse_attention_indexer_latent_amd import workloads as W

from parity_util import RTOL_FP32, assert_scores_close, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(1000, 533, 70, 33), (777, 300, 256, 192)],
                         ids=["ragged", "vector-rows"])
@pytest.mark.parametrize("bf16", [False, True])
def test_calib_gram_against_float64(bf16, shape):
    """Two batches accumulated against the float64 products of the same
    values: ragged sizes (not multiples of the 128 x 128 blocks, the 16-row
    slabs or a 16-byte row), and rows that take the vector loads with partial
    slabs and several blocks on and off the diagonal; fp32 sums of exact
    products: relative error ~ n 2^-24."""
    n1, n2, d, e = shape
    say(f"calib gram bf16={bf16} n={n1}+{n2} d={d} e={e}")
    rng = np.random.default_rng(50)
    X = rng.standard_normal((n1 + n2, d)).astype(np.float32) * 3
    Y = rng.standard_normal((n1 + n2, e)).astype(np.float32)
    dt = torch.bfloat16 if bf16 else torch.float32
    Xd, Yd = torch.from_numpy(X).cuda().to(dt), torch.from_numpy(Y).cuda().to(dt)
    G, H, xs, ys = ops.calib_gram(Xd[:n1].contiguous(), Yd[:n1].contiguous())
    ops.calib_gram(Xd[n1:].contiguous(), Yd[n1:].contiguous(), G, H, xs, ys, accumulate=True)
    Xe, Ye = Xd.double().cpu().numpy(), Yd.double().cpu().numpy()
    for got, ref, nm in ((G, Xe.T @ Xe, "XtX"), (H, Xe.T @ Ye, "XtY"), (xs, Xe.sum(0), "x_sum"),
                         (ys, Ye.sum(0), "y_sum")):
        g = got.double().cpu().numpy()
        scale = np.abs(ref).max()
        err = np.abs(g - ref).max() / scale
        say(f"  {nm}: max err {err:.2e} of the largest entry")
        assert err < 1e-5, nm


def _keys(X, WR, WN, E, off):
    """The layers' native keys: rotary part before rotation, NoPE part."""
    m, d_R = WR.shape[0], WR.shape[2]
    R = [X.astype(np.float64) @ WR[l] + E[l][:, :d_R] for l in range(m)]
    N = [X.astype(np.float64) @ WN[l] + E[l][:, d_R:] + off[l] for l in range(m)]
    return R, N


def test_fit_group_matches_oracle_calibration():
    """GPU normal equations + closed form against the oracle's float64
    regression from the raw data: the fitted maps P D^T of every layer and
    branch and the NoPE biases (the factors themselves are unique only up to
    a basis of the latent)."""
    say("calibration fit vs oracle")
    X, WR, WN, E, off, theta = W.calibration_set(0, n=4096, d_model=96, m=4, d_R=16, d_N=32)
    R, N = _keys(X, WR, WN, E, off)
    r_N, a, lam = 12, 1, 0.5
    dev = lambda a_: torch.from_numpy(np.ascontiguousarray(a_, dtype=np.float32)).cuda()  # noqa: E731
    cal = calibrate.fit_group(dev(X), [dev(k) for k in R], [dev(k) for k in N], theta, r_N, a, lam)
    P_N, D_N, b_N = O.calibrate_nope(X, N, r_N, lam)
    P_R, D_R = O.calibrate_rope(X, R, a, lam)
    m, d_R = 4, 16
    for l in range(m):
        ref_N = P_N @ D_N[l].T
        got_N = cal.P[:, cal.r_R:] @ cal.Dt[l, cal.r_R:, d_R:]
        eN = np.abs(got_N - ref_N).max() / np.abs(ref_N).max()
        ref_R = P_R @ D_R[l].T
        got_R = cal.P[:, :cal.r_R] @ cal.Dt[l, :cal.r_R, :d_R]
        eR = np.abs(got_R - ref_R).max() / np.abs(ref_R).max()
        eb = np.abs(cal.b[l] - b_N[l]).max() / np.abs(b_N[l]).max()
        say(f"  layer {l}: NoPE map err {eN:.2e}, RoPE map err {eR:.2e}, bias err {eb:.2e}")
        assert eN < 1e-3 and eR < 1e-3 and eb < 1e-3, l
    assert np.allclose(cal.rope_theta, theta)


def test_calibrated_group_scores_through_the_library():
    """The calibrated projection, rotary frequencies, decoders and biases
    drive li_append_latent (projection + rotation at append, fp32 cache),
    li_absorb_queries and li_score for new tokens; every score matches the
    oracle's reconstructed-key scores of the same calibrated model."""
    say("calibrated group end to end")
    X, WR, WN, E, off, theta = W.calibration_set(1, n=4096, d_model=96, m=4, d_R=16, d_N=32)
    R, N = _keys(X, WR, WN, E, off)
    dev = lambda a_: torch.from_numpy(np.ascontiguousarray(a_, dtype=np.float32)).cuda()  # noqa: E731
    cal = calibrate.fit_group(dev(X), [dev(k) for k in R], [dev(k) for k in N], theta, 16, 1, 0.5)
    r = cal.P.shape[1]
    assert r == 32 and cal.r_R == 16
    rng = np.random.default_rng(51)
    L, H = 450, 8
    x = (rng.standard_normal((L, 96)) * 1.5).astype(np.float32)
    pos = np.arange(L, dtype=np.int32)
    bt = torch.arange(16, dtype=torch.int32, device="cuda").reshape(1, 16)
    cache = ops.Cache.empty(16, r, "fp32", bt)
    ops.append_latent(dev(x), cache, torch.zeros(L, dtype=torch.int32, device="cuda"),
                      torch.from_numpy(pos).cuda(), P=dev(cal.P), rope_theta=dev(cal.rope_theta))
    C = O.project_latent(x, cal.P.astype(np.float32), cal.rope_theta.astype(np.float32), pos)
    q = rng.standard_normal((4, 1, H, 48)).astype(np.float32)
    w = (rng.standard_normal((4, 1, H)) / np.sqrt(H)).astype(np.float32)
    Dt32 = cal.Dt.astype(np.float32)
    b32 = cal.b.astype(np.float32)
    qt, beta = ops.absorb_queries(dev(q), dev(Dt32), dev(b32), cal.nope_off)
    for l in range(4):
        u = ops.score(qt[l], dev(w[l]), beta[l], torch.zeros(1, dtype=torch.int32, device="cuda"),
                      torch.full((1,), L, dtype=torch.int32, device="cuda"), L, cache)
        o = O.layer_scores(C, q[l, 0], Dt32[l], b32[l], cal.nope_off, w[l, 0])
        assert_scores_close(u[0, :L].cpu().numpy(), o, RTOL_FP32, f"calibrated layer {l}")


def test_calib_gram_sums_without_cross_products():
    """Through the C ABI: y_sum requested with G_xy NULL, and n = 0 (zeros
    written), against float64."""
    say("calib gram: y_sum without G_xy, n = 0")
    rng = np.random.default_rng(52)
    X = torch.from_numpy(rng.standard_normal((300, 40)).astype(np.float32)).cuda()
    Y = torch.from_numpy(rng.standard_normal((300, 130)).astype(np.float32)).cuda()
    G = torch.full((40, 40), 7.0, device="cuda")
    xs = torch.full((40,), 7.0, device="cuda")
    ys = torch.full((130,), 7.0, device="cuda")
    lib = ops.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert lib.li_calib_gram(X.data_ptr(), ops.LI_FP32, 300, 40, Y.data_ptr(), ops.LI_FP32, 130,
                             G.data_ptr(), None, xs.data_ptr(), ys.data_ptr(), 0, st) == ops.LI_OK
    torch.cuda.synchronize()
    Xe, Ye = X.double().cpu().numpy(), Y.double().cpu().numpy()
    assert np.allclose(ys.double().cpu().numpy(), Ye.sum(0), rtol=1e-5, atol=1e-4)
    assert np.allclose(xs.double().cpu().numpy(), Xe.sum(0), rtol=1e-5, atol=1e-4)
    assert np.allclose(G.double().cpu().numpy(), Xe.T @ Xe, rtol=1e-5, atol=1e-3)
    assert lib.li_calib_gram(X.data_ptr(), ops.LI_FP32, 0, 40, Y.data_ptr(), ops.LI_FP32, 130,
                             G.data_ptr(), None, xs.data_ptr(), ys.data_ptr(), 0, st) == ops.LI_OK
    torch.cuda.synchronize()
    assert torch.all(G == 0) and torch.all(xs == 0) and torch.all(ys == 0)
