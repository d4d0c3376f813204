"""Host-side checks of the seeded workload generator (CPU only)."""

import numpy as np

from sparse_attention_indexer_latent_amd import workloads as W


def test_config0_shapes_and_determinism():
    a, b = W.named("tiny-4k"), W.named("tiny-4k")
    assert a.H == 8 and a.r == 32 and a.d_I == 64 and a.k == 256 and a.G == 4
    assert a.lens.tolist() == [4096] and a.cache_dtype == "fp32"
    assert a.Dt.shape == (4, 32, 64) and a.q.shape == (4, 1, 8, 64) and a.w.shape == (4, 1, 8)
    assert np.array_equal(a.latent(0), b.latent(0))
    assert np.array_equal(a.Dt, b.Dt) and np.array_equal(a.q, b.q) and np.array_equal(a.w, b.w)
    assert len(a.planted[0]) == 16
    assert np.array_equal(a.block_table[0], np.arange(64, dtype=np.int32))
    # planted rows carry the planting factor
    lat = a.latent(0)
    mask = np.zeros(4096, bool)
    mask[a.planted[0]] = True
    assert np.linalg.norm(lat[mask], axis=1).mean() > 3 * np.linalg.norm(lat[~mask], axis=1).mean()


def test_seeds_differ():
    assert not np.array_equal(W.named("tiny-4k", seed=0).latent(0), W.named("tiny-4k", seed=1).latent(0))


def test_config2_ragged_paged():
    wl = W.named("ragged-16x8k-128k-fp8")
    assert wl.n_seq == 16 and wl.cache_dtype == "fp8"
    assert wl.lens.min() >= 8192 and wl.lens.max() <= 131072
    nblk = (wl.lens + 63) // 64
    used = np.concatenate([wl.block_table[s, :nblk[s]] for s in range(16)])
    assert np.array_equal(np.sort(used), np.arange(wl.n_phys_blocks))
    assert not np.array_equal(used, np.arange(wl.n_phys_blocks))       # really permuted
    for s in range(16):
        assert np.all(wl.block_table[s, nblk[s]:] == -1)
        assert len(wl.planted[s]) == int(round(0.01 * wl.lens[s]))


def test_config3_and_prefill_shapes():
    wl = W.named("hs-128k-b4")
    assert wl.lens.tolist() == [131072] * 4 and wl.B == 8192 and wl.k == 2048
    assert wl.block_table.shape == (4, 2048)
    pf = W.named("prefill-2048x64k")
    assert pf.n_q == 2048 and pf.prefill_positions[0] == 63488 and pf.prefill_positions[-1] == 65535
    assert pf.q_len[0] == 63489 and pf.q_len[-1] == 65536
    bits, w = pf.prefill_queries(0)
    assert bits.shape == (2048, 64, 256) and bits.dtype == np.uint16 and w.shape == (2048, 64)
    assert np.array_equal(w, pf.w[0])


def test_latent_stream_independent_of_other_sequences():
    wl = W.small_decode(3, n_seq=3)
    one = W.small_decode(3, n_seq=3)
    assert np.array_equal(wl.latent(2), one.latent(2))


def test_calibration_host_solve_matches_oracle(monkeypatch):
    """The host half of the calibration (closed form from the normal
    equations) against the oracle's regression on the raw data, with the
    normal equations formed in float64 on the CPU in place of the GPU Gram."""
    import torch
    from oracle import oracle as O
    from sparse_attention_indexer_latent_amd import calibrate

    def cpu_normal_equations(X, keys, batch=1 << 16):
        Xn = X.double().numpy()
        Y = np.concatenate([k.double().numpy() for k in keys], axis=1)
        return Xn.T @ Xn, Xn.T @ Y, Xn.sum(0), Y.sum(0), Xn.shape[0]

    monkeypatch.setattr(calibrate, "normal_equations", cpu_normal_equations)
    X, WR, WN, E, off, theta = W.calibration_set(2, n=2000, d_model=40, m=3, d_R=8, d_N=12)
    R = [X.astype(np.float64) @ WR[l] + E[l][:, :8] for l in range(3)]
    N = [X.astype(np.float64) @ WN[l] + E[l][:, 8:] + off[l] for l in range(3)]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    cal = calibrate.fit_group(t(X), [t(k) for k in R], [t(k) for k in N], theta, 6, 2, 0.3)
    P_N, D_N, b_N = O.calibrate_nope(X, N, 6, 0.3)
    P_R, D_R = O.calibrate_rope(X, R, 2, 0.3)
    assert cal.r_R == 16 and cal.P.shape == (40, 22) and cal.Dt.shape == (3, 22, 20)
    for l in range(3):
        assert np.allclose(cal.P[:, 16:] @ cal.Dt[l, 16:, 8:], P_N @ D_N[l].T, atol=1e-9)
        assert np.allclose(cal.P[:, :16] @ cal.Dt[l, :16, :8], P_R @ D_R[l].T, atol=1e-9)
        assert np.allclose(cal.b[l], b_N[l], atol=1e-9)
        assert np.all(cal.Dt[l, :16, 8:] == 0) and np.all(cal.Dt[l, 16:, :8] == 0)
    assert np.allclose(cal.rope_theta, np.repeat(theta, 2))


def test_layer_correlated_queries():
    """rho = 0 leaves the independent draws unchanged; rho > 0 keeps each
    layer's marginal variance and correlates layers at about rho."""
    a = W.small_decode(5, n_seq=2, H=64, d_I=128, G=4)
    b = W.make_decode("x", 90, 5, G=4, H=64, r=32, d_I=128, k=16, B=None, cache_dtype="fp32",
                      lens=[100, 137], n_plant=0, plant_factor=4.0, permute_blocks=True)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.w, b.w)
    c = W.make_decode("x", 90, 5, G=4, H=64, r=32, d_I=128, k=16, B=None, cache_dtype="fp32",
                      lens=[100, 137], n_plant=0, plant_factor=4.0, permute_blocks=True,
                      layer_corr=0.9)
    q = c.q.reshape(4, -1).astype(np.float64)
    assert np.allclose(q.std(axis=1), 1.0, atol=0.02)
    cc = np.corrcoef(q)
    assert np.all(np.abs(cc[np.triu_indices(4, 1)] - 0.81) < 0.03)   # rho^2 between layers
    w = c.w.reshape(4, -1).astype(np.float64)
    assert np.allclose(w.std(axis=1), 1 / 8.0, rtol=0.3)   # 128 draws per layer
