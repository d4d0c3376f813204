"""Host-side checks of the seeded workload generator (CPU only)."""

import numpy as np

from sparse_attention_indexer_latent_amd import workloads as W


def test_config0_shapes_and_determinism():
    a, b = W.config(0), W.config(0)
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
    assert not np.array_equal(W.config(0, seed=0).latent(0), W.config(0, seed=1).latent(0))


def test_config2_ragged_paged():
    wl = W.config(2)
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
    wl = W.config(3)
    assert wl.lens.tolist() == [131072] * 4 and wl.B == 8192 and wl.k == 2048
    assert wl.block_table.shape == (4, 2048)
    pf = W.config(4)
    assert pf.n_q == 2048 and pf.prefill_positions[0] == 63488 and pf.prefill_positions[-1] == 65535
    assert pf.q_len[0] == 63489 and pf.q_len[-1] == 65536
    bits, w = pf.prefill_queries(0)
    assert bits.shape == (2048, 64, 256) and bits.dtype == np.uint16 and w.shape == (2048, 64)
    assert np.array_equal(w, pf.w[0])


def test_latent_stream_independent_of_other_sequences():
    wl = W.small_decode(3, n_seq=3)
    one = W.small_decode(3, n_seq=3)
    assert np.array_equal(wl.latent(2), one.latent(2))
