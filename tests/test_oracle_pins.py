"""Pins of the CPU oracle against things other than itself (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- codecs ---

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3fn_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], got[~nan])
    # spec landmarks: max normal, min normal, min subnormal, one
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0


def _e4m3_probe_values():
    pos = O.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)          # exact ties
    ex = pos.astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    rng = np.random.default_rng(7)
    rnd = (rng.standard_normal(20000) * rng.choice([1e-3, 0.1, 1, 10, 100], 20000)).astype(np.float32)
    v = np.concatenate([ex, mids, up, dn, rnd, np.array([0.0, 447.9, 440.0, 2 ** -10, 3 * 2 ** -11], np.float32)])
    v = v[np.abs(v) < 448.0 + 1e-3]
    v = np.concatenate([v, -v]).astype(np.float32)
    return v


def test_e4m3_encode_matches_torch_including_ties():
    v = _e4m3_probe_values()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3fn_encode(v)
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 460.0, 464.0, 1000.0, 1e30, -500.0], dtype=np.float32)
    got = O.e4m3fn_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_bf16_encode_matches_torch_including_ties():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * rng.choice([1e-30, 1e-3, 1, 1e3, 1e30], 200000)).astype(np.float32)
    bits = x.view(np.uint32)
    tie_even = ((bits & 0xFFFE0000) | 0x00008000).view(np.float32)   # kept LSB 0
    tie_odd = ((bits | 0x00010000) & 0xFFFF0000 | 0x00008000).astype(np.uint32).view(np.float32)
    v = np.concatenate([x, tie_even, tie_odd, np.array([0.0, -0.0, 3.0e38], np.float32)])
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_encode(v)
    assert np.array_equal(ref, got)


def test_quantize_fp8_invariants():
    rng = np.random.default_rng(11)
    c = (rng.standard_normal((64, 256)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float32)
    c[5] = 0.0
    codes, scale = O.quantize_fp8(c)
    assert scale.dtype == np.float32 and codes.dtype == np.uint8
    assert scale[5] == 1.0 and np.all(codes[5] == 0)
    deq = O.dequantize_fp8(codes, scale)
    for i in range(64):
        if i == 5:
            continue
        j = int(np.argmax(np.abs(c[i])))
        assert codes[i, j] & 0x7F == 0x7E            # the amax element maps to 448
        mag = np.abs(O.e4m3fn_decode(codes[i] & 0x7F))
        e = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
        half_step = 2.0 ** (e - 4) * scale[i]       # half of 2^(e-3)
        assert np.all(np.abs(deq[i] - c[i]) <= half_step * (1 + 1e-6) + 1e-12)


# ---------------------------------------------------------------- scores ---

def _rand_case(rng, L=50, H=5, r=12, d_I=10, nope_off=4, per_head=False):
    C = rng.standard_normal((L, r))
    q = rng.standard_normal((H, d_I))
    Dt = rng.standard_normal((H, r, d_I) if per_head else (r, d_I)) / math.sqrt(r)
    b = rng.standard_normal(d_I - nope_off)
    w = rng.standard_normal(H)
    return C, q, Dt, b, w


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("nope_off", [0, 4, 10])
def test_absorption_identity(per_head, nope_off):
    """eq. (7): q . (D c + b) = (D^T q) . c + q^N . b, through ReLU and w."""
    rng = np.random.default_rng(nope_off + 10 * per_head)
    C, q, Dt, b, w = _rand_case(rng, nope_off=nope_off, per_head=per_head)
    u_rec = O.layer_scores(C, q, Dt, b, nope_off, w)
    qt, beta = O.absorb(q, Dt, b, nope_off)
    u_abs = O.absorbed_scores(C, qt, beta, w)
    scale = np.sqrt(np.mean(u_rec ** 2))
    assert np.max(np.abs(u_rec - u_abs)) <= 1e-5 * scale
    # the bias must matter whenever it acts on a coordinate
    if nope_off < 10:
        u_nob = O.layer_scores(C, q, Dt, np.zeros_like(b), nope_off, w)
        assert np.max(np.abs(u_nob - u_rec)) > 1e-3 * scale


def test_identity_decoder_reduces_to_relu_matvec():
    rng = np.random.default_rng(1)
    C = rng.standard_normal((40, 8))
    q = rng.standard_normal((1, 8))
    u = O.layer_scores(C, q, np.eye(8), np.zeros(0), 8, np.ones(1))
    assert np.allclose(u, np.maximum(C @ q[0], 0.0), rtol=0, atol=1e-12)


def test_all_positive_operands_reduce_to_one_gemv():
    rng = np.random.default_rng(2)
    C = rng.uniform(0, 1, (30, 6))
    q = rng.uniform(0, 1, (4, 5))
    Dt = rng.uniform(0, 1, (6, 5))
    w = rng.standard_normal(4)
    u = O.layer_scores(C, q, Dt, np.zeros(0), 5, w)
    qbar = (q * w[:, None]).sum(axis=0)            # sum_h w_h q_h
    assert np.allclose(u, C @ (Dt @ qbar), rtol=1e-12, atol=1e-12)


def test_positive_homogeneity_is_exact():
    rng = np.random.default_rng(4)
    C, q, Dt, b, w = _rand_case(rng, nope_off=10)
    u1 = O.layer_scores(C, q, Dt, b, 10, w)
    u4 = O.layer_scores(4.0 * C, q, Dt, b, 10, w)
    assert np.array_equal(u4, 4.0 * u1)


def test_relu_is_applied_per_head_before_weighting():
    # two heads with opposite pre-activations: ReLU per head keeps one term
    C = np.array([[1.0, 0.0]])
    q = np.array([[2.0, 0.0], [-3.0, 0.0]])
    u = O.layer_scores(C, q, np.eye(2), np.zeros(0), 2, np.array([1.0, 1.0]))
    assert u[0] == 2.0
    qt, beta = O.absorb(q, np.eye(2), np.array([0.5, 0.0]), 0)
    u = O.absorbed_scores(C, qt, beta, np.array([1.0, 1.0]))
    # beta_h = q_h . b enters before ReLU: head 0: 2 + 1 = 3; head 1: -3 - 1.5 < 0
    assert u[0] == 3.0


# ------------------------------------------------------------- selection ---

VALS = [-1.5, -0.0, 0.0, 0.5, 2.0, 7.25, float("-inf")]


def _brute(u, k):
    n = len(u)
    sel = []
    for t in range(n):
        rank = sum(1 for s in range(n) if u[s] > u[t] or (u[s] == u[t] and s < t))
        if rank < k:
            sel.append(t)
    return np.array(sel, dtype=np.int64)


@settings(max_examples=400, deadline=None)
@given(st.lists(st.sampled_from(VALS), min_size=0, max_size=12), st.integers(0, 14))
def test_topk_bruteforce(vals, k):
    u = np.array(vals, dtype=np.float64)
    got = O.topk(u, k)
    assert np.array_equal(got, _brute(vals, k))
    assert len(got) == min(k, len(vals))


def test_topk_custom_ids_and_padding():
    u = np.array([1.0, 3.0, 3.0, 0.0])
    ids = np.array([10, 4, 7, 12])
    assert list(O.topk(u, 2, ids)) == [4, 7]
    assert list(O.topk(u, 1, ids)) == [4]
    assert list(O.pad(O.topk(u, 9), 6)) == [0, 1, 2, 3, -1, -1]


def test_hs_invariants():
    rng = np.random.default_rng(5)
    for trial in range(30):
        L = int(rng.integers(1, 300))
        B = int(rng.integers(1, 64))
        k = int(rng.integers(1, B + 1))
        ua = np.round(rng.standard_normal(L), 1)           # rounding forces ties
        uf_full = np.round(rng.standard_normal(L), 1)
        cand = O.hs_candidates(ua, B)
        assert len(cand) == min(B, L) and np.all(np.diff(cand) > 0)
        sel_f = O.hs_follower(cand, uf_full[cand], k)
        assert set(sel_f) <= set(cand)
        assert set(O.topk(ua, k)) <= set(cand)                   # anchor top-k inside C
        assert np.array_equal(O.hs_follower(cand, ua[cand], k), O.topk(ua, k))
        big = O.hs_candidates(ua, L + B)                         # B >= L: C = everything
        assert np.array_equal(O.hs_follower(big, uf_full[big], k), O.topk(uf_full, k))


# ------------------------------------------------------------------ rope ---

def test_rope_norm_identity_and_commutation():
    rng = np.random.default_rng(6)
    n, r, rR = 9, 10, 6
    z = rng.standard_normal((n, r))
    theta = np.array([1.0, 0.1, 0.01])
    pos = rng.integers(0, 100000, n)
    zr = O.rope_rotate(z, pos, theta)
    assert np.allclose(np.linalg.norm(zr[:, :rR].reshape(n, 3, 2), axis=2),
                       np.linalg.norm(z[:, :rR].reshape(n, 3, 2), axis=2), rtol=1e-12)
    assert np.array_equal(zr[:, rR:], z[:, rR:])
    assert np.allclose(O.rope_rotate(z, np.zeros(n), theta), z, rtol=0, atol=0)
    # eq. (4): a decoder made of complex scalars per frequency commutes with
    # rotation.  Keys have 2 pairs per frequency here.
    zc = z[:, 0:rR:2] + 1j * z[:, 1:rR:2]                      # [n, 3]
    a = rng.standard_normal((2, 3)) + 1j * rng.standard_normal((2, 3))
    DR = np.zeros((12, rR))                                     # real form of k_pair = a * z_pair
    for f in range(3):
        for m in range(2):
            row = 2 * (2 * f + m)
            ar, ai = a[m, f].real, a[m, f].imag
            DR[row, 2 * f], DR[row, 2 * f + 1] = ar, -ai
            DR[row + 1, 2 * f], DR[row + 1, 2 * f + 1] = ai, ar
    keys_from_roped_latent = zr[:, :rR] @ DR.T
    kc = np.empty((n, 6), dtype=complex)            # R_t D^R z: rotate each key pair
    for f in range(3):
        for m in range(2):
            kc[:, 2 * f + m] = a[m, f] * zc[:, f] * np.exp(1j * pos * theta[f])
    ref = np.empty((n, 12))
    ref[:, 0::2], ref[:, 1::2] = kc.real, kc.imag
    assert np.allclose(keys_from_roped_latent, ref, rtol=1e-9, atol=1e-9)


# ------------------------------------------------------------ accounting ---

def test_storage_and_scoring_accounting_golden():
    g = json.load(open(os.path.join(GOLDEN, "storage_accounting.json")))
    dsa, li = O.indexer_cache_bytes_per_token(g["dsa_layers"], g["dsa_bytes_per_layer_token"],
                                              g["group"], g["latent_bytes"], g["native_layers"])
    assert dsa == g["expect_dsa_bytes_per_token"] and li == g["expect_li_bytes_per_token"]
    assert round(100 * (1 - li / dsa), 1) == g["expect_reduction_percent_1dp"]
    T = g["context_tokens"]
    assert round(dsa * T / 1e9, 2) == g["expect_dsa_gb_2dp"]
    assert round(li * T / 1e9, 2) == g["expect_li_gb_2dp"]
    Bud = g["hs_budget"]
    hs = O.scored_positions(T, 4, Bud)
    full = O.scored_positions(T, 4)
    assert (hs - T) // 3 == g["expect_follower_scored"] and full // 4 == g["expect_full_scored"]
    assert full // 4 // ((hs - T) // 3) == g["expect_follower_ratio"]
    # at L = B the HS count equals the full scan count (no positions saved)
    assert O.scored_positions(8192, 4, 8192) == O.scored_positions(8192, 4)
