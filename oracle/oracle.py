"""CPU oracle for the LatentIndex decode indexer.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
imports nothing from the HIP library or its Python binding.

Everything here is plain NumPy in float64 on exactly the operand values the
cache stores (fp32 as is, bf16 and fp8 codes decoded exactly).  The scorer
reconstructs every layer's keys explicitly and never uses decoder absorption:
the absorbed form appears only as the other side of the identity that pins it.

Sources (the pages this follows; sections, equations and tables named):
  [P1] "LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for
       Sparse Attention", picx.dev summary: Methodology (eqs. 1-4, 6-8, the
       TopK definition, Hierarchical Selection), Theoretical and Practical
       Implications (Storage Efficiency).
  [P4] "LatentIndex - Shared indexer cache, per-layer token choice",
       learnaivisually explainer: the decoder-absorption paragraph and the
       storage/compute accounting paragraph.
  [OCP] OCP 8-bit Floating Point Specification (E4M3 with the FN encoding:
       no infinities, one NaN mantissa, max 448) -- named by the cache layout,
       not by the pages.

Pins (tests/test_oracle_pins.py; none re-types the formula it checks):
  e4m3 decode/encode  torch.float8_e4m3fn over all 256 codes and all ties
  bf16_encode         torch.bfloat16 cast, including every tie case
  bf16_decode         torch.bfloat16 -> float64 over all 65,536 bit patterns
  quantize_fp8        invariants: amax code is +-448, |error| <= half step
  reconstructed score eq. 7 identity vs the absorbed score (1e-5 rel, fp64);
                      D = I, H = 1 reduces to max(C q, 0) (library matmul);
                      all-positive operands reduce to one GEMV;
                      exact positive homogeneity u(4c) = 4 u(c)
  topk                brute-force rank definition on tiny inputs with ties
  hs_candidates/      subset / equality invariants of the HS definition
    hs_follower
  rope_rotate         norm preservation, identity at t = 0, and eq. 4
                      commutation with a complex-block decoder
  project_latent      a per-column dot-product loop (no rotation); P = I
                      equals rope_rotate; a rotation built with Python
                      complex numbers fixes the R-branch-first column order
                      and projection-then-rotation (eqs. 1-2)
  decode_group        every score against plain-Python sums and every
                      selection against the brute-force rank; B >= L gives
                      HS = full for every follower; a follower with the
                      anchor's operands returns S_anchor; HS picks stay in C
  accounting          the numbers printed in [P4] and [P1] (tests/golden)
  ridge_rrr           full rank and lam = 0 is numpy's least squares; lam > 0
                      is least squares on the augmented system [X; sqrt(lam)
                      I]; rank r at lam = 0 is the Eckart-Young truncation of
                      the least-squares fit (numpy SVD of X B_ls)
  calibrate_nope      recovers an exact shared-rank group model (projection,
                      decoders and biases up to the latent basis) from noise-
                      free keys
  calibrate_rope      the fitted decoder commutes with the rotation (eq. 4)
                      and recovers keys made by an exact complex-per-frequency
                      model
Parity unpinned: none of the functions above.  The planted-token structure of
the synthetic workloads is not pinned by the pages (they print no scores).
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

F64 = np.float64

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------


def e4m3fn_value(code: int) -> float:
    """Exact value of one OCP E4M3FN byte (sign 1, exponent 4, mantissa 3,
    bias 7; exponent field 0 is subnormal; 0x7F/0xFF are NaN; no inf)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=F64)
E4M3_MAX = 448.0
# The 127 non-negative finite codes 0x00..0x7E in ascending value order.
_POS_VALUES = E4M3_TABLE[:0x7F].copy()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest E4M3FN value, ties to the even code
    (mantissa LSB 0), saturating to +-448.  The sign bit follows the input."""
    x = np.asarray(x32, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3fn_encode: non-finite input")
    a = np.abs(x).astype(F64)
    sat = a >= E4M3_MAX
    # index of the largest code value <= a (codes are value-ordered)
    i = np.searchsorted(_POS_VALUES, np.where(sat, 0.0, a), side="right") - 1
    i = np.minimum(i, 0x7D)
    lo = _POS_VALUES[i]
    hi = _POS_VALUES[i + 1]
    dlo = a - lo
    dhi = hi - a
    up = (dhi < dlo) | ((dhi == dlo) & ((i & 1) == 1))
    code = np.where(up, i + 1, i)
    code = np.where(sat, 0x7E, code).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the upper half of an fp32 pattern."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(F64)


def bf16_encode(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (8 significant bits), nearest, ties to even.

    The two bf16 neighbours of x are the value with the low 16 bits cleared
    (toward zero) and the next one away from zero; pick the nearer in exact
    float64 arithmetic, on a tie the one whose last kept bit is 0."""
    x = np.asarray(x32, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_encode: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    lo_bits = u & 0xFFFF0000
    hi_bits = lo_bits + 0x10000
    xv = x.astype(F64)
    lo = lo_bits.astype(np.uint32).view(np.float32).astype(F64)
    with np.errstate(over="ignore", invalid="ignore"):
        hi = hi_bits.astype(np.uint32).view(np.float32).astype(F64)
    dlo = np.abs(xv - lo)
    dhi = np.abs(hi - xv)
    even_lo = ((lo_bits >> 16) & 1) == 0
    take_hi = (dhi < dlo) | ((dhi == dlo) & ~even_lo)
    take_hi &= (u & 0xFFFF) != 0
    res = np.where(take_hi, hi_bits, lo_bits) >> 16
    return res.astype(np.uint16)


# ---------------------------------------------------------------------------
# Latent construction and storage ([P1] Methodology, eqs. 1-2; storage
# format per token: bf16, or fp8 E4M3FN codes with one fp32 scale)
# ---------------------------------------------------------------------------


def rope_rotate(z: np.ndarray, pos: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """Apply the rotary map Q_t of eq. (1) to the leading 2*len(theta)
    coordinates of each row: pair (2j, 2j+1) is read as the complex number
    z_{2j} + i z_{2j+1} and multiplied by exp(i * t * theta_j).  Float64."""
    z = np.array(z, dtype=F64, copy=True)
    pos = np.asarray(pos, dtype=F64).reshape(-1, 1)
    th = np.asarray(theta, dtype=F64).reshape(1, -1)
    ang = pos * th
    c, s = np.cos(ang), np.sin(ang)
    x0 = z[:, 0:2 * th.shape[1]:2].copy()
    x1 = z[:, 1:2 * th.shape[1]:2].copy()
    z[:, 0:2 * th.shape[1]:2] = c * x0 - s * x1
    z[:, 1:2 * th.shape[1]:2] = s * x0 + c * x1
    return z


def project_latent(x: np.ndarray, P: Optional[np.ndarray], theta: Optional[np.ndarray],
                   pos: np.ndarray) -> np.ndarray:
    """c_t = [Q_t P_R^T x_t ; P_N^T x_t] (eqs. 1-2), float64.  P holds the
    R-branch columns first, then the N-branch ([d_model, r]); P = None means
    x already is the latent.  theta = None (or empty) means r_R = 0."""
    z = np.asarray(x, dtype=F64)
    if P is not None:
        z = z @ np.asarray(P, dtype=F64)
    if theta is not None and len(theta):
        z = rope_rotate(z, pos, theta)
    return z


def quantize_fp8(c32: np.ndarray, block: int = 0):
    """fp8 storage of fp32 latent rows [n, r], one scale per row (block = 0)
    or per `block` consecutive values of a row: amax = max|c| over the row
    or block (fp32), scale = amax/448 and inv = 448/amax as IEEE fp32
    divisions (scale = inv = 1 when amax = 0), codes = E4M3FN-RNE(fp32(c *
    inv)).  Returns (codes uint8 [n, r], scale float32 [n] for block = 0,
    else [n, ceil(r / block)])."""
    c = np.asarray(c32, dtype=np.float32)
    n, r = c.shape
    blk = block or r
    nb = -(-r // blk)
    codes = np.empty((n, r), dtype=np.uint8)
    scales = np.empty((n, nb), dtype=np.float32)
    for g in range(nb):
        part = c[:, g * blk:(g + 1) * blk]
        amax = np.max(np.abs(part), axis=1).astype(np.float32)
        zero = amax == 0
        safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
        scales[:, g] = np.where(zero, np.float32(1.0), safe / np.float32(448.0))
        inv = np.where(zero, np.float32(1.0), np.float32(448.0) / safe).astype(np.float32)
        codes[:, g * blk:(g + 1) * blk] = e4m3fn_encode((part * inv[:, None]).astype(np.float32))
    return codes, (scales[:, 0].copy() if block == 0 else scales)


def dequantize_fp8(codes: np.ndarray, scale: np.ndarray, block: int = 0) -> np.ndarray:
    """Exact value of fp8 codes [n, r] with their scales (per row, or per
    `block` values of a row)."""
    vals = e4m3fn_decode(codes)
    sc = np.asarray(scale, dtype=F64)
    if block == 0:
        return vals * sc[:, None]
    return vals * np.repeat(sc, block, axis=1)[:, :vals.shape[1]]


def store_latent(c32: np.ndarray, dtype: str, scale_block: int = 0):
    """What the cache stores for fp32 rows c32, and its exact float64 value.
    Returns (stored, scale_or_None, exact_f64)."""
    c32 = np.asarray(c32, dtype=np.float32)
    if dtype == "fp32":
        return c32.copy(), None, c32.astype(F64)
    if dtype == "bf16":
        bits = bf16_encode(c32)
        return bits, None, bf16_decode(bits)
    if dtype == "fp8":
        codes, scale = quantize_fp8(c32, scale_block)
        return codes, scale, dequantize_fp8(codes, scale, scale_block)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Keys, scores ([P1] Methodology, eqs. 3, 6-8)
# ---------------------------------------------------------------------------


def reconstruct_keys(C: np.ndarray, Dt: np.ndarray, b: np.ndarray, nope_off: int) -> np.ndarray:
    """k_t = D c_t, plus b on the NoPE key coordinates [nope_off, d_I) (eq. 3).
    C: [L, r] float64, Dt: D transposed, [r, d_I].  Returns [L, d_I]."""
    K = np.asarray(C, dtype=F64) @ np.asarray(Dt, dtype=F64)
    if K.shape[1] > nope_off:
        K[:, nope_off:] += np.asarray(b, dtype=F64)[None, :]
    return K


def layer_scores(C: np.ndarray, q: np.ndarray, Dt: np.ndarray, b: np.ndarray,
                 nope_off: int, w: np.ndarray) -> np.ndarray:
    """u_t = sum_h w_h ReLU(q_h . k_t) over explicitly reconstructed keys
    (the left side of eq. 7 substituted into eq. 8).  q: [H, d_I]; Dt: [r, d_I]
    shared by heads or [H, r, d_I] per head; w: [H].  Returns [L] float64."""
    q = np.asarray(q, dtype=F64)
    w = np.asarray(w, dtype=F64)
    Dt = np.asarray(Dt)
    if Dt.ndim == 2:
        K = reconstruct_keys(C, Dt, b, nope_off)
        X = K @ q.T                                   # [L, H]
    else:
        X = np.empty((np.asarray(C).shape[0], q.shape[0]), dtype=F64)
        for h in range(q.shape[0]):
            X[:, h] = reconstruct_keys(C, Dt[h], b, nope_off) @ q[h]
    return np.maximum(X, 0.0) @ w


def absorb(q: np.ndarray, Dt: np.ndarray, b: np.ndarray, nope_off: int):
    """q~_h = D^T q_h and beta_h = q_h^N . b (eq. 6).  Returns ([H, r], [H])."""
    q = np.asarray(q, dtype=F64)
    Dt = np.asarray(Dt, dtype=F64)
    if Dt.ndim == 2:
        qt = q @ Dt.T
    else:
        qt = np.einsum("hrd,hd->hr", Dt, q)
    beta = q[:, nope_off:] @ np.asarray(b, dtype=F64) if q.shape[1] > nope_off \
        else np.zeros(q.shape[0], dtype=F64)
    return qt, beta


def absorbed_scores(C: np.ndarray, qt: np.ndarray, beta: Optional[np.ndarray],
                    w: np.ndarray) -> np.ndarray:
    """u_t = sum_h w_h ReLU(q~_h . c_t + beta_h) (eq. 8) for given absorbed
    queries.  Used as the right side of eq. 7 and for the prefill chunk,
    whose stored input already is the absorbed query."""
    X = np.asarray(C, dtype=F64) @ np.asarray(qt, dtype=F64).T
    if beta is not None:
        X = X + np.asarray(beta, dtype=F64)[None, :]
    return np.maximum(X, 0.0) @ np.asarray(w, dtype=F64)


# ---------------------------------------------------------------------------
# Selection ([P1] Methodology: TopK over V_s with min(k, |V_s|); Hierarchical
# Selection).  Order: larger score first, then lower token index.
# ---------------------------------------------------------------------------


def topk(u: np.ndarray, k: int, ids: Optional[np.ndarray] = None) -> np.ndarray:
    """The first min(k, n) entries of u under (score desc, id asc), returned
    as ascending ids.  ids defaults to 0..n-1.  -0.0 and +0.0 tie."""
    u = np.asarray(u, dtype=F64)
    n = u.shape[0]
    if ids is None:
        ids = np.arange(n, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -u))
    return np.sort(ids[order[:min(k, n)]])


def pad(sel: np.ndarray, k: int) -> np.ndarray:
    out = np.full(k, -1, dtype=np.int32)
    out[:len(sel)] = sel
    return out


def hs_candidates(u_anchor: np.ndarray, B: int) -> np.ndarray:
    """C = the anchor's top-min(B, L) positions (ascending ids)."""
    return topk(u_anchor, B)


def hs_follower(cand: np.ndarray, u_f_cand: np.ndarray, k: int) -> np.ndarray:
    """The follower's top-min(k, |C|) within C, from its scores on C."""
    return topk(u_f_cand, k, ids=cand)


# ---------------------------------------------------------------------------
# Whole group steps on a workload (used by tests and the CPU baseline)
# ---------------------------------------------------------------------------


def sequence_latent(wl, s: int) -> np.ndarray:
    """Exact float64 latent of sequence s as the configured cache stores it."""
    return store_latent(wl.latent(s), wl.cache_dtype, getattr(wl, "scale_block", 0))[2]


def decode_group(wl, s: int, C: Optional[np.ndarray] = None, layers=None,
                 hs: bool = False, rows: Optional[np.ndarray] = None):
    """One decode step of the layer group for query s (sequence wl.q_seq[s]).

    Returns a dict with per-layer score rows 'u' (full scan, [L]) and
    selections 'sel' (ascending ids); with hs=True also 'cand', 'u_f'
    (follower scores on the candidates) and 'hs_sel'; with hs=True and
    layers=[0] only the anchor scans the whole cache, as the HS step does.
    rows restricts the scored tokens to a sample (no selection then)."""
    seq = int(wl.q_seq[s])
    L = int(wl.q_len[s])
    if C is None:
        C = sequence_latent(wl, seq)
    C = C[:L]
    layers = range(wl.G) if layers is None else layers
    out = {"u": {}, "sel": {}}
    for l in layers:
        Cs = C if rows is None else C[rows]
        u = layer_scores(Cs, wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
        out["u"][l] = u
        if rows is None:
            out["sel"][l] = topk(u, wl.k)
    if hs and rows is None:
        cand = hs_candidates(out["u"][0], wl.B)
        out["cand"] = cand
        out["u_f"], out["hs_sel"] = {}, {0: topk(out["u"][0], wl.k)}
        for l in range(1, wl.G):
            uf = layer_scores(C[cand], wl.q[l, s], wl.Dt[l], wl.b[l], wl.nope_off, wl.w[l, s])
            out["u_f"][l] = uf
            out["hs_sel"][l] = hs_follower(cand, uf, wl.k)
    return out


# ---------------------------------------------------------------------------
# Training-free calibration ([P1] Methodology, Training-free Calibration:
# ridge reduced-rank regression jointly fits the group's shared projection and
# every layer's decoder from calibration hidden states and the layers' own
# indexer keys, minimising key-reconstruction error at a given latent rank;
# the NoPE and RoPE branches are fitted separately, each in closed form).
# ---------------------------------------------------------------------------


def ridge_rrr(X: np.ndarray, Y: np.ndarray, rank: int, lam: float):
    """min_B ||Y - X B||_F^2 + lam ||B||_F^2 subject to rank(B) <= rank, the
    reduced-rank ridge regression of Mukherjee and Zhu ("Reduced rank ridge
    regression and its kernel extensions", 2011): B_lam = (X^T X + lam I)^-1
    X^T Y is the ridge fit; the rank constraint keeps the top `rank` right
    singular vectors V of the augmented fit [X B_lam; sqrt(lam) B_lam], and
    B = B_lam V V^*.  Works for real or complex Y (X real).  Returns
    (P = B_lam V [d, rank], D = conj(V) [e, rank]) with B = P D^T."""
    X = np.asarray(X, dtype=F64)
    Y = np.asarray(Y)
    Y = Y.astype(np.complex128 if np.iscomplexobj(Y) else F64)
    d = X.shape[1]
    B_lam = np.linalg.solve(X.T @ X + lam * np.eye(d), X.T @ Y)
    aug = np.concatenate([X @ B_lam, np.sqrt(lam) * B_lam], axis=0)
    V = np.linalg.svd(aug, full_matrices=False)[2].conj().T[:, :rank]    # [e, rank]
    return B_lam @ V, V.conj()


def calibrate_nope(X: np.ndarray, keys: list, rank: int, lam: float):
    """NoPE branch: one projection P_N [d_model, r_N] shared by the group and
    each layer's decoder D^(l),N [d_N, r_N] and bias b^(l) (eq. 3) from
    hidden states X [n, d_model] and the layers' NoPE keys keys[l] [n, d_N].
    The bias takes the means (the fit runs on centred data).  Returns
    (P_N, [D^(l),N], [b^(l)])."""
    X = np.asarray(X, dtype=F64)
    Ys = [np.asarray(k, dtype=F64) for k in keys]
    xm = X.mean(axis=0)
    Y = np.concatenate(Ys, axis=1)
    ym = Y.mean(axis=0)
    P, D = ridge_rrr(X - xm, Y - ym, rank, lam)
    b = ym - D @ (P.T @ xm)
    dn = Ys[0].shape[1]
    return P, [D[l * dn:(l + 1) * dn] for l in range(len(Ys))], \
        [b[l * dn:(l + 1) * dn] for l in range(len(Ys))]


def calibrate_rope(X: np.ndarray, keys: list, pairs_per_freq: int, lam: float):
    """RoPE branch (eqs. 1, 3-4): keys[l] [n, d_R] are layer l's rotary
    key coordinates before rotation, pair (2j, 2j+1) at frequency j.  The
    decoder may only mix pairs of one frequency, as complex scalars (then it
    commutes with the rotation, eq. 4), so each frequency is its own complex
    ridge reduced-rank regression of the layers' pairs [n, m] on X, at rank
    pairs_per_freq.  Returns (P_R [d_model, r_R] with latent pair (2q, 2q+1) =
    (Re, Im) of the q-th complex latent, q = j * pairs_per_freq + i, and
    [D^(l),R [d_R, r_R]] in real form)."""
    X = np.asarray(X, dtype=F64)
    Ks = [np.asarray(k, dtype=F64) for k in keys]
    m, n_freq = len(Ks), Ks[0].shape[1] // 2
    a = pairs_per_freq
    P_R = np.zeros((X.shape[1], 2 * n_freq * a))
    D_R = [np.zeros((2 * n_freq, 2 * n_freq * a)) for _ in range(m)]
    for j in range(n_freq):
        Yf = np.stack([K[:, 2 * j] + 1j * K[:, 2 * j + 1] for K in Ks], axis=1)   # [n, m]
        P, D = ridge_rrr(X, Yf, a, lam)          # zeta = X P [n, a]; pair_l = zeta D[l]^T
        for i in range(a):
            q = j * a + i
            P_R[:, 2 * q], P_R[:, 2 * q + 1] = P[:, i].real, P[:, i].imag
            for l in range(m):
                c = D[l, i]                        # complex scalar: pair_j += c * zeta_q
                D_R[l][2 * j, 2 * q], D_R[l][2 * j, 2 * q + 1] = c.real, -c.imag
                D_R[l][2 * j + 1, 2 * q], D_R[l][2 * j + 1, 2 * q + 1] = c.imag, c.real
    return P_R, D_R


# ---------------------------------------------------------------------------
# Accounting ([P4] storage/compute paragraph; [P1] Hierarchical Selection)
# ---------------------------------------------------------------------------


def scored_positions(L: int, m: int, B: Optional[int] = None) -> int:
    """Positions scored per query by a group of m layers: m*L for full scan,
    L + (m - 1) * min(B, L) under hierarchical selection."""
    return m * L if B is None else L + (m - 1) * min(B, L)


def indexer_cache_bytes_per_token(n_layers: int, dsa_bytes: int, group: int,
                                  latent_bytes: int, native_layers: int):
    """(native DSA bytes, LatentIndex bytes) per token: every layer keeps its
    own key in DSA; LatentIndex keeps the native layers' keys plus one latent
    per group of the rest."""
    dsa = n_layers * dsa_bytes
    shared = n_layers - native_layers
    assert shared % group == 0
    li = native_layers * dsa_bytes + (shared // group) * latent_bytes
    return dsa, li
