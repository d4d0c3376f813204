"""Training-free calibration of one layer group (LatentIndex summary,
"Methodology", Training-free Calibration; eqs. 1-4).

The group's shared projection P = [P_R | P_N] and every layer's decoder
D^(l) = blockdiag(D^(l),R, D^(l),N) and NoPE bias b^(l) are fitted offline
to the layers' own indexer keys by ridge reduced-rank regression, the NoPE
and RoPE branches separately, each in closed form:

  * the O(n d^2) normal equations over the calibration tokens (X^T X, X^T Y,
    column sums) run on the GPU matrix cores (li_calib_gram);
  * the closed-form solves on those small matrices run in float64 on the
    host: (G + lam I) B = H by Cholesky (one factor per branch, shared by
    every rotary frequency), then the rank constraint keeps the
    top eigenvectors V of B^* H (= the augmented fit's Gram [X B;
    sqrt(lam) B]^* [X B; sqrt(lam) B]), P = B V and D = conj(V) (Mukherjee
    and Zhu, "Reduced rank ridge regression", 2011).

NoPE: one real regression of the stacked NoPE keys of all layers on the
centred hidden states (the bias takes the means).  RoPE (eq. 4): keys are
taken before their rotation; a decoder that commutes with the rotation
mixes only pairs of one frequency, as complex scalars, so every frequency
is its own complex regression of the layers' pairs, and its latent pairs
rotate at that frequency.

The result is in the library's operand formats: P [d_model, r] for
li_append_latent (R columns first), Dt [r, d_I] per layer (key coordinates
R first, then NoPE from nope_off = d_R) and b [d_N] per layer for
li_absorb_queries, and the latent's rotary frequencies for li_append_latent.
"""

from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np
import torch
from scipy.linalg import cho_factor, cho_solve

from . import ops


@dataclasses.dataclass
class GroupCalibration:
    P: np.ndarray            # [d_model, r] float64, columns [P_R | P_N]
    Dt: np.ndarray           # [m, r, d_I] float64, D^(l) transposed
    b: np.ndarray            # [m, d_N] float64 NoPE biases
    rope_theta: np.ndarray   # [r_R / 2] rotary frequency of each latent pair
    r_R: int
    nope_off: int            # key coordinates [nope_off, d_I) are NoPE


def _top_eigvecs(M: np.ndarray, k: int) -> np.ndarray:
    M = 0.5 * (M + M.conj().T)
    w, V = np.linalg.eigh(M)
    return V[:, np.argsort(w)[::-1][:k]]


def _ridge_rank_solve(cf, H: np.ndarray, rank: int):
    """(P, D) with P D^T the rank-`rank` ridge fit from the Cholesky factor
    cf of G + lam I (G = X^T X) and H = X^T Y (Y real or complex)."""
    if np.iscomplexobj(H):
        B = cho_solve(cf, H.real) + 1j * cho_solve(cf, H.imag)
    else:
        B = cho_solve(cf, H)
    V = _top_eigvecs(B.conj().T @ H, rank)
    return B @ V, V.conj()


def normal_equations(X: torch.Tensor, keys: Sequence[torch.Tensor], batch: int = 1 << 16):
    """Accumulate X^T X, X^T Y and the column sums on the GPU over batches of
    rows (Y = the key blocks side by side).  Returns float64 host arrays."""
    n, d = X.shape
    # the keys keep their precision: bf16 only when every block is bf16
    ydt = torch.bfloat16 if all(k.dtype == torch.bfloat16 for k in keys) else torch.float32
    Y = torch.cat([k.to(ydt) for k in keys], dim=1).contiguous()
    e = Y.shape[1]
    dev = X.device
    G = torch.zeros((d, d), dtype=torch.float32, device=dev)
    H = torch.zeros((d, e), dtype=torch.float32, device=dev)
    xs = torch.zeros(d, dtype=torch.float32, device=dev)
    ys = torch.zeros(e, dtype=torch.float32, device=dev)
    for a in range(0, n, batch):
        ops.calib_gram(X[a:a + batch].contiguous(), Y[a:a + batch].contiguous(), G, H, xs, ys,
                       accumulate=a > 0)
    torch.cuda.synchronize()
    return (G.double().cpu().numpy(), H.double().cpu().numpy(), xs.double().cpu().numpy(),
            ys.double().cpu().numpy(), n)


def fit_group(X: torch.Tensor, rope_keys: Sequence[torch.Tensor], nope_keys: Sequence[torch.Tensor],
              key_theta: np.ndarray, r_N: int, pairs_per_freq: int, lam: float) -> GroupCalibration:
    """X: device [n, d_model] anchor hidden states; rope_keys[l] device
    [n, d_R] (before rotation, pair (2j, 2j+1) at frequency key_theta[j]) and
    nope_keys[l] device [n, d_N] of each layer of the group."""
    d_R = rope_keys[0].shape[1] if rope_keys else 0
    ne = normal_equations(X, list(rope_keys) + list(nope_keys))
    return fit_from_normal_equations(ne, len(nope_keys), d_R, key_theta, r_N, pairs_per_freq, lam)


def fit_from_normal_equations(ne, m: int, d_R: int, key_theta: np.ndarray, r_N: int,
                              pairs_per_freq: int, lam: float) -> GroupCalibration:
    """The closed form from (X^T X, X^T Y, x_sum, y_sum, n) of normal_equations,
    Y = [rope keys of layers 0..m-1 | nope keys of layers 0..m-1]."""
    G, H, xs, ys, n = ne
    d = G.shape[0]
    d_N = (H.shape[1] - m * d_R) // m
    xm, ym = xs / n, ys / n
    # NoPE: centred regression of every layer's NoPE keys together
    HN = H[:, m * d_R:] - n * np.outer(xm, ym[m * d_R:])
    GN = G - n * np.outer(xm, xm)
    eye = lam * np.eye(d)
    P_N, D_N = _ridge_rank_solve(cho_factor(GN + eye), HN, r_N)
    b_all = ym[m * d_R:] - D_N @ (P_N.T @ xm)
    # RoPE: per frequency, a complex regression of the layers' pairs
    nf = d_R // 2
    a = pairs_per_freq
    r_R = 2 * nf * a
    P_R = np.zeros((d, r_R))
    D_R = np.zeros((m, d_R, r_R))
    cf = cho_factor(G + eye) if nf else None   # one factor serves every frequency
    for j in range(nf):
        cols_re = [l * d_R + 2 * j for l in range(m)]
        Hf = H[:, cols_re] + 1j * H[:, [c + 1 for c in cols_re]]
        Pf, Df = _ridge_rank_solve(cf, Hf, a)
        for i in range(a):
            q = j * a + i
            P_R[:, 2 * q], P_R[:, 2 * q + 1] = Pf[:, i].real, Pf[:, i].imag
            for l in range(m):
                c = Df[l, i]
                D_R[l, 2 * j, 2 * q], D_R[l, 2 * j, 2 * q + 1] = c.real, -c.imag
                D_R[l, 2 * j + 1, 2 * q], D_R[l, 2 * j + 1, 2 * q + 1] = c.imag, c.real
    r = r_R + r_N
    Dt = np.zeros((m, r, d_R + d_N))
    for l in range(m):
        Dt[l, :r_R, :d_R] = D_R[l].T
        Dt[l, r_R:, d_R:] = D_N[l * d_N:(l + 1) * d_N].T
    return GroupCalibration(P=np.concatenate([P_R, P_N], axis=1), Dt=Dt,
                            b=b_all.reshape(m, d_N), rope_theta=np.repeat(np.asarray(key_theta), a),
                            r_R=r_R, nope_off=d_R)
