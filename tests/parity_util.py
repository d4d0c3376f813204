"""Shared comparison helpers for the GPU parity tests."""

import sys

import numpy as np

RTOL_BF16 = 2e-3   # bf16 latent, fp32 accumulation
RTOL_FP8 = 2e-2    # fp8 latent with per-token scale
RTOL_FP32 = 1e-4   # fp32 latent (tiny configuration)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def score_err(g, o):
    """Per-element error normalised by |o| + rho, rho = RMS of the row."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    rho = np.sqrt(np.mean(o ** 2)) if o.size else 1.0
    return np.abs(g - o) / (np.abs(o) + rho + 1e-300), rho


def assert_scores_close(g, o, rtol, what=""):
    e, rho = score_err(g, o)
    if e.size:
        say(f"  {what}: max err {e.max():.3e}, p99.99 {np.quantile(e, 0.9999):.3e} (rtol {rtol})")
        bad = np.nonzero(e > rtol)[0]
        assert bad.size == 0, f"{what}: {bad.size} scores beyond rtol {rtol}; first {bad[:5]} " \
                              f"gpu {np.asarray(g)[bad[:5]]} oracle {np.asarray(o)[bad[:5]]}"


def assert_selection_band(sel_gpu, u_oracle, k, rtol, what=""):
    """Selections against the oracle's own scores: every id in the symmetric
    difference must score within 2*rtol*(|theta_k| + rho) of the k-th score."""
    u = np.asarray(u_oracle, dtype=np.float64)
    n = len(u)
    m = min(k, n)
    order = np.lexsort((np.arange(n), -u))
    ref = set(order[:m].tolist())
    got = set(int(x) for x in np.asarray(sel_gpu) if x >= 0)
    assert len(got) == m, f"{what}: {len(got)} selected, expected {m}"
    diff = ref ^ got
    if not diff:
        return
    theta = u[order[m - 1]]
    rho = np.sqrt(np.mean(u ** 2))
    band = 2 * rtol * (abs(theta) + rho)
    worst = max(abs(u[t] - theta) for t in diff)
    say(f"  {what}: {len(diff)} ids differ, all within {worst:.3e} of theta (band {band:.3e})")
    assert worst <= band, f"{what}: id off the threshold band by {worst} > {band}"
