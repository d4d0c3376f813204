"""Shared comparison helpers for the GPU parity tests."""

import sys

import numpy as np

RTOL_BF16 = 2e-3   # bf16 latent, fp32 accumulation
RTOL_FP8 = 2e-2    # fp8 latent with per-token scale
RTOL_FP32 = 1e-4   # fp32 latent (tiny configuration)


# (what, max error, p99.99 error, rtol) of every score comparison, printed at
# the end of the session by conftest.py so the run's log carries the margins.
MARGINS = []


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
        mx, p = float(e.max()), float(np.quantile(e, 0.9999))
        MARGINS.append((what, mx, p, rtol, e.size))
        say(f"  {what}: max err {mx:.3e}, p99.99 {p:.3e} (rtol {rtol})")
        bad = np.nonzero(e > rtol)[0]
        assert bad.size == 0, f"{what}: {bad.size} scores beyond rtol {rtol}; first {bad[:5]} " \
                              f"gpu {np.asarray(g)[bad[:5]]} oracle {np.asarray(o)[bad[:5]]}"


def assert_selection_band(sel_gpu, u_oracle, k, rtol, what="", ids=None):
    """Selections against the oracle's own scores: every id in the symmetric
    difference must score within 2*rtol*(|theta_k| + rho) of the k-th score.
    ids (optional): the token id of each entry of u_oracle (ascending), for a
    selection within a candidate set."""
    u = np.asarray(u_oracle, dtype=np.float64)
    n = len(u)
    m = min(k, n)
    ids = np.arange(n) if ids is None else np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -u))
    ref = set(ids[order[:m]].tolist())
    got_arr = np.asarray(sel_gpu)
    got = set(int(x) for x in got_arr if x >= 0)
    assert len(got) == m, f"{what}: {len(got)} selected, expected {m}"
    assert np.all(got_arr[m:] == -1), f"{what}: padding beyond {m} entries"
    diff = ref ^ got
    theta = u[order[m - 1]] if m else 0.0
    rho = np.sqrt(np.mean(u ** 2)) if n else 1.0
    band = 2 * rtol * (abs(theta) + rho)
    if not diff:
        MARGINS.append((f"{what} [selection]", 0.0, 0.0, band, m))
        return
    pos = {int(t): j for j, t in enumerate(ids)}
    assert all(t in pos for t in diff), f"{what}: selected ids outside the candidate set"
    worst = max(abs(u[pos[t]] - theta) for t in diff)
    MARGINS.append((f"{what} [selection: {len(diff)} ids differ]", worst, worst, band, m))
    say(f"  {what}: {len(diff)} ids differ, all within {worst:.3e} of theta (band {band:.3e})")
    assert worst <= band, f"{what}: id off the threshold band by {worst} > {band}"


def margins_summary():
    """Per comparison group (its description with numbers and parenthesised
    details masked) and tolerance: the worst max and p99.99 errors, the worst
    ratio of error to tolerance, and how many checks and values it covers."""
    import re
    groups = {}
    for what, mx, p, tol, n in MARGINS:
        key = re.sub(r"\([^)]*\)", "", what)
        key = re.sub(r"\d+", "#", key).strip()
        g = groups.setdefault((key, tol), [0.0, 0.0, 0.0, 0, 0])
        g[0] = max(g[0], mx)
        g[1] = max(g[1], p)
        g[2] = max(g[2], mx / tol if tol else 0.0)
        g[3] += 1
        g[4] += n
    return groups
