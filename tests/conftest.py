import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU-side oracle work")


def pytest_collection_modifyitems(config, items):
    """Build the library if nothing is built; skip GPU tests without a GPU."""
    import torch

    lib = os.path.join(ROOT, "sparse_attention_indexer_latent_amd", "liblatentindex.so")
    if not os.path.exists(lib):
        from sparse_attention_indexer_latent_amd import build
        build.build()
    if not torch.cuda.is_available():
        skip = pytest.mark.skip(reason="no GPU in this environment")
        for it in items:
            if "gpu" in it.keywords:
                it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """The error margins of every score comparison that ran (worst per
    group), so that a quiet run's log still shows them."""
    try:
        from parity_util import margins_summary
    except Exception:  # pragma: no cover
        return
    groups = margins_summary()
    if not groups:
        return
    terminalreporter.write_sep("-", "parity margins (worst per group and tolerance)")
    for (key, tol), (mx, p, ratio, c, n) in sorted(groups.items()):
        terminalreporter.write_line(f"{key}: max {mx:.3e} p99.99 {p:.3e} tol {tol:.3e} "
                                    f"(worst {ratio:.3f} of tol; {c} checks, {n} values)")
