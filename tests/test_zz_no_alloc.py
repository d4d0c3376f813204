"""li_hs_select_noalloc (the follower step on the library's own fixed
workspace, for callers that cannot allocate) against li_hs_select on a
caller-owned workspace: identical selections and candidate scores, bit for
bit, over calls in a row that shrink and change path (matrix-core candidate
scan on a bf16 cache, the fp8 scorer, candidate rows longer than 16K), so
that a call never depends on what an earlier one left in the array."""

import numpy as np
import pytest
import torch

from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload

from parity_util import say

pytestmark = pytest.mark.gpu


def _candidates(rng, lens, B):
    """Ascending distinct token ids per query, min(B, L) of them, -1 padded."""
    out = np.full((len(lens), B), -1, dtype=np.int32)
    for i, L in enumerate(lens):
        m = min(B, int(L))
        out[i, :m] = np.sort(rng.choice(int(L), m, replace=False))
    return out


CASES = [
    # (cache dtype, lens, B, k, n_f): the benchmark's follower shape first
    ("bf16", [20000, 9000, 15000, 8292], 8192, 2048, 3),
    ("fp8", [700, 1500], 700, 50, 1),        # smaller, another scorer
    ("bf16", [30000, 25000], 20000, 2048, 2),  # rows > 16K: lengths and multi-pass top-k
    ("bf16", [3000], 256, 16, 1),            # smallest last
]


def test_noalloc_equals_workspace_call_over_calls_in_a_row():
    rng = np.random.default_rng(77)
    for dt, lens, B, k, n_f in CASES:
        say(f"hs_select_noalloc: {dt} lens={lens} B={B} k={k} n_f={n_f}")
        wl = W.small_decode(50 + B, n_seq=len(lens), lens=lens, H=64, r=256, d_I=128, G=n_f + 1,
                            k=k, B=B, cache_dtype=dt, plant=10, factor=3.0)
        dw = DeviceWorkload(wl, hold_last=False)
        dw.absorb()
        cand = torch.from_numpy(_candidates(rng, lens, B)).cuda()
        n_q = len(lens)
        qt, w, beta = dw.q_tilde[1:], dw.w[1:], dw.beta[1:]
        ref_idx, ref_cs = ops.hs_select(cand, qt, w, beta, dw.q_seq, dw.cache, k,
                                        want_scores=True)
        out_idx = torch.full((n_f, n_q, k), -7, dtype=torch.int32, device="cuda")
        out_cs = torch.full((n_f, n_q, B), 0.5, dtype=torch.float32, device="cuda")
        ops.hs_select(cand, qt, w, beta, dw.q_seq, dw.cache, k, out_idx=out_idx,
                      cand_scores=out_cs, noalloc=True)
        # and once more without candidate scores (the array holds them then)
        out_idx2 = torch.full((n_f, n_q, k), -7, dtype=torch.int32, device="cuda")
        ops.hs_select(cand, qt, w, beta, dw.q_seq, dw.cache, k, out_idx=out_idx2, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(out_idx, ref_idx), (dt, lens, B)
        assert torch.equal(out_idx2, ref_idx), (dt, lens, B)
        assert torch.equal(out_cs.view(torch.int32), ref_cs.view(torch.int32)), (dt, lens, B)
        # sanity of what both returned: ids inside the candidate lists
        ci = cand.cpu().numpy()
        ri = ref_idx.cpu().numpy()
        for f in range(n_f):
            for s in range(n_q):
                got = ri[f, s][ri[f, s] >= 0]
                assert len(got) == min(k, lens[s], B)
                assert set(got.tolist()) <= set(ci[s][ci[s] >= 0].tolist())
        del dw
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_call_beyond_its_array():
    """More rows x B than the fixed array holds: refused on the host."""
    wl = W.small_decode(60, n_seq=1, lens=[100], H=64, r=256, d_I=128, G=2, k=16, B=65536,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    need = ops.lib().li_hs_workspace_bytes(64, 1, 65536, 16)
    assert need > ops.HS_NOALLOC_SCRATCH_BYTES
    qt = torch.zeros((64, 1, 64, 256), device="cuda")
    w = torch.zeros((64, 1, 64), device="cuda")
    cand = torch.full((1, 65536), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(ops.LiError) as e:
        ops.hs_select(cand, qt, w, None, dw.q_seq, dw.cache, 16,
                      out_idx=torch.empty((64, 1, 16), dtype=torch.int32, device="cuda"),
                      noalloc=True)
    assert e.value.status == ops.LI_ERR_UNSUPPORTED and "scratch" in str(e.value)
