"""The fused scans (li_score_topk, li_hs_anchor: scores plus the key
histograms the selection starts from) against the plain scan (li_score):
every position scored bit for bit as li_score scores it, nothing written past
a length, and the same results on three calls in a row on one workspace."""

import numpy as np
import pytest
import torch

from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload

from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["b4-32k-bf16", "b1-128k-bf16", "b4-128k-fp8r192", "ragged-fp8"])
def test_fused_scan_equals_plain_scan(case):
    """Scores of li_score_topk and li_hs_anchor against li_score, bit for
    bit, into NaN-filled buffers, three calls in a row on one workspace;
    selections identical across the calls and to li_topk on li_score's."""
    say(f"fused scan {case}")
    if case == "b4-32k-bf16":
        wl = W.make_decode("b4-32k", 3, 7, G=1, H=64, r=256, d_I=128, k=2048, B=8192,
                           cache_dtype="bf16", lens=[32768] * 4, plant_frac=0.01,
                           plant_factor=3.0, permute_blocks=True)
    elif case == "b1-128k-bf16":
        wl = W.hs_128k(1, G=1)
    elif case == "b4-128k-fp8r192":
        wl = W.hs_128k(4, r=192, cache_dtype="fp8", scale_block=128, G=1)
    else:
        wl = W.named("ragged-16x8k-128k-fp8")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb()
    args = (dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, dw.q_len, dw.max_len, dw.cache)
    ref = ops.score(*args)
    torch.cuda.synchronize()
    ref_np = ref.cpu().numpy()
    ws = ops.hs_anchor_workspace(wl.n_q, dw.max_len)
    ql = wl.q_len
    sels = []
    for call in range(3):
        out = torch.full((wl.n_q, dw.max_len + 5), float("nan"), device="cuda")
        if call == 1:
            _, cand, sel = ops.hs_anchor(*args, 8192, 2048, scores=out, ws=ws)
            s = (cand.cpu().numpy(), sel.cpu().numpy())
        else:
            _, sel = ops.score_topk(*args, 2048, scores=out, ws=ws)
            s = sel.cpu().numpy()
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for q in range(wl.n_q):
            L = int(ql[q])
            assert not np.isnan(o[q, :L]).any(), (call, q, "a position was not scored")
            assert np.array_equal(o[q, :L].view(np.uint32), ref_np[q, :L].view(np.uint32)), (call, q)
            assert np.isnan(o[q, L:]).all(), (call, q, "written past the length")
        sels.append(s)
    assert np.array_equal(sels[0], sels[2])
    ref_sel = ops.topk(ref, dw.q_len, dw.max_len, 2048).cpu().numpy()
    assert np.array_equal(sels[0], ref_sel)
    assert np.array_equal(sels[1][1], ref_sel)
