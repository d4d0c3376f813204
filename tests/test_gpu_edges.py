"""GPU edge cases of the selection and scoring calls: rows at the longest
length the few-long-rows selection supports (2,097,152 positions, 1024
segments), empty rows inside a batch, and empty batches."""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_indexer_latent_amd import ops
from sparse_attention_indexer_latent_amd import workloads as W
from sparse_attention_indexer_latent_amd.runtime import DeviceWorkload

from parity_util import say

pytestmark = pytest.mark.gpu

MAXLEN = 2_097_152


def _rows(n_rows, L, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((n_rows, L)).astype(np.float32)
    u[:, ::1000] *= 4.0                       # a heavy tail
    u[0, 5:40] = u[0, 4]                       # ties
    return u


def test_topk_at_the_longest_row():
    """Two rows of 2,097,152 positions (one cut to 1,500,001): li_topk and the
    nested anchor selection exact against the brute-force rank of the same
    scores."""
    say("top-k / anchor selection at 2,097,152 positions")
    u = _rows(2, MAXLEN, 60)
    valid = np.array([MAXLEN, 1_500_001], dtype=np.int32)
    ud = torch.from_numpy(u).cuda()
    vd = torch.from_numpy(valid).cuda()
    idx = ops.topk(ud, vd, MAXLEN, 2048)
    cand, sel = ops.hs_anchor_select(ud, vd, MAXLEN, 8192, 2048)
    torch.cuda.synchronize()
    idx, cand, sel = idx.cpu().numpy(), cand.cpu().numpy(), sel.cpu().numpy()
    for r in range(2):
        L = int(valid[r])
        row = u[r, :L].astype(np.float64)
        ref_k = O.topk(row, 2048)
        assert np.array_equal(idx[r], ref_k), r
        assert np.array_equal(sel[r], ref_k), r
        assert np.array_equal(cand[r], O.topk(row, 8192)), r


def test_empty_rows_inside_a_batch():
    """valid_len 0 rows next to ordinary ones: all -1 for top-k and both
    anchor outputs; the scan writes nothing for a zero-length query."""
    say("empty rows inside a batch")
    u = _rows(3, 20000, 61)
    valid = np.array([0, 20000, 0], dtype=np.int32)
    ud = torch.from_numpy(u).cuda()
    vd = torch.from_numpy(valid).cuda()
    idx = ops.topk(ud, vd, 20000, 100).cpu().numpy()
    cand, sel = ops.hs_anchor_select(ud, vd, 20000, 500, 100)
    cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
    for r in (0, 2):
        assert np.all(idx[r] == -1) and np.all(cand[r] == -1) and np.all(sel[r] == -1)
    assert np.array_equal(idx[1], O.topk(u[1].astype(np.float64), 100))
    assert np.array_equal(cand[1], O.topk(u[1].astype(np.float64), 500))
    # a zero-length query between two others, on the matrix-core scan
    wl = W.small_decode(62, n_seq=3, lens=[300, 700, 128], H=64, r=256, d_I=128, G=1, k=16,
                        cache_dtype="bf16")
    dw = DeviceWorkload(wl, hold_last=False)
    dw.absorb()
    q_len = torch.tensor([300, 0, 128], dtype=torch.int32, device="cuda")
    out = torch.full((3, 704), 12345.0, device="cuda")
    ops.score(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, q_len, 300, dw.cache, scores=out)
    _, sel = ops.score_topk(dw.q_tilde[0], dw.w[0], dw.beta[0], dw.q_seq, q_len, 300, dw.cache, 16)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[1] == 12345.0) and np.all(o[0, 300:] == 12345.0) and np.all(o[2, 128:] == 12345.0)
    s = sel.cpu().numpy()
    assert np.all(s[1] == -1)
    assert np.array_equal(s[0], O.topk(o[0, :300].astype(np.float64), 16))
    assert np.array_equal(s[2], O.topk(o[2, :128].astype(np.float64), 16))


def test_empty_batches_are_no_ops():
    """n_q = 0 / n_rows = 0 through the C ABI with real buffers: success and
    nothing written."""
    say("empty batches")
    lib = ops.lib()
    st = torch.cuda.current_stream().cuda_stream
    u = torch.zeros((1, 64), device="cuda")
    v = torch.ones(1, dtype=torch.int32, device="cuda")
    out = torch.full((1, 8), 7, dtype=torch.int32, device="cuda")
    assert lib.li_topk(u.data_ptr(), 64, 0, v.data_ptr(), 64, 8, out.data_ptr(), None, None, 0,
                       st) == ops.LI_OK
    ws = ops.hs_anchor_workspace(1, 64)
    assert lib.li_hs_anchor_select(u.data_ptr(), 64, 0, v.data_ptr(), 64, 8, out.data_ptr(), 4,
                                   None, ws.data_ptr(), ws.numel(), st) == ops.LI_OK
    torch.cuda.synchronize()
    assert torch.all(out == 7)


@pytest.mark.parametrize("L", [8192, 40000])
def test_selection_lengths_out_of_range_are_clamped(L):
    """Device-side valid lengths outside [0, max_len] (a caller error the host
    cannot see) are clamped by every selection kernel: a negative length
    selects nothing, one above max_len selects as max_len; both the
    single-workgroup path (rows <= 8192) and the multi-workgroup path."""
    say(f"out-of-range valid lengths, L={L}")
    rng = np.random.default_rng(L)
    u = np.round(rng.standard_normal((3, L)), 2).astype(np.float32)
    valid = np.array([-5, L + 1000, L // 2], dtype=np.int32)
    ud = torch.from_numpy(u).cuda()
    vd = torch.from_numpy(valid).cuda()
    idx = ops.topk(ud, vd, L, 2048).cpu().numpy()
    cand, sel = ops.hs_anchor_select(ud, vd, L, 4096, 2048)
    cand, sel = cand.cpu().numpy(), sel.cpu().numpy()
    for i, n in enumerate([0, L, L // 2]):
        row = u[i, :n].astype(np.float64)
        assert np.array_equal(idx[i], O.pad(O.topk(row, 2048), 2048)), i
        assert np.array_equal(cand[i], O.pad(O.hs_candidates(row, 4096), 4096)), i
        assert np.array_equal(sel[i], O.pad(O.topk(row, 2048), 2048)), i


def test_short_rows_candidates_only_and_zero_length():
    """The single-workgroup anchor selection when only C is asked for (B
    covering the row: C is every position), and max_len = 0 (every output
    padding)."""
    say("short rows: C only, and max_len = 0")
    u = np.round(np.random.default_rng(5).standard_normal((2, 3000)), 1).astype(np.float32)
    vd = torch.tensor([3000, 1234], dtype=torch.int32, device="cuda")
    ud = torch.from_numpy(u).cuda()
    cand, sel = ops.hs_anchor_select(ud, vd, 3000, 4096, 100, want_sel=False)
    assert sel is None
    c = cand.cpu().numpy()
    for i, n in enumerate([3000, 1234]):
        assert np.array_equal(c[i], O.pad(np.arange(n), 4096)), i
    z = torch.zeros((2, 16), device="cuda")
    vz = torch.zeros(2, dtype=torch.int32, device="cuda")
    cand, sel = ops.hs_anchor_select(z, vz, 0, 64, 8)
    idx = ops.topk(z, vz, 0, 8)
    assert torch.all(cand == -1) and torch.all(sel == -1) and torch.all(idx == -1)
