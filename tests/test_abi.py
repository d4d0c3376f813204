"""C-ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before touching any device (CPU only)."""

import ctypes

import pytest

from sparse_attention_indexer_latent_amd import ops


@pytest.fixture(scope="module")
def L():
    return ops.lib()


def test_every_declared_symbol_is_exported(L):
    names = ops.header_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    for core in ["li_append_latent", "li_absorb_queries", "li_append_absorb", "li_score", "li_topk", "li_hs_anchor",
                 "li_hs_anchor_select", "li_hs_select"]:
        assert core in names


def _cache(**kw):
    c = dict(data=1, scale=None, block_table=2, n_seq=1, max_blocks=4, n_blocks=4, block_size=64,
             r=256, dtype=ops.LI_BF16)
    c.update(kw)
    return ops.LiCacheStruct(**c)


def test_validation_errors_are_host_side(L):
    FAKE = 0x1000  # never dereferenced: every case fails validation first
    assert L.li_topk(FAKE, 100, 1, FAKE, 100, 0, FAKE, None, None, 0, None) == ops.LI_ERR_INVALID
    assert b"k = 0" in L.li_last_error()
    assert L.li_topk(FAKE, 10, 1, FAKE, 100, 5, FAKE, None, None, 0, None) == ops.LI_ERR_INVALID
    assert L.li_topk(None, 10, 1, FAKE, 10, 5, FAKE, None, None, 0, None) == ops.LI_ERR_INVALID
    # no rows: a no-op that succeeds without a device
    assert L.li_topk(None, 10, 0, None, 10, 5, None, None, None, 0, None) == ops.LI_OK
    c = _cache(block_size=32)
    assert L.li_score(FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, FAKE, 64, ctypes.byref(c), FAKE,
                      64, None) == ops.LI_ERR_UNSUPPORTED
    c = _cache(r=250)
    assert L.li_score(FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, FAKE, 64, ctypes.byref(c), FAKE,
                      64, None) == ops.LI_ERR_UNSUPPORTED
    c = _cache(dtype=ops.LI_FP8_E4M3)  # fp8 without a scale array
    assert L.li_score(FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, FAKE, 64, ctypes.byref(c), FAKE,
                      64, None) == ops.LI_ERR_INVALID
    c = _cache()
    assert L.li_score(FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, FAKE, 300, ctypes.byref(c), FAKE,
                      300, None) == ops.LI_ERR_INVALID          # max_len beyond the block table
    assert L.li_score(FAKE, ops.LI_FP8_E4M3, FAKE, None, 1, 64, FAKE, FAKE, 64, ctypes.byref(c),
                      FAKE, 64, None) == ops.LI_ERR_INVALID     # q~ cannot be fp8
    # HS: B < k is invalid (the candidate set must hold k)
    assert L.li_hs_select(FAKE, 100, 3, FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, ctypes.byref(c),
                          200, FAKE, None, FAKE, 1 << 30, None) == ops.LI_ERR_INVALID
    assert b"B (100) < k (200)" in L.li_last_error()
    assert L.li_hs_select(FAKE, 100, 0, FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, ctypes.byref(c),
                          50, FAKE, None, FAKE, 1 << 30, None) == ops.LI_ERR_INVALID  # n_f < 1
    # append: P NULL requires d_model == r; odd r_R
    assert L.li_append_latent(FAKE, ops.LI_FP32, 4, 100, None, None, 0, FAKE, FAKE,
                              ctypes.byref(c), None, 0, None) == ops.LI_ERR_INVALID
    assert L.li_append_latent(FAKE, ops.LI_FP32, 4, 256, None, FAKE, 3, FAKE, FAKE,
                              ctypes.byref(c), None, 0, None) == ops.LI_ERR_INVALID
    assert L.li_absorb_queries(FAKE, ops.LI_FP32, 1, 1, 64, 128, FAKE, 0, None, 129, 256, FAKE,
                               None, None) == ops.LI_ERR_INVALID  # nope_off > d_I
    assert L.li_absorb_queries(FAKE, ops.LI_FP32, 0, 1, 64, 128, FAKE, 0, None, 64, 256, FAKE,
                               None, None) == ops.LI_ERR_INVALID  # n_layers < 1
    # the one-launch prelude: each half's own checks
    assert L.li_append_absorb(FAKE, ops.LI_FP32, 4, FAKE, 3, FAKE, FAKE, ctypes.byref(c), FAKE,
                              ops.LI_FP32, 1, 1, 64, 128, FAKE, 0, None, 64, FAKE, None,
                              None) == ops.LI_ERR_INVALID  # odd r_R
    assert L.li_append_absorb(FAKE, ops.LI_FP32, 4, None, 0, FAKE, FAKE, ctypes.byref(c), FAKE,
                              ops.LI_FP32, 0, 1, 64, 128, FAKE, 0, None, 64, FAKE, None,
                              None) == ops.LI_ERR_INVALID  # n_layers < 1
    assert L.li_append_absorb(FAKE, ops.LI_FP32, 4, None, 0, FAKE, FAKE, ctypes.byref(c), FAKE,
                              ops.LI_FP32, 1, 1, 64, 130, FAKE, 0, None, 64, FAKE, None,
                              None) == ops.LI_ERR_UNSUPPORTED  # d_I not a multiple of 4
    assert L.li_append_absorb(FAKE, ops.LI_FP32, 0, None, 0, FAKE, FAKE, ctypes.byref(c), FAKE,
                              ops.LI_FP32, 1, 0, 64, 128, FAKE, 0, None, 64, FAKE, None,
                              None) == ops.LI_OK  # nothing to do: no launch
    # the fused anchor call: B < k, max_len > ld, NULL outputs, too small a workspace
    # (rows of 20000 positions: a length that needs the workspace)
    c = _cache(max_blocks=400)
    big = L.li_hs_anchor_workspace_bytes(4, 20000)
    assert big > 0
    assert L.li_hs_anchor(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                          FAKE, 20000, 100, FAKE, 200, FAKE, FAKE, big, None,
                          None) == ops.LI_ERR_INVALID
    assert b"B (100) < k (200)" in L.li_last_error()
    assert L.li_hs_anchor(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                          FAKE, 128, 100, FAKE, 10, FAKE, FAKE, big, None,
                          None) == ops.LI_ERR_INVALID  # max_len > ld
    assert L.li_hs_anchor(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                          None, 20000, 100, FAKE, 10, FAKE, FAKE, big, None,
                          None) == ops.LI_ERR_INVALID  # scores NULL
    assert L.li_hs_anchor(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                          FAKE, 20000, 100, FAKE, 10, FAKE, FAKE, big - 1, None,
                          None) == ops.LI_ERR_INVALID  # workspace too small
    assert b"workspace needs" in L.li_last_error()
    # no queries: a no-op that succeeds without a device
    assert L.li_hs_anchor(FAKE, ops.LI_FP32, FAKE, None, 0, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                          FAKE, 20000, 100, FAKE, 10, FAKE, FAKE, big, None, None) == ops.LI_OK


def test_workspace_sizes(L):
    assert L.li_append_workspace_bytes(4, 7168, 256, 0) == 0
    assert L.li_append_workspace_bytes(4, 7168, 256, 1) > 0
    assert L.li_hs_workspace_bytes(1, 4, 8192, 2048) >= 4 * 8192 * 4
    assert L.li_hs_workspace_bytes(3, 4, 8192, 2048) >= 3 * 4 * 8192 * 4
    # the anchor workspace: none for rows of at most 8192 positions (one single-workgroup
    # selection per output), else sized by rows and length
    assert L.li_hs_anchor_workspace_bytes(4, 4096) == 0
    assert L.li_hs_anchor_workspace_bytes(4, 8192) == 0
    assert L.li_hs_anchor_workspace_bytes(4, 131072) > L.li_hs_anchor_workspace_bytes(4, 8193) > 0
    assert L.li_hs_anchor_workspace_bytes(64, 16384) >= 64 * 16384 * 4


def test_anchor_selection_rejects_rows_beyond_its_segment_table(L):
    """The anchor selection handles rows of at most 1024 segments of 2048
    positions; longer rows are refused on the host, before any launch."""
    FAKE = 0x1000
    lim = 1024 * 2048
    big_ws = 1 << 40  # never reached: the length check comes first
    assert L.li_hs_anchor_select(FAKE, lim + 1, 1, FAKE, lim + 1, 8192, FAKE, 2048, FAKE, FAKE,
                                 big_ws, None) == ops.LI_ERR_UNSUPPORTED
    assert b"exceeds" in L.li_last_error()
    c = _cache(max_blocks=(lim // 64) + 2, n_blocks=(lim // 64) + 2)
    assert L.li_hs_anchor(FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE, FAKE, lim + 1,
                          ctypes.byref(c), FAKE, lim + 1, 8192, FAKE, 2048, FAKE, FAKE, big_ws, None,
                          None) == ops.LI_ERR_UNSUPPORTED
    assert b"exceeds" in L.li_last_error()
    # at the limit the length check passes (the workspace check fails next)
    assert L.li_hs_anchor_select(FAKE, lim, 1, FAKE, lim, 8192, FAKE, 2048, FAKE, FAKE, 1, None) \
        == ops.LI_ERR_INVALID
    assert b"workspace needs" in L.li_last_error()


def test_hs_select_noalloc_checks_on_the_host(L):
    """The no-allocation follower step takes li_hs_select's checks, and
    refuses calls whose workspace would not fit its fixed array, before
    touching a device."""
    FAKE = 0x1000
    c = _cache()
    assert "li_hs_select_noalloc" in ops.header_symbols()
    assert L.li_hs_select_noalloc(FAKE, 100, 3, FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE,
                                  ctypes.byref(c), 200, FAKE, None, None) == ops.LI_ERR_INVALID
    assert b"B (100) < k (200)" in L.li_last_error()
    assert L.li_hs_workspace_bytes(64, 1, 65536, 16) > ops.HS_NOALLOC_SCRATCH_BYTES
    assert L.li_hs_select_noalloc(FAKE, 65536, 64, FAKE, ops.LI_FP32, FAKE, None, 1, 64, FAKE,
                                  ctypes.byref(c), 16, FAKE, None, None) == ops.LI_ERR_UNSUPPORTED
    assert b"scratch" in L.li_last_error()
    # the benchmark's follower step fits
    assert L.li_hs_workspace_bytes(3, 4, 8192, 2048) <= ops.HS_NOALLOC_SCRATCH_BYTES
    assert L.li_hs_select_noalloc(None, 8192, 3, None, ops.LI_FP32, None, None, 0, 64, None,
                                  ctypes.byref(c), 2048, None, None, None) == ops.LI_OK  # no queries


def test_header_constant_matches_binding():
    import re
    txt = open(ops.HEADER).read()
    m = re.search(r"#define LI_HS_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == ops.HS_NOALLOC_SCRATCH_BYTES


def test_score_topk_checks_on_the_host(L):
    FAKE = 0x1000
    c = _cache(max_blocks=400)
    big = L.li_hs_anchor_workspace_bytes(4, 20000)
    assert L.li_score_topk(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                           FAKE, 20000, 0, FAKE, FAKE, big, None, None) == ops.LI_ERR_INVALID
    assert b"k = 0" in L.li_last_error()
    assert L.li_score_topk(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                           FAKE, 20000, 70000, FAKE, FAKE, big, None, None) == ops.LI_ERR_INVALID
    assert L.li_score_topk(FAKE, ops.LI_FP32, FAKE, None, 4, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                           FAKE, 20000, 16, FAKE, FAKE, big - 1, None, None) == ops.LI_ERR_INVALID
    assert b"workspace needs" in L.li_last_error()
    assert L.li_score_topk(FAKE, ops.LI_FP32, FAKE, None, 0, 64, FAKE, FAKE, 20000, ctypes.byref(c),
                           FAKE, 20000, 16, FAKE, FAKE, big, None, None) == ops.LI_OK
