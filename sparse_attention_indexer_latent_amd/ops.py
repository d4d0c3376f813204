"""Thin Python binding of liblatentindex.so (include/latentindex.h).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors must be contiguous device tensors of the current CUDA (HIP) device;
work is enqueued on torch's current stream.  Outputs that are not passed in
are allocated with torch.  A missing library raises immediately: there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblatentindex.so")
HEADER = os.path.join(HERE, "..", "include", "latentindex.h")

LI_OK, LI_ERR_INVALID, LI_ERR_UNSUPPORTED, LI_ERR_HIP = 0, 1, 2, 3
LI_FP32, LI_BF16, LI_FP8_E4M3 = 0, 1, 2
BLOCK = 64


class LiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class LiCacheStruct(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("n_seq", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("r", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale_block", ctypes.c_int32),
    ]


_lib = None

_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "li_last_error": (ctypes.c_char_p, []),
    "li_check_device": (_I32, []),
    "li_append_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "li_append_latent": (_I32, [_P, _I32, _I32, _I32, _P, _P, _I32, _P, _P,
                                ctypes.POINTER(LiCacheStruct), _P, _SZ, _P]),
    "li_absorb_queries": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _I32, _I32, _P, _P,
                                 _P]),
    "li_append_absorb": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, ctypes.POINTER(LiCacheStruct),
                                _P, _I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _I32, _P, _P,
                                _P]),
    "li_score": (_I32, [_P, _I32, _P, _P, _I32, _I32, _P, _P, _I32,
                        ctypes.POINTER(LiCacheStruct), _P, _I64, _P]),
    "li_topk_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "li_topk": (_I32, [_P, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "li_hs_anchor_workspace_bytes": (_SZ, [_I32, _I32]),
    "li_hs_anchor_select": (_I32, [_P, _I64, _I32, _P, _I32, _I32, _P, _I32, _P, _P, _SZ, _P]),
    "li_hs_anchor": (_I32, [_P, _I32, _P, _P, _I32, _I32, _P, _P, _I32,
                            ctypes.POINTER(LiCacheStruct), _P, _I64, _I32, _P, _I32, _P, _P, _SZ,
                            _P, _P]),
    "li_score_topk": (_I32, [_P, _I32, _P, _P, _I32, _I32, _P, _P, _I32,
                             ctypes.POINTER(LiCacheStruct), _P, _I64, _I32, _P, _P, _SZ, _P, _P]),
    "li_hs_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "li_calib_gram": (_I32, [_P, _I32, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _P, _I32, _P]),
    "li_hs_select": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, _P,
                            ctypes.POINTER(LiCacheStruct), _I32, _P, _P, _P, _SZ, _P]),
    "li_hs_select_noalloc": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, _P,
                                    ctypes.POINTER(LiCacheStruct), _I32, _P, _P, _P]),
}

HS_NOALLOC_SCRATCH_BYTES = 8 << 20  # LI_HS_NOALLOC_SCRATCH_BYTES


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_indexer_latent_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Function names declared in include/latentindex.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(li_[a-z_0-9]+)\s*\(", txt)))


def _check(status: int) -> None:
    if status != LI_OK:
        raise LiError(status, lib().li_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LI_FP32
    if t.dtype == torch.bfloat16:
        return LI_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return LI_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _numel(t: torch.Tensor, n: int, name: str):
    """The library takes raw pointers: check the extent it will touch."""
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")


class Cache:
    """A paged shared latent cache of one layer group (device tensors).

    data: [n_blocks, 64, r] float32 | bfloat16 | uint8 (E4M3FN codes)
    scale: fp8 only: float32 [n_blocks, 64] (one scale per token) or
           [n_blocks, 64, ceil(r / 128)] with scale_block = 128
    block_table: int32 [n_seq, max_blocks]
    """

    def __init__(self, data: torch.Tensor, block_table: torch.Tensor,
                 scale: Optional[torch.Tensor] = None, scale_block: int = 0):
        _need(data, "cache data")
        _need(block_table, "block_table", torch.int32)
        if scale is not None:
            _need(scale, "scale", torch.float32)
            ns = 1 if scale_block == 0 else -(-data.shape[2] // scale_block)
            if scale.numel() != data.shape[0] * data.shape[1] * ns:
                raise ValueError(f"scale must hold [n_blocks, 64, {ns}] values")
        self.data, self.block_table, self.scale = data, block_table, scale
        self.scale_block = scale_block
        self.dtype = _dtype_code(data)
        self._s = LiCacheStruct(
            data=data.data_ptr(), scale=_ptr(scale), block_table=block_table.data_ptr(),
            n_seq=block_table.shape[0], max_blocks=block_table.shape[1],
            n_blocks=data.shape[0], block_size=data.shape[1], r=data.shape[2], dtype=self.dtype,
            scale_block=scale_block)

    @classmethod
    def empty(cls, n_blocks: int, r: int, dtype: str, block_table: torch.Tensor, device="cuda",
              scale_block: int = 0):
        tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]
        data = torch.empty((n_blocks, BLOCK, r), dtype=tdt, device=device)
        scale = None
        if dtype == "fp8":
            ns = 1 if scale_block == 0 else -(-r // scale_block)
            shape = (n_blocks, BLOCK) if scale_block == 0 else (n_blocks, BLOCK, ns)
            scale = torch.empty(shape, dtype=torch.float32, device=device)
        return cls(data, block_table, scale, scale_block)

    @property
    def bytes_per_token(self) -> int:
        """Bytes one token occupies in the cache (codes plus scales)."""
        el = self.data.element_size() * self.data.shape[2]
        return el + (0 if self.scale is None else
                     4 * (self.scale.numel() // (self.data.shape[0] * self.data.shape[1])))

    @property
    def r(self) -> int:
        return self.data.shape[2]

    def struct(self):
        return ctypes.byref(self._s)


def append_latent(x: torch.Tensor, cache: Cache, seq_idx: torch.Tensor, pos: torch.Tensor,
                  P: Optional[torch.Tensor] = None, rope_theta: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None) -> None:
    _need(x, "x", (torch.float32, torch.bfloat16))
    _need(seq_idx, "seq_idx", torch.int32)
    _need(pos, "pos", torch.int32)
    n_tok, d_model = x.shape
    if seq_idx.numel() != n_tok or pos.numel() != n_tok:
        raise ValueError("seq_idx and pos must hold n_tok entries")
    if P is not None:
        _need(P, "P", x.dtype)
        if P.numel() != d_model * cache.r:
            raise ValueError("P must be [d_model, r]")
    r_R = 0
    if rope_theta is not None:
        _need(rope_theta, "rope_theta", torch.float32)
        r_R = 2 * rope_theta.numel()
    need = lib().li_append_workspace_bytes(n_tok, d_model, cache.r, int(P is not None))
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().li_append_latent(x.data_ptr(), _dtype_code(x), n_tok, d_model, _ptr(P),
                                  _ptr(rope_theta), r_R, seq_idx.data_ptr(), pos.data_ptr(),
                                  cache.struct(), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream()))


def absorb_queries(q: torch.Tensor, Dt: torch.Tensor, b: Optional[torch.Tensor] = None,
                   nope_off: Optional[int] = None, q_tilde: Optional[torch.Tensor] = None,
                   beta: Optional[torch.Tensor] = None, per_head: bool = False):
    """One layer: q [n_q, H, d_I], Dt [r, d_I] (or [H, r, d_I] with per_head),
    b [d_I - nope_off] -> (q~ [n_q, H, r], beta [n_q, H]).  Several layers in
    one call: every operand gains a leading layer dimension."""
    _need(q, "q", (torch.float32, torch.bfloat16))
    _need(Dt, "Dt", torch.float32)
    layered = q.dim() == 4
    L = q.shape[0] if layered else 1
    n_q, H, d_I = q.shape[-3:]
    r = Dt.shape[-2]
    stride = r * d_I if per_head else 0
    no = d_I if nope_off is None else nope_off
    if b is not None:
        _need(b, "b", torch.float32)
    lead = (L,) if layered else ()
    if Dt.numel() != L * (H if per_head else 1) * r * d_I:
        raise ValueError("Dt must hold [r, d_I] (per head with per_head) for every layer")
    if b is not None and b.numel() != L * (d_I - no):
        raise ValueError("b must be [layers, d_I - nope_off]")
    if q_tilde is None:
        q_tilde = torch.empty(lead + (n_q, H, r), dtype=torch.float32, device=q.device)
    if beta is None:
        beta = torch.empty(lead + (n_q, H), dtype=torch.float32, device=q.device)
    _need(q_tilde, "q_tilde", torch.float32)
    _need(beta, "beta", torch.float32)
    if q_tilde.numel() != L * n_q * H * r or beta.numel() != L * n_q * H:
        raise ValueError("q_tilde must be [layers, n_q, H, r] and beta [layers, n_q, H]")
    _check(lib().li_absorb_queries(q.data_ptr(), _dtype_code(q), L, n_q, H, d_I, Dt.data_ptr(),
                                   stride, _ptr(b), no, r, q_tilde.data_ptr(), _ptr(beta),
                                   _stream()))
    return q_tilde, beta


def append_absorb(x: torch.Tensor, cache: Cache, seq_idx: torch.Tensor, pos: torch.Tensor,
                  q: torch.Tensor, Dt: torch.Tensor, b: Optional[torch.Tensor],
                  nope_off: Optional[int], q_tilde: torch.Tensor, beta: Optional[torch.Tensor],
                  rope_theta: Optional[torch.Tensor] = None, per_head: bool = False) -> None:
    """append_latent(x, cache, seq_idx, pos, rope_theta=rope_theta) (no
    projection: x is [n_tok, r]) and absorb_queries(q, Dt, b, nope_off,
    q_tilde, beta, per_head) in one launch; operands as for those two."""
    _need(x, "x", (torch.float32, torch.bfloat16))
    _need(seq_idx, "seq_idx", torch.int32)
    _need(pos, "pos", torch.int32)
    _need(q, "q", (torch.float32, torch.bfloat16))
    _need(Dt, "Dt", torch.float32)
    _need(q_tilde, "q_tilde", torch.float32)
    if b is not None:
        _need(b, "b", torch.float32)
    if beta is not None:
        _need(beta, "beta", torch.float32)
    n_tok, d_model = x.shape
    if d_model != cache.r or Dt.shape[-2] != cache.r:
        raise ValueError(f"x and Dt must have r = {cache.r} columns / rows")
    r_R = 0
    if rope_theta is not None:
        _need(rope_theta, "rope_theta", torch.float32)
        r_R = 2 * rope_theta.numel()
    L = q.shape[0] if q.dim() == 4 else 1
    n_q, H, d_I = q.shape[-3:]
    stride = cache.r * d_I if per_head else 0
    no = d_I if nope_off is None else nope_off
    # the library takes raw pointers: check the extents it will touch
    if seq_idx.numel() != n_tok or pos.numel() != n_tok:
        raise ValueError("seq_idx and pos must hold n_tok entries")
    if Dt.numel() != L * (H if per_head else 1) * cache.r * d_I:
        raise ValueError(f"Dt must hold {L} layers of {'H x ' if per_head else ''}[r, d_I]")
    if q_tilde.numel() != L * n_q * H * cache.r:
        raise ValueError("q_tilde must be [layers, n_q, H, r]")
    if beta is not None and beta.numel() != L * n_q * H:
        raise ValueError("beta must be [layers, n_q, H]")
    if b is not None and b.numel() != L * (d_I - no):
        raise ValueError("b must be [layers, d_I - nope_off]")
    _check(lib().li_append_absorb(x.data_ptr(), _dtype_code(x), n_tok, _ptr(rope_theta), r_R,
                                  seq_idx.data_ptr(), pos.data_ptr(), cache.struct(),
                                  q.data_ptr(), _dtype_code(q), L, n_q, H, d_I, Dt.data_ptr(),
                                  stride, _ptr(b), no, q_tilde.data_ptr(), _ptr(beta),
                                  _stream()))


def score(q_tilde: torch.Tensor, w: torch.Tensor, beta: Optional[torch.Tensor],
          q_seq: torch.Tensor, q_len: torch.Tensor, max_len: int, cache: Cache,
          scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(q_tilde, "q_tilde", (torch.float32, torch.bfloat16))
    _need(w, "w", torch.float32)
    _need(q_seq, "q_seq", torch.int32)
    _need(q_len, "q_len", torch.int32)
    if beta is not None:
        _need(beta, "beta", torch.float32)
    n_q, H, _ = q_tilde.shape
    _numel(w, n_q * H, "w")
    if beta is not None:
        _numel(beta, n_q * H, "beta")
    _numel(q_seq, n_q, "q_seq")
    _numel(q_len, n_q, "q_len")
    if scores is None:
        scores = torch.empty((n_q, max(1, max_len)), dtype=torch.float32, device=q_tilde.device)
    _need(scores, "scores", torch.float32)
    if scores.dim() != 2 or scores.shape[0] < n_q or scores.shape[1] < max_len:
        raise ValueError(f"scores must be [>= {n_q}, >= {max_len}]")
    _check(lib().li_score(q_tilde.data_ptr(), _dtype_code(q_tilde), w.data_ptr(), _ptr(beta), n_q,
                          H, q_seq.data_ptr(), q_len.data_ptr(), max_len, cache.struct(),
                          scores.data_ptr(), scores.shape[1], _stream()))
    return scores


def prepared_score(q_tilde: torch.Tensor, w: torch.Tensor, beta: Optional[torch.Tensor],
                   q_seq: torch.Tensor, q_len: torch.Tensor, max_len: int, cache: Cache,
                   scores: torch.Tensor):
    """A zero-argument callable that enqueues li_score on the current stream
    with every argument marshalled once (for tight decode loops)."""
    _need(q_tilde, "q_tilde", (torch.float32, torch.bfloat16))
    _need(scores, "scores", torch.float32)
    n_q, H, _ = q_tilde.shape
    fn = lib().li_score
    args = (q_tilde.data_ptr(), _dtype_code(q_tilde), w.data_ptr(), _ptr(beta), n_q, H,
            q_seq.data_ptr(), q_len.data_ptr(), max_len, cache.struct(), scores.data_ptr(),
            scores.shape[1])

    def call():
        _check(fn(*args, _stream()))
    return call


def topk(scores: torch.Tensor, valid_len: torch.Tensor, max_len: int, k: int,
         out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None,
         ws: Optional[torch.Tensor] = None, want_val: bool = False):
    _need(scores, "scores", torch.float32)
    _need(valid_len, "valid_len", torch.int32)
    n_rows = scores.shape[0]
    _numel(valid_len, n_rows, "valid_len")
    if out_idx is None:
        out_idx = torch.empty((n_rows, k), dtype=torch.int32, device=scores.device)
    if out_val is None and want_val:
        out_val = torch.empty((n_rows, k), dtype=torch.float32, device=scores.device)
    _need(out_idx, "out_idx", torch.int32)
    _numel(out_idx, n_rows * k, "out_idx")
    if out_val is not None:
        _need(out_val, "out_val", torch.float32)
        _numel(out_val, n_rows * k, "out_val")
    need = lib().li_topk_workspace_bytes(n_rows, max_len, k)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    if ws is not None:
        _need(ws, "ws")
    _check(lib().li_topk(scores.data_ptr(), scores.shape[1], n_rows, valid_len.data_ptr(), max_len,
                         k, out_idx.data_ptr(), _ptr(out_val), _ptr(ws),
                         0 if ws is None else ws.numel(), _stream()))
    return (out_idx, out_val) if want_val else out_idx


def hs_anchor_workspace(n_rows: int, max_len: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace for li_hs_anchor_select: zeroed once here, reusable
    by later calls of any size it covers (one call at a time)."""
    return torch.zeros(lib().li_hs_anchor_workspace_bytes(n_rows, max_len), dtype=torch.uint8,
                       device=device)


def hs_anchor_select(scores: torch.Tensor, valid_len: torch.Tensor, max_len: int, B: int, k: int,
                     cand: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, want_sel: bool = True):
    """The anchor's candidate set (top-B) and own selection (top-k) in one pass."""
    _need(scores, "scores", torch.float32)
    _need(valid_len, "valid_len", torch.int32)
    n_rows = scores.shape[0]
    _numel(valid_len, n_rows, "valid_len")
    if cand is None:
        cand = torch.empty((n_rows, B), dtype=torch.int32, device=scores.device)
    if sel is None and want_sel:
        sel = torch.empty((n_rows, k), dtype=torch.int32, device=scores.device)
    _need(cand, "cand", torch.int32)
    _numel(cand, n_rows * B, "cand")
    if sel is not None:
        _need(sel, "sel", torch.int32)
        _numel(sel, n_rows * k, "sel")
    if ws is None:
        ws = hs_anchor_workspace(n_rows, max_len, scores.device)
    _need(ws, "ws")
    _check(lib().li_hs_anchor_select(scores.data_ptr(), scores.shape[1], n_rows,
                                     valid_len.data_ptr(), max_len, B, cand.data_ptr(), k,
                                     _ptr(sel), ws.data_ptr(), ws.numel(), _stream()))
    return cand, sel


def hs_anchor(q_tilde: torch.Tensor, w: torch.Tensor, beta: Optional[torch.Tensor],
              q_seq: torch.Tensor, q_len: torch.Tensor, max_len: int, cache: Cache, B: int, k: int,
              scores: Optional[torch.Tensor] = None, cand: Optional[torch.Tensor] = None,
              sel: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
              want_sel: bool = True, scan_events=None):
    """The anchor's scores of every position and its candidate set (top-B) and
    own selection (top-k), in one call.  scan_events: None, or two raw
    hipEvent_t handles recorded around the scoring launch.  Returns
    (scores, cand, sel)."""
    _need(q_tilde, "q_tilde", (torch.float32, torch.bfloat16))
    _need(w, "w", torch.float32)
    _need(q_seq, "q_seq", torch.int32)
    _need(q_len, "q_len", torch.int32)
    if beta is not None:
        _need(beta, "beta", torch.float32)
    n_q, H, _ = q_tilde.shape
    dev = q_tilde.device
    _numel(w, n_q * H, "w")
    if beta is not None:
        _numel(beta, n_q * H, "beta")
    _numel(q_seq, n_q, "q_seq")
    _numel(q_len, n_q, "q_len")
    if scores is None:
        scores = torch.empty((n_q, max(1, max_len)), dtype=torch.float32, device=dev)
    _need(scores, "scores", torch.float32)
    if scores.dim() != 2 or scores.shape[0] < n_q or scores.shape[1] < max_len:
        raise ValueError(f"scores must be [>= {n_q}, >= {max_len}]")
    if cand is None:
        cand = torch.empty((n_q, B), dtype=torch.int32, device=dev)
    if sel is None and want_sel:
        sel = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    _need(cand, "cand", torch.int32)
    _numel(cand, n_q * B, "cand")
    if sel is not None:
        _need(sel, "sel", torch.int32)
        _numel(sel, n_q * k, "sel")
    if ws is None:
        ws = hs_anchor_workspace(n_q, max_len, dev)
    _need(ws, "ws")
    evs = None
    if scan_events is not None:
        evs = (ctypes.c_void_p * 2)(*[e.value if isinstance(e, ctypes.c_void_p) else int(e)
                                      for e in scan_events])
    _check(lib().li_hs_anchor(q_tilde.data_ptr(), _dtype_code(q_tilde), w.data_ptr(), _ptr(beta),
                              n_q, H, q_seq.data_ptr(), q_len.data_ptr(), max_len, cache.struct(),
                              scores.data_ptr(), scores.shape[1], B, cand.data_ptr(), k, _ptr(sel),
                              ws.data_ptr(), ws.numel(), evs, _stream()))
    return scores, cand, sel


def _events(scan_events):
    if scan_events is None:
        return None
    return (ctypes.c_void_p * 2)(*[e.value if isinstance(e, ctypes.c_void_p) else int(e)
                                  for e in scan_events])


def score_topk(q_tilde: torch.Tensor, w: torch.Tensor, beta: Optional[torch.Tensor],
               q_seq: torch.Tensor, q_len: torch.Tensor, max_len: int, cache: Cache, k: int,
               scores: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, scan_events=None):
    """One layer's full-scan step: scores of every position and each query's
    top-k, in one call.  ws: a workspace from hs_anchor_workspace (zeroed
    once, reusable).  Returns (scores, out_idx)."""
    _need(q_tilde, "q_tilde", (torch.float32, torch.bfloat16))
    _need(w, "w", torch.float32)
    _need(q_seq, "q_seq", torch.int32)
    _need(q_len, "q_len", torch.int32)
    if beta is not None:
        _need(beta, "beta", torch.float32)
        _numel(beta, q_tilde.shape[0] * q_tilde.shape[1], "beta")
    n_q, H, _ = q_tilde.shape
    dev = q_tilde.device
    _numel(w, n_q * H, "w")
    _numel(q_seq, n_q, "q_seq")
    _numel(q_len, n_q, "q_len")
    if scores is None:
        scores = torch.empty((n_q, max(1, max_len)), dtype=torch.float32, device=dev)
    _need(scores, "scores", torch.float32)
    if scores.dim() != 2 or scores.shape[0] < n_q or scores.shape[1] < max_len:
        raise ValueError(f"scores must be [>= {n_q}, >= {max_len}]")
    if out_idx is None:
        out_idx = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32)
    _numel(out_idx, n_q * k, "out_idx")
    if ws is None:
        ws = hs_anchor_workspace(n_q, max_len, dev)
    _need(ws, "ws")
    _check(lib().li_score_topk(q_tilde.data_ptr(), _dtype_code(q_tilde), w.data_ptr(), _ptr(beta),
                               n_q, H, q_seq.data_ptr(), q_len.data_ptr(), max_len, cache.struct(),
                               scores.data_ptr(), scores.shape[1], k, out_idx.data_ptr(),
                               ws.data_ptr(), ws.numel(), _events(scan_events), _stream()))
    return scores, out_idx


def hs_workspace(n_q: int, B: int, k: int, device="cuda", n_f: int = 1) -> torch.Tensor:
    return torch.empty(lib().li_hs_workspace_bytes(n_f, n_q, B, k), dtype=torch.uint8,
                       device=device)


def hs_select(cand: torch.Tensor, q_tilde: torch.Tensor, w: torch.Tensor,
              beta: Optional[torch.Tensor], q_seq: torch.Tensor, cache: Cache, k: int,
              out_idx: Optional[torch.Tensor] = None, cand_scores: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None, want_scores: bool = False,
              noalloc: bool = False):
    """One follower: q_tilde [n_q, H, r], w/beta [n_q, H] -> out_idx [n_q, k].
    n_f followers sharing the candidates: q_tilde [n_f, n_q, H, r], w/beta
    [n_f, n_q, H] -> out_idx [n_f, n_q, k] (cand_scores likewise).
    noalloc: call li_hs_select_noalloc (the library's own fixed workspace;
    ws is ignored; pass out_idx, and cand_scores if wanted, to allocate
    nothing here either)."""
    _need(cand, "cand", torch.int32)
    _need(q_tilde, "q_tilde", (torch.float32, torch.bfloat16))
    _need(w, "w", torch.float32)
    _need(q_seq, "q_seq", torch.int32)
    if beta is not None:
        _need(beta, "beta", torch.float32)
    n_q, B = cand.shape
    layered = q_tilde.dim() == 4
    n_f = q_tilde.shape[0] if layered else 1
    H = q_tilde.shape[-2]
    if q_tilde.shape[-3] != n_q or q_tilde.shape[-1] != cache.r:
        raise ValueError(f"q_tilde must be [{n_f}, {n_q}, H, {cache.r}] to match cand and the cache")
    _numel(w, n_f * n_q * H, "w")
    if beta is not None:
        _numel(beta, n_f * n_q * H, "beta")
    _numel(q_seq, n_q, "q_seq")
    lead = (n_f,) if layered else ()
    if out_idx is None:
        out_idx = torch.empty(lead + (n_q, k), dtype=torch.int32, device=cand.device)
    if cand_scores is None and want_scores:
        cand_scores = torch.empty(lead + (n_q, B), dtype=torch.float32, device=cand.device)
    _need(out_idx, "out_idx", torch.int32)
    _numel(out_idx, n_f * n_q * k, "out_idx")
    if cand_scores is not None:
        _need(cand_scores, "cand_scores", torch.float32)
        _numel(cand_scores, n_f * n_q * B, "cand_scores")
    if noalloc:
        _check(lib().li_hs_select_noalloc(cand.data_ptr(), B, n_f, q_tilde.data_ptr(),
                                          _dtype_code(q_tilde), w.data_ptr(), _ptr(beta), n_q, H,
                                          q_seq.data_ptr(), cache.struct(), k, out_idx.data_ptr(),
                                          _ptr(cand_scores), _stream()))
        return (out_idx, cand_scores) if want_scores else out_idx
    if ws is None:
        ws = hs_workspace(n_q, B, k, cand.device, n_f=n_f)
    _need(ws, "ws")
    _check(lib().li_hs_select(cand.data_ptr(), B, n_f, q_tilde.data_ptr(), _dtype_code(q_tilde),
                              w.data_ptr(), _ptr(beta), n_q, H, q_seq.data_ptr(), cache.struct(),
                              k, out_idx.data_ptr(), _ptr(cand_scores), ws.data_ptr(), ws.numel(),
                              _stream()))
    return (out_idx, cand_scores) if want_scores else out_idx


def calib_gram(X: torch.Tensor, Y: Optional[torch.Tensor] = None, G_xx=None, G_xy=None,
               x_sum=None, y_sum=None, accumulate: bool = False):
    """Normal equations of the calibration: (X^T X, X^T Y, X^T 1, Y^T 1) over
    the rows of X [n, d] and Y [n, e] (fp32 or bf16 device tensors), written
    or, with accumulate, added to the given outputs."""
    _need(X, "X", (torch.float32, torch.bfloat16))
    n, d = X.shape
    dev = X.device
    if Y is not None:
        _need(Y, "Y", (torch.float32, torch.bfloat16))
        if Y.shape[0] != n:
            raise ValueError("X and Y must have the same rows")
    e = Y.shape[1] if Y is not None else 1
    mk = lambda shape: torch.zeros(shape, dtype=torch.float32, device=dev)  # noqa: E731
    G_xx = mk((d, d)) if G_xx is None else G_xx
    x_sum = mk((d,)) if x_sum is None else x_sum
    if Y is not None:
        G_xy = mk((d, e)) if G_xy is None else G_xy
        y_sum = mk((e,)) if y_sum is None else y_sum
    for t, nm, cnt in ((G_xx, "G_xx", d * d), (G_xy, "G_xy", d * e), (x_sum, "x_sum", d),
                       (y_sum, "y_sum", e)):
        if t is not None:
            _need(t, nm, torch.float32)
            _numel(t, cnt, nm)
    _check(lib().li_calib_gram(X.data_ptr(), _dtype_code(X), n, d, _ptr(Y),
                               _dtype_code(Y) if Y is not None else LI_FP32, e, G_xx.data_ptr(),
                               _ptr(G_xy), _ptr(x_sum), _ptr(y_sum), int(accumulate), _stream()))
    return G_xx, G_xy, x_sum, y_sum
