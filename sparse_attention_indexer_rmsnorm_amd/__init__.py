"""DSA indexer hot path on MI355X: paged key store, scoring and top-k behind a C ABI.

Thin ctypes binding over ``libdsa_indexer.so`` (built from ``csrc/`` for gfx950 by
``build.py``; the C ABI is ``include/dsa_indexer.h``).  Functions here only check tensor
dtypes/devices/shapes and pass raw device pointers and torch's current HIP stream; every step of
the computation runs in the HIP kernels.  There is no fallback: if the library is not built, or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HEAD_DIM = 128
N_HEADS = 64
PAGE_KEYS = 64
COMPRESS_RATIO = 4
MAX_TOPK = 2048
FP8 = 0      # IDX_KV_FP8_E4M3
BF16 = 1     # IDX_KV_BF16
FP4 = 2      # IDX_KV_FP4_E2M1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_indexer.so")
_lib = None

_p, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t

# (name, restype, argtypes) of every symbol include/dsa_indexer.h declares
SIGNATURES = [
    ("idx_abi_version", ctypes.c_int, []),
    ("idx_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("idx_page_bytes", _sz, [ctypes.c_int]),
    ("idx_store_keys", ctypes.c_int,
     [_p, _p, ctypes.c_float, _p, _p, _i64, _p, _i32, _i32, ctypes.c_int, _p, _i64, _p]),
    ("idx_store_keys_rotated", ctypes.c_int,
     [_p, _p, ctypes.c_float, _p, _p, _i64, _p, _i32, _i32, ctypes.c_int, _p, _i64, _p]),
    ("idx_rotate_q", ctypes.c_int, [_p, _p, _i64, _p]),
    ("idx_logits_topk_workspace_size", _sz, [_i64, _i32, _i32, _i32]),
    ("idx_logits_topk_min_workspace", _sz, [_i32, _i32, _i32]),
    ("idx_logits_topk_plan", ctypes.c_int, [_i64, _i32, _i32, _i32, _sz, _p, _p]),
    ("idx_logits_topk", ctypes.c_int,
     [_p, _p, _p, ctypes.c_int, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _i32, _p, _p, _p, _sz,
      _p]),
    ("idx_logits_topk_noalloc", ctypes.c_int,
     [_p, _p, _p, ctypes.c_int, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _i32, _p, _p, _p]),
    ("idx_logits_topk_noalloc_scratch_bytes", _sz, []),
    ("idx_logits_topk_timed", ctypes.c_int,
     [_p, _p, _p, ctypes.c_int, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _i32, _p, _p, _p, _sz,
      _p, _p, _p]),
    ("idx_logits_dense", ctypes.c_int,
     [_p, _p, _p, ctypes.c_int, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _p, _i32, _p]),
    ("idx_quantize_q", ctypes.c_int, [_p, _p, _p, _i64, _p]),
    ("idx_logits_topk_fp8q", ctypes.c_int,
     [_p, _p, _p, _p, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _i32, _p, _p, _p, _sz, _p]),
    ("idx_logits_topk_fp8q_timed", ctypes.c_int,
     [_p, _p, _p, _p, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _i32, _p, _p, _p, _sz, _p, _p,
      _p]),
    ("idx_logits_dense_fp8q", ctypes.c_int,
     [_p, _p, _p, _p, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _p, _i32, _p]),
    ("idx_topk_rows_workspace_size", _sz, [_i64, _i64, _i32]),
    ("idx_topk_rows", ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _p, _p, _sz, _p]),
    ("idx_sparse_attn_workspace_size", _sz, [_i64, _i32, _i32]),
    ("idx_sparse_attn", ctypes.c_int,
     [_p, _p, _i64, _p, _i32, _i32, _p, _p, _i64, _i32, _i32, ctypes.c_float, _p, _p, _p, _sz,
      _p]),
]


class IndexerError(RuntimeError):
    pass


def lib():
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m sparse_attention_indexer_rmsnorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().idx_status_string(status).decode()
        raise IndexerError(f"{what}: {msg} (status {status})")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def page_bytes(dtype: int) -> int:
    return int(lib().idx_page_bytes(int(dtype)))


def new_cache(n_pages: int, dtype: int, device="cuda", fill: int = 0xA5) -> torch.Tensor:
    """A flat byte pool of n_pages cache pages (pre-filled with a sentinel byte)."""
    return torch.full((n_pages * page_bytes(dtype),), fill, dtype=torch.uint8, device=device)


def workspace_size(n_q: int, n_seq: int, max_pages: int, k: int) -> int:
    return int(lib().idx_logits_topk_workspace_size(n_q, n_seq, max_pages, k))


def min_workspace(n_seq: int, max_pages: int, k: int) -> int:
    return int(lib().idx_logits_topk_min_workspace(n_seq, max_pages, k))


def topk_plan(n_q: int, n_seq: int, max_pages: int, k: int,
              workspace_bytes: int) -> Tuple[int, int]:
    """(query rows per chunk, most workspace bytes any chunk touches) for a workspace budget.
    Host only; raises IndexerError when not even one row fits."""
    rows = ctypes.c_int64(0)
    most = ctypes.c_size_t(0)
    _check(lib().idx_logits_topk_plan(n_q, n_seq, max_pages, k, workspace_bytes,
                                      ctypes.byref(rows), ctypes.byref(most)),
           "idx_logits_topk_plan")
    return int(rows.value), int(most.value)


def store_keys(x: torch.Tensor, gamma: torch.Tensor, key_idx: torch.Tensor,
               page_table: torch.Tensor, kcache: torch.Tensor, dtype: int, *, eps: float = 1e-6,
               key_seq: Optional[torch.Tensor] = None, rotate: bool = False,
               stream=None) -> None:
    """S1: RMSNorm + RoPE + quantise/store rows of x [n, 128] fp32 into the paged cache.
    ``rotate``: the rotated store (Hadamard transform after RoPE); q then needs rotate_q."""
    n = x.shape[0] if x.dim() == 2 else -1
    if x.dim() != 2 or x.shape[1] != HEAD_DIM:
        raise ValueError("x must be [n_keys, 128]")
    if page_table.dim() != 2:
        raise ValueError("page_table must be [n_seq, max_pages]")
    n_seq, max_pages = page_table.shape
    pb = page_bytes(dtype)
    if pb == 0:
        raise ValueError(f"unknown dtype {dtype}")
    n_pool = kcache.numel() // pb
    fn = lib().idx_store_keys_rotated if rotate else lib().idx_store_keys
    st = fn(
        _dev(x, "x", torch.float32), _dev(gamma, "gamma", torch.float32, HEAD_DIM), float(eps),
        _dev(key_idx, "key_idx", torch.int32, n), _dev(key_seq, "key_seq", torch.int32, n), n,
        _dev(page_table, "page_table", torch.int32), n_seq, max_pages, int(dtype),
        _dev(kcache, "kcache", torch.uint8), n_pool, _stream(stream))
    _check(st, "idx_store_keys_rotated" if rotate else "idx_store_keys")


def rotate_q(q: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q (bf16, last dim 128) for a rotated cache; ``out`` may be q itself."""
    if q.shape[-1] != HEAD_DIM:
        raise ValueError("the last dim of q must be 128")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    n_vec = q.numel() // HEAD_DIM
    st = lib().idx_rotate_q(_dev(q, "q", torch.bfloat16), _dev(out, "out", torch.bfloat16),
                            n_vec, _stream(stream))
    _check(st, "idx_rotate_q")
    return out


def _logits_args(q, w, kcache, dtype, page_table, seq_lens, cu_q):
    if q.dim() != 3 or q.shape[1:] != (N_HEADS, HEAD_DIM):
        raise ValueError("q must be [n_q, 64, 128]")
    n_q = q.shape[0]
    n_seq, max_pages = page_table.shape
    pb = page_bytes(dtype)
    if pb == 0:
        raise ValueError(f"unknown dtype {dtype}")
    return (_dev(q, "q", torch.bfloat16), _dev(w, "w", torch.float32, n_q * N_HEADS),
            _dev(kcache, "kcache", torch.uint8), int(dtype), kcache.numel() // pb,
            _dev(page_table, "page_table", torch.int32), n_seq, max_pages,
            _dev(seq_lens, "seq_lens", torch.int32, n_seq),
            _dev(cu_q, "cu_q", torch.int32, n_seq + 1), n_q, N_HEADS)


def logits_topk(q: torch.Tensor, w: torch.Tensor, kcache: torch.Tensor, dtype: int,
                page_table: torch.Tensor, seq_lens: torch.Tensor, cu_q: torch.Tensor, k: int, *,
                out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None,
                want_values: bool = False, workspace: Optional[torch.Tensor] = None,
                events=None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """S2+S3: top-k key indices (and optionally logits) per query row, in an unspecified order
    within the row."""
    args = _logits_args(q, w, kcache, dtype, page_table, seq_lens, cu_q)
    n_q = q.shape[0]
    n_seq, max_pages = page_table.shape
    if out_idx is None:
        out_idx = torch.empty((n_q, k), dtype=torch.int32, device=q.device)
    if out_val is None and want_values:
        out_val = torch.empty((n_q, k), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(workspace_size(n_q, n_seq, max_pages, k), dtype=torch.uint8,
                                device=q.device)
    common = args + (int(k), _dev(out_idx, "out_idx", torch.int32, n_q * k),
                     _dev(out_val, "out_val", torch.float32, n_q * k),
                     _dev(workspace, "workspace", torch.uint8), workspace.numel())
    if events is None:
        st = lib().idx_logits_topk(*common, _stream(stream))
    else:
        ev0, ev1 = events
        st = lib().idx_logits_topk_timed(*common, ctypes.c_void_p(ev0.cuda_event),
                                         ctypes.c_void_p(ev1.cuda_event), _stream(stream))
    _check(st, "idx_logits_topk")
    return out_idx, out_val


def quantize_q(q: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """q (bf16, [..., 128]) -> (e4m3 codes uint8 [..., 128], fp32 scales [...]) per 128-dim vector,
    for fp8 x fp8 scoring."""
    if q.shape[-1] != HEAD_DIM:
        raise ValueError("the last dim of q must be 128")
    codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    scales = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    n_vec = q.numel() // HEAD_DIM
    st = lib().idx_quantize_q(_dev(q, "q", torch.bfloat16), _dev(codes, "q_codes", torch.uint8),
                              _dev(scales, "q_scales", torch.float32, n_vec), n_vec,
                              _stream(stream))
    _check(st, "idx_quantize_q")
    return codes, scales


def _fp8q_args(q_codes, q_scales, w, kcache, page_table, seq_lens, cu_q):
    if q_codes.dim() != 3 or q_codes.shape[1:] != (N_HEADS, HEAD_DIM):
        raise ValueError("q_codes must be [n_q, 64, 128]")
    n_q = q_codes.shape[0]
    n_seq, max_pages = page_table.shape
    return (_dev(q_codes, "q_codes", torch.uint8), _dev(q_scales, "q_scales", torch.float32,
                                                         n_q * N_HEADS),
            _dev(w, "w", torch.float32, n_q * N_HEADS), _dev(kcache, "kcache", torch.uint8),
            kcache.numel() // page_bytes(0), _dev(page_table, "page_table", torch.int32), n_seq,
            max_pages, _dev(seq_lens, "seq_lens", torch.int32, n_seq),
            _dev(cu_q, "cu_q", torch.int32, n_seq + 1), n_q, N_HEADS)


def logits_topk_fp8q(q_codes: torch.Tensor, q_scales: torch.Tensor, w: torch.Tensor,
                     kcache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                     cu_q: torch.Tensor, k: int, *, out_idx: Optional[torch.Tensor] = None,
                     out_val: Optional[torch.Tensor] = None, want_values: bool = False,
                     workspace: Optional[torch.Tensor] = None, events=None,
                     stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """S2+S3 with fp8 q (from quantize_q) against an fp8 cache."""
    args = _fp8q_args(q_codes, q_scales, w, kcache, page_table, seq_lens, cu_q)
    n_q = q_codes.shape[0]
    n_seq, max_pages = page_table.shape
    if out_idx is None:
        out_idx = torch.empty((n_q, k), dtype=torch.int32, device=q_codes.device)
    if out_val is None and want_values:
        out_val = torch.empty((n_q, k), dtype=torch.float32, device=q_codes.device)
    if workspace is None:
        workspace = torch.empty(workspace_size(n_q, n_seq, max_pages, k), dtype=torch.uint8,
                                device=q_codes.device)
    common = args + (int(k), _dev(out_idx, "out_idx", torch.int32, n_q * k),
                     _dev(out_val, "out_val", torch.float32, n_q * k),
                     _dev(workspace, "workspace", torch.uint8), workspace.numel())
    if events is None:
        st = lib().idx_logits_topk_fp8q(*common, _stream(stream))
    else:
        ev0, ev1 = events
        st = lib().idx_logits_topk_fp8q_timed(*common, ctypes.c_void_p(ev0.cuda_event),
                                              ctypes.c_void_p(ev1.cuda_event), _stream(stream))
    _check(st, "idx_logits_topk_fp8q")
    return out_idx, out_val


def logits_dense_fp8q(q_codes: torch.Tensor, q_scales: torch.Tensor, w: torch.Tensor,
                      kcache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                      cu_q: torch.Tensor, max_keys: int, *, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """S2 only with fp8 q, for checking: logits [n_q, max_keys], -inf where not visible."""
    args = _fp8q_args(q_codes, q_scales, w, kcache, page_table, seq_lens, cu_q)
    n_q = q_codes.shape[0]
    if out is None:
        out = torch.empty((n_q, max_keys), dtype=torch.float32, device=q_codes.device)
    st = lib().idx_logits_dense_fp8q(*args, _dev(out, "out", torch.float32, n_q * max_keys),
                                     int(max_keys), _stream(stream))
    _check(st, "idx_logits_dense_fp8q")
    return out


def logits_dense(q: torch.Tensor, w: torch.Tensor, kcache: torch.Tensor, dtype: int,
                 page_table: torch.Tensor, seq_lens: torch.Tensor, cu_q: torch.Tensor,
                 max_keys: int, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """S2 only (for checking): head-reduced logits [n_q, max_keys], -inf where not visible."""
    args = _logits_args(q, w, kcache, dtype, page_table, seq_lens, cu_q)
    n_q = q.shape[0]
    if out is None:
        out = torch.empty((n_q, max_keys), dtype=torch.float32, device=q.device)
    st = lib().idx_logits_dense(*args, _dev(out, "out", torch.float32, n_q * max_keys),
                                int(max_keys), _stream(stream))
    _check(st, "idx_logits_dense")
    return out


def topk_rows(scores: torch.Tensor, k: int, row_len: Optional[torch.Tensor] = None, *,
              want_values: bool = True, stream=None):
    """S3 only: top-k column indices of each row of scores [n_rows, row_stride] fp32."""
    if scores.dim() != 2:
        raise ValueError("scores must be 2-D")
    n_rows, stride = scores.shape
    out_idx = torch.empty((n_rows, k), dtype=torch.int32, device=scores.device)
    out_val = torch.empty((n_rows, k), dtype=torch.float32, device=scores.device) \
        if want_values else None
    ws_bytes = int(lib().idx_topk_rows_workspace_size(n_rows, stride, int(k)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device) if ws_bytes else None
    st = lib().idx_topk_rows(_dev(scores, "scores", torch.float32), n_rows, stride,
                             _dev(row_len, "row_len", torch.int32, n_rows), int(k),
                             _dev(out_idx, "out_idx", torch.int32),
                             _dev(out_val, "out_val", torch.float32), _dev(ws, "workspace"),
                             ws_bytes, _stream(stream))
    _check(st, "idx_topk_rows")
    return out_idx, out_val


LATENT_DIM = 512


def sparse_attn_workspace_size(n_q: int, n_heads: int, k: int) -> int:
    return int(lib().idx_sparse_attn_workspace_size(int(n_q), int(n_heads), int(k)))


def sparse_attn(q: torch.Tensor, kv: torch.Tensor, kv_slot: torch.Tensor, cu_q: torch.Tensor,
                idx: torch.Tensor, softmax_scale: float, *, want_lse: bool = True,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None):
    """Sparse attention of q [n_q, n_heads, 512] bf16 over the latents kv [n_slots, 512] bf16 of
    the keys listed in idx [n_q, k] int32 (kv_slot [n_seq, max_keys] int32 maps a sequence's key
    to its kv row).  Returns (out [n_q, n_heads, 512] bf16, lse [n_q, n_heads] fp32 or None)."""
    if q.dim() != 3 or q.shape[2] != LATENT_DIM:
        raise ValueError("q must be [n_q, n_heads, 512]")
    if kv.dim() != 2 or kv.shape[1] != LATENT_DIM:
        raise ValueError("kv must be [n_slots, 512]")
    if idx.dim() != 2 or idx.shape[0] != q.shape[0]:
        raise ValueError("idx must be [n_q, k]")
    if kv_slot.dim() != 2:
        raise ValueError("kv_slot must be [n_seq, max_keys]")
    n_q, n_heads, _ = q.shape
    n_seq, max_keys = kv_slot.shape
    k = idx.shape[1]
    if out is None:
        out = torch.empty((n_q, n_heads, LATENT_DIM), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((n_q, n_heads), dtype=torch.float32, device=q.device) if want_lse else None
    ws_bytes = sparse_attn_workspace_size(n_q, n_heads, k)
    if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib().idx_sparse_attn(_dev(q, "q", torch.bfloat16), _dev(kv, "kv", torch.bfloat16),
                               kv.shape[0], _dev(kv_slot, "kv_slot", torch.int32), n_seq, max_keys,
                               _dev(cu_q, "cu_q", torch.int32, n_seq + 1),
                               _dev(idx, "idx", torch.int32), n_q, n_heads, k,
                               float(softmax_scale),
                               _dev(out, "out", torch.bfloat16, n_q * n_heads * LATENT_DIM),
                               _dev(lse, "lse", torch.float32), _dev(workspace, "workspace"),
                               ws_bytes if workspace is None else workspace.numel(),
                               _stream(stream))
    _check(st, "idx_sparse_attn")
    return out, lse
