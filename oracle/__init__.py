"""CPU oracle of the DSA indexer hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product path (``sparse_attention_indexer_rmsnorm_amd``) never does, and this
package never imports the product path: the two share only the seeded inputs.

The arithmetic lives in ``oracle.c`` (plain fp64 loops; see its header for the passages of the four
DSA-indexer blog pages each step follows and for the readings taken where they are silent).  This
module is ctypes marshalling plus two small harness helpers (needle vectors and recall), which use
the C routines for all of the indexer's arithmetic.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against closed forms, library
routines on special cases, invariants and brute force; ``tests/test_oracle_mutations.py`` plants
mistakes in the C code and checks that some pin fails for each.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

FP8, BF16, FP4 = 0, 1, 2
D, H, PAGE, RATIO = 128, 64, 64, 4

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b  # noqa: PLC0415
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_encode.argtypes = [ctypes.c_float]
        L.oracle_page_bytes.restype = _i64
        L.oracle_page_bytes.argtypes = [ctypes.c_int]
        L.oracle_n_visible.restype = _i64
        L.oracle_n_visible.argtypes = [_i64, _i32]
        L.oracle_rope_inv_freq.restype = None
        L.oracle_rope_inv_freq.argtypes = [_p]
        L.oracle_store_keys.restype = _i64
        L.oracle_store_keys.argtypes = [_p, _p, ctypes.c_float, _p, _p, _i64, _p, _i32, _i32,
                                        ctypes.c_int, _p, _i64, _p, ctypes.c_int]
        L.oracle_logits_fp8q.restype = None
        L.oracle_logits_fp8q.argtypes = [_p, _p, _p, _p, ctypes.c_int, _i64, _p, _i32, _i32, _p,
                                         _p, _p, _i64, _i64, _p, _p]
        L.oracle_quantize_q.restype = None
        L.oracle_quantize_q.argtypes = [_p, _i64, _p, _p]
        L.oracle_hadamard_scale.restype = ctypes.c_double
        L.oracle_hadamard_scale.argtypes = []
        L.oracle_hadamard128.restype = None
        L.oracle_hadamard128.argtypes = [_p]
        L.oracle_rotate_q.restype = None
        L.oracle_rotate_q.argtypes = [_p, _i64, _p]
        L.oracle_logits.restype = None
        L.oracle_logits.argtypes = [_p, _p, _p, ctypes.c_int, _i64, _p, _i32, _i32, _p, _p, _p,
                                    _i64, _i64, _p, _i64, _p, _p]
        L.oracle_topk.restype = None
        L.oracle_topk.argtypes = [_p, _i64, _i64, _p, _i32, _p, _p]
        L.oracle_plant_keys.restype = None
        L.oracle_plant_keys.argtypes = [_p, _p, _i64, _p, _p]
        L.oracle_sparse_attn.argtypes = [_p, _p, _i64, _p, _i32, _i32, _p, _p, _i32, _i32,
                                         ctypes.c_double, _p, _i64, _p, _p]
        L.oracle_sparse_attn.restype = None
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_mutation.restype = None
        L.oracle_set_mutation.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_mutation(m: int) -> None:
    lib().oracle_set_mutation(int(m))


# ---- number formats -------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_e4m3_decode(int(c)) for c in np.asarray(codes).ravel()])


def e4m3_encode(v) -> np.ndarray:
    L = lib()
    v = np.asarray(v, dtype=np.float32).ravel()
    return np.array([L.oracle_e4m3_encode(float(x)) for x in v], dtype=np.uint8)


def bf16_encode(v) -> np.ndarray:
    L = lib()
    v = np.asarray(v, dtype=np.float32).ravel()
    return np.array([L.oracle_bf16_encode(float(x)) for x in v], dtype=np.uint16)


def e2m1_decode(codes) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_e2m1_decode(int(c)) for c in np.asarray(codes).ravel()])


def e2m1_encode(v) -> np.ndarray:
    L = lib()
    v = np.asarray(v, dtype=np.float32).ravel()
    return np.array([L.oracle_e2m1_encode(float(x)) for x in v], dtype=np.uint8)


def page_bytes(dtype: int) -> int:
    return int(lib().oracle_page_bytes(dtype))


def n_visible(t: int, max_pages: int) -> int:
    return int(lib().oracle_n_visible(int(t), int(max_pages)))


def rope_inv_freq() -> np.ndarray:
    out = np.zeros(32, np.float32)
    lib().oracle_rope_inv_freq(_ptr(out))
    return out


# ---- S1 ---------------------------------------------------------------------------------------

def new_pool(n_pages: int, dtype: int, fill: int = 0xA5) -> np.ndarray:
    return np.full(n_pages * page_bytes(dtype), fill, dtype=np.uint8)


def hadamard_scale() -> float:
    return float(lib().oracle_hadamard_scale())


def hadamard128(v) -> np.ndarray:
    """The normalised 128-point Walsh-Hadamard transform of each fp64 row of v (a copy)."""
    v = np.array(v, dtype=np.float64, copy=True).reshape(-1, D)
    for row in v:
        lib().oracle_hadamard128(_ptr(row))
    return v


def rotate_q(q_bits) -> np.ndarray:
    """bf16 bit patterns [..., 128] rotated like the keys of the rotated store."""
    q_bits = _c(q_bits, np.uint16)
    out = np.zeros_like(q_bits)
    lib().oracle_rotate_q(_ptr(q_bits), q_bits.size // D, _ptr(out))
    return out


def store_keys(x, gamma, eps, key_idx, key_seq, page_table, dtype, pool, want_k32=False,
               hadamard=False):
    """Store rows of x into ``pool`` (modified in place).  Returns (skipped, k32 or None).
    ``hadamard``: the rotated store (normalised Walsh-Hadamard transform after RoPE)."""
    x = _c(x, np.float32)
    gamma = _c(gamma, np.float32)
    key_idx = _c(key_idx, np.int32)
    key_seq = None if key_seq is None else _c(key_seq, np.int32)
    pt = _c(page_table, np.int32)
    n_seq, max_pages = pt.shape
    n_pool = pool.size // page_bytes(dtype)
    k32 = np.zeros((x.shape[0], D), np.float32) if want_k32 else None
    skipped = lib().oracle_store_keys(_ptr(x), _ptr(gamma), float(eps), _ptr(key_idx),
                                      _ptr(key_seq), x.shape[0], _ptr(pt), n_seq, max_pages,
                                      int(dtype), _ptr(pool), n_pool, _ptr(k32),
                                      1 if hadamard else 0)
    return int(skipped), k32


def store_workload(wl, dtype, pool=None, want_k32=False, mask=None, hadamard=False):
    if pool is None:
        pool = new_pool(wl.n_pages_pool, dtype)
    sel = slice(None) if mask is None else mask
    skipped, k32 = store_keys(wl.x[sel], wl.gamma, wl.eps, wl.key_idx[sel], wl.key_seq[sel],
                              wl.page_table, dtype, pool, want_k32, hadamard)
    return pool, k32


# ---- S2 ---------------------------------------------------------------------------------------

def logits(q_bits, w, pool, dtype, page_table, seq_lens, cu_q, rows=None, row_len=None,
           keys_ref=None, ref_stride=None):
    """fp64 logits of the given query rows; returns (logits [n_rows, row_len], n_vis [n_rows]).

    ``keys_ref`` ([n_seq, ref_stride, 128] fp32) replaces the pool as key source when given."""
    q_bits = _c(q_bits, np.uint16)
    w = _c(w, np.float32)
    pt = _c(page_table, np.int32)
    n_seq, max_pages = pt.shape
    n_q = q_bits.shape[0]
    rows = np.arange(n_q, dtype=np.int64) if rows is None else _c(rows, np.int64)
    row_len = max_pages * PAGE if row_len is None else int(row_len)
    out = np.empty((rows.size, row_len), np.float64)
    nv = np.empty(rows.size, np.int64)
    n_pool = 0 if pool is None else pool.size // page_bytes(dtype)
    kr = None if keys_ref is None else _c(keys_ref, np.float32)
    lib().oracle_logits(_ptr(q_bits), _ptr(w), _ptr(pool), int(dtype), n_pool, _ptr(pt), n_seq,
                        max_pages, _ptr(_c(seq_lens, np.int32)), _ptr(_c(cu_q, np.int32)),
                        _ptr(rows), rows.size, row_len, _ptr(kr),
                        0 if ref_stride is None else int(ref_stride), _ptr(out), _ptr(nv))
    return out, nv


def quantize_q(q_bits):
    """bf16 q [..., 128] -> (e4m3 codes [..., 128] uint8, fp32 scales [...]) per 128-dim vector."""
    q_bits = _c(q_bits, np.uint16)
    codes = np.zeros(q_bits.shape, np.uint8)
    scales = np.zeros(q_bits.shape[:-1], np.float32)
    lib().oracle_quantize_q(_ptr(q_bits), q_bits.size // D, _ptr(codes), _ptr(scales))
    return codes, scales


def logits_fp8q(q_codes, q_scales, w, pool, page_table, seq_lens, cu_q, rows=None,
                row_len=None):
    """fp64 logits with fp8 q (codes [n_q, 64, 128], scales [n_q, 64]) against an fp8 pool."""
    q_codes = _c(q_codes, np.uint8)
    q_scales = _c(q_scales, np.float32)
    w = _c(w, np.float32)
    pt = _c(page_table, np.int32)
    n_seq, max_pages = pt.shape
    n_q = q_codes.shape[0]
    rows = np.arange(n_q, dtype=np.int64) if rows is None else _c(rows, np.int64)
    row_len = max_pages * PAGE if row_len is None else int(row_len)
    out = np.empty((rows.size, row_len), np.float64)
    nv = np.empty(rows.size, np.int64)
    n_pool = pool.size // page_bytes(FP8)
    lib().oracle_logits_fp8q(_ptr(q_codes), _ptr(q_scales), _ptr(w), _ptr(pool), FP8, n_pool,
                             _ptr(pt), n_seq, max_pages, _ptr(_c(seq_lens, np.int32)),
                             _ptr(_c(cu_q, np.int32)), _ptr(rows), rows.size, row_len,
                             _ptr(out), _ptr(nv))
    return out, nv


# ---- S3 ---------------------------------------------------------------------------------------

def topk(scores, k, row_len=None):
    """Top-k of each row of ``scores`` (float64 or float32, compared exactly); ties to lower s.
    Returns (idx int32 [n, k], val float64 [n, k]); short rows are padded with -1 / -inf."""
    s = _c(scores, np.float64)
    n_rows, stride = s.shape
    rl = None if row_len is None else _c(row_len, np.int64)
    idx = np.empty((n_rows, k), np.int32)
    val = np.empty((n_rows, k), np.float64)
    lib().oracle_topk(_ptr(s), n_rows, stride, _ptr(rl), int(k), _ptr(idx), _ptr(val))
    return idx, val


# ---- sparse attention over the selected keys ---------------------------------------------------

def sparse_attn(q_bits, kv_bits, kv_slot, cu_q, idx, scale, rows=None):
    """fp64 sparse attention of the given query rows over their listed keys.

    q_bits [n_q, n_heads, 512] and kv_bits [n_slots, 512] are bf16 bit patterns, kv_slot
    [n_seq, max_keys] int32 maps a sequence's key index to a kv row, idx [n_q, k] int32 lists
    each row's keys (-1 = none).  Returns (out [n_rows, n_heads, 512], lse [n_rows, n_heads])."""
    q_bits = _c(q_bits, np.uint16)
    kv_bits = _c(kv_bits, np.uint16)
    kv_slot = _c(kv_slot, np.int32)
    idx = _c(idx, np.int32)
    n_q, n_heads, dv = q_bits.shape
    assert dv == 512 and kv_bits.shape[1] == 512 and idx.shape[0] == n_q
    n_seq, max_keys = kv_slot.shape
    rows = np.arange(n_q, dtype=np.int64) if rows is None else _c(rows, np.int64)
    out = np.empty((rows.size, n_heads, 512), np.float64)
    lse = np.empty((rows.size, n_heads), np.float64)
    lib().oracle_sparse_attn(_ptr(q_bits), _ptr(kv_bits), kv_bits.shape[0], _ptr(kv_slot), n_seq,
                             max_keys, _ptr(_c(cu_q, np.int32)), _ptr(idx), n_heads,
                             idx.shape[1], float(scale), _ptr(rows), rows.size, _ptr(out),
                             _ptr(lse))
    return out, lse


# ---- needle helpers (harness) -----------------------------------------------------------------

def needle_vectors(wl, construction: str) -> np.ndarray:
    """Key-space needle directions for wl.needles: 3 * unit(direction) + noise, where direction
    is the head-mean of the needle's query ('literal') or the w-weighted head sum ('weighted')."""
    nd = wl.needles
    q = _bf16_to_f64(wl.q_bits[nd["qrow"]])                    # [n, 64, 128]
    if construction == "literal":
        v = q.mean(axis=1)
    elif construction == "weighted":
        v = np.einsum("nh,nhd->nd", wl.w[nd["qrow"]].astype(np.float64), q)
    else:
        raise ValueError(construction)
    v = v / np.linalg.norm(v, axis=1, keepdims=True)
    return 3.0 * v + nd["noise"]


def plant_needles(wl, construction: str) -> np.ndarray:
    """Return a copy of wl.x whose needle rows store keys along the needle vectors."""
    kstar = _c(needle_vectors(wl, construction), np.float64)
    nd = wl.needles
    s = _c(nd["s"], np.int32)
    xo = np.empty((s.size, D), np.float32)
    lib().oracle_plant_keys(_ptr(kstar), _ptr(s), s.size, _ptr(_c(wl.gamma, np.float32)), _ptr(xo))
    x = wl.x.copy()
    x[nd["krow"]] = xo
    return x


def _bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)
