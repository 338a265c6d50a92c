"""The C-ABI library loads, exports every declared symbol, and validates arguments on the host.

No GPU is needed: every call here returns from host-side validation before any HIP call.
"""
import ctypes

import pytest

import sparse_attention_indexer_rmsnorm_amd as ix
from tests.helpers import header_functions

E_OK, E_INVAL, E_UNSUP, E_WS, E_HIP = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    return ix.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 22, names
    for n in names:
        assert hasattr(L, n), f"missing export {n}"
    assert sorted(n for n, _, _ in ix.SIGNATURES) == names


def test_version_and_strings(L):
    assert L.idx_abi_version() == 1
    for s in range(5):
        assert L.idx_status_string(s)
    assert L.idx_status_string(99) == b"unknown status"


def test_page_bytes(L):
    assert L.idx_page_bytes(0) == 8448      # 64 keys x (128 codes + 4 B scale)
    assert L.idx_page_bytes(1) == 16384     # 64 keys x 256 B
    assert L.idx_page_bytes(2) == 4352      # 64 keys x (64 B of 4-bit codes + 4 B scale)
    assert L.idx_page_bytes(3) == 0
    assert L.idx_page_bytes(-1) == 0


def test_workspace_sizes(L):
    # decode batch of 32 queries over 512 pages: visible counts, then per row the keys of its 16
    # scoring workgroups bucketed by histogram bin (32768 (key, index) pairs) and the 16
    # workgroups' histograms and bucket starts (2048 16-bit bins each)
    lists = 256 + 32 * 32768 * 8
    hist = 32 * 16 * 2048 * 2
    assert L.idx_logits_topk_workspace_size(32, 32, 512, 1024) == lists + hist + hist
    # 256 such rows go through the segmented two-pass selection: two candidate buffers of
    # 6 segments x k (index, value) pairs per row
    cand = 2 * (256 * 6 * 1024 * 8 + 256)
    assert L.idx_topk_rows_workspace_size(256, 32768, 1024) == cand
    # long prefill chunk: 8192 queries x 5632 keys fits the 256 MiB cap in one pass, one-pass top-k
    ws = L.idx_logits_topk_workspace_size(8192, 1, 88, 512)
    assert ws == 8192 * 4 + 8192 * 5632 * 4 and ws <= 256 << 20
    # a 128K-token prefill of 8192 queries is chunked to stay under the cap
    big = L.idx_logits_topk_workspace_size(8192, 1, 2048, 512)
    assert big <= 256 << 20 and big >= 131072 * 4
    assert L.idx_logits_topk_min_workspace(1, 88, 512) >= 256 + 5632 * 4
    # never depends on the head count: the per-head tensor is never formed
    assert L.idx_logits_topk_workspace_size(8192, 1, 88, 512) < 8192 * 5632 * 64 * 4 / 50
    # stand-alone selection: one pass needs none; long rows of a small batch need candidates
    assert L.idx_topk_rows_workspace_size(8192, 5632, 512) == 0
    assert L.idx_topk_rows_workspace_size(32, 32768, 1024) == 0     # one workgroup per row
    assert L.idx_topk_rows_workspace_size(32, 40000, 1024) > 0      # longer than a workgroup


def test_chunk_plan_fits_workspace(L):
    """Every query chunk of idx_logits_topk fits the workspace it is given: the planner's row
    bound must cover the segmented selection's candidate buffers, which a batch of more than 128
    long rows needs even where a single row is selected with none, and the histogram selection's
    histograms, bucket starts and bucketed keys (decode-shaped batches)."""
    for max_pages in (1, 16, 97, 128, 192, 256, 384, 512, 640, 2048):  # 64 .. 131072 key columns
        for k in (512, 1024, 2048):
            mins = ix.min_workspace(1, max_pages, k)
            for n_q in (1, 2, 128, 129, 200, 517, 1000, 4096, 8192):
                for n_seq in sorted({1, max(1, n_q // 2), n_q}):
                    rec = ix.workspace_size(n_q, n_seq, max_pages, k)
                    budgets = {rec, mins, mins + 12345, 4 << 20, 8 << 20, 11 << 20, 64 << 20,
                               rec // 3, rec - 1}
                    for b in sorted(budgets):
                        if b < mins:
                            continue
                        rows, most = ix.topk_plan(n_q, n_seq, max_pages, k, b)
                        assert 1 <= rows <= n_q, (max_pages, k, n_q, n_seq, b, rows)
                        assert most <= b, (max_pages, k, n_q, n_seq, b, rows, most)
                    rows, _ = ix.topk_plan(n_q, n_seq, max_pages, k, rec)
                    assert rows == n_q or rec <= (256 << 20) + 4096, (max_pages, k, n_q, rec)
    # the long prefill chunk still runs in one pass within the 256 MiB cap
    rec = ix.workspace_size(8192, 1, 88, 512)
    assert ix.topk_plan(8192, 1, 88, 512, rec)[0] == 8192 and rec <= 256 << 20
    # too small for a single row
    with pytest.raises(ix.IndexerError):
        ix.topk_plan(10, 1, 88, 512, 100)
    assert L.idx_logits_topk_plan(0, 1, 88, 512, 1 << 20, FAKE, FAKE) == E_INVAL


def _store(L, **kw):
    a = dict(x=FAKE, gamma=FAKE, eps=1e-6, key_idx=FAKE, key_seq=None, n=10, pt=FAKE, n_seq=1,
             max_pages=1, dtype=0, kc=FAKE, pool=1)
    a.update(kw)
    return L.idx_store_keys(a["x"], a["gamma"], a["eps"], a["key_idx"], a["key_seq"], a["n"],
                            a["pt"], a["n_seq"], a["max_pages"], a["dtype"], a["kc"], a["pool"],
                            None)


def test_store_validation(L):
    assert _store(L, n=-1) == E_INVAL
    assert _store(L, dtype=5) == E_UNSUP
    assert _store(L, x=None) == E_INVAL
    assert _store(L, kc=None) == E_INVAL
    assert _store(L, pt=None) == E_INVAL
    assert _store(L, eps=-1.0) == E_INVAL
    assert _store(L, eps=float("nan")) == E_INVAL
    assert _store(L, n_seq=-2) == E_INVAL
    assert _store(L, x=ctypes.c_void_p(0x1008)) == E_INVAL               # x, gamma, kcache: 16-byte aligned
    assert _store(L, gamma=ctypes.c_void_p(0x1004)) == E_INVAL
    assert _store(L, kc=ctypes.c_void_p(0x1002)) == E_INVAL
    assert _store(L, n=0, x=None, kc=None) == E_OK        # empty store is a no-op


def _topk(L, fn="idx_logits_topk", **kw):
    a = dict(q=FAKE, w=FAKE, kc=FAKE, dtype=1, pool=4, pt=FAKE, n_seq=1, max_pages=2,
             seq_lens=FAKE, cu_q=FAKE, n_q=3, n_heads=64, k=512, oi=FAKE, ov=None, ws=FAKE,
             ws_bytes=1)
    a.update(kw)
    return getattr(L, fn)(a["q"], a["w"], a["kc"], a["dtype"], a["pool"], a["pt"], a["n_seq"],
                          a["max_pages"], a["seq_lens"], a["cu_q"], a["n_q"], a["n_heads"], a["k"],
                          a["oi"], a["ov"], a["ws"], a["ws_bytes"], None)


def test_logits_topk_validation(L):
    assert _topk(L, n_heads=32) == E_UNSUP
    assert _topk(L, dtype=3) == E_UNSUP
    assert _topk(L, k=0) == E_INVAL
    assert _topk(L, k=2049) == E_INVAL
    assert _topk(L, n_q=-1) == E_INVAL
    assert _topk(L, q=None) == E_INVAL
    assert _topk(L, cu_q=None) == E_INVAL
    assert _topk(L, oi=None) == E_INVAL
    assert _topk(L, ws=None, ws_bytes=10 ** 9) == E_WS
    assert _topk(L, ws_bytes=100) == E_WS                    # < one row (256 + 128 * 4)
    assert _topk(L, ws=ctypes.c_void_p(0x1008), ws_bytes=10 ** 9) == E_INVAL   # 16-byte aligned
    assert _topk(L, n_q=0, q=None, w=None, oi=None, ws=None) == E_OK
    assert _topk(L, q=ctypes.c_void_p(0x1008), ws_bytes=10 ** 9) == E_INVAL   # q, kcache: 16-byte
    assert _topk(L, kc=ctypes.c_void_p(0x1004), ws_bytes=10 ** 9) == E_INVAL  # aligned


def test_fp8q_rotate_quantize_validation(L):
    MIS = ctypes.c_void_p(0x1008)

    def fp8q(codes=FAKE, scales=FAKE, n_q=3, ws=FAKE, ws_bytes=10 ** 9):
        return L.idx_logits_topk_fp8q(codes, scales, FAKE, FAKE, 4, FAKE, 1, 2, FAKE, FAKE, n_q,
                                      64, 512, FAKE, None, ws, ws_bytes, None)
    assert fp8q(scales=None) == E_INVAL
    assert fp8q(codes=MIS) == E_INVAL
    assert fp8q(ws=MIS) == E_INVAL
    assert fp8q(n_q=0, codes=None, scales=None, ws=None) == E_OK
    assert L.idx_rotate_q(FAKE, FAKE, -1, None) == E_INVAL
    assert L.idx_rotate_q(None, None, 0, None) == E_OK
    assert L.idx_rotate_q(None, FAKE, 4, None) == E_INVAL
    assert L.idx_rotate_q(MIS, FAKE, 4, None) == E_INVAL
    assert L.idx_rotate_q(FAKE, MIS, 4, None) == E_INVAL
    assert L.idx_quantize_q(FAKE, FAKE, None, 4, None) == E_INVAL
    assert L.idx_quantize_q(None, None, None, 0, None) == E_OK
    assert L.idx_quantize_q(MIS, FAKE, FAKE, 4, None) == E_INVAL
    assert L.idx_quantize_q(FAKE, MIS, FAKE, 4, None) == E_INVAL


def test_logits_dense_validation(L):
    def dense(**kw):
        a = dict(q=FAKE, w=FAKE, kc=FAKE, dtype=0, pool=4, pt=FAKE, n_seq=1, max_pages=2,
                 seq_lens=FAKE, cu_q=FAKE, n_q=3, n_heads=64, out=FAKE, max_keys=128)
        a.update(kw)
        return L.idx_logits_dense(a["q"], a["w"], a["kc"], a["dtype"], a["pool"], a["pt"],
                                  a["n_seq"], a["max_pages"], a["seq_lens"], a["cu_q"], a["n_q"],
                                  a["n_heads"], a["out"], a["max_keys"], None)
    assert dense(max_keys=0) == E_INVAL
    assert dense(out=None) == E_INVAL
    assert dense(n_heads=128) == E_UNSUP
    assert dense(n_q=0, out=None) == E_OK


def test_topk_rows_validation(L):
    f = L.idx_topk_rows
    assert f(FAKE, 4, 0, None, 10, FAKE, None, None, 0, None) == E_INVAL     # row_stride < 1
    assert f(FAKE, 4, 100, None, 0, FAKE, None, None, 0, None) == E_INVAL
    assert f(FAKE, 4, 100, None, 4096, FAKE, None, None, 0, None) == E_INVAL
    assert f(None, 4, 100, None, 10, FAKE, None, None, 0, None) == E_INVAL
    assert f(FAKE, -1, 100, None, 10, FAKE, None, None, 0, None) == E_INVAL
    assert f(None, 0, 100, None, 10, None, None, None, 0, None) == E_OK
    # a two-pass selection without its workspace
    assert f(FAKE, 4, 40000, None, 1024, FAKE, None, None, 0, None) == E_WS
    assert f(FAKE, 4, 40000, None, 1024, FAKE, None, ctypes.c_void_p(0x1004), 10 ** 9,
             None) == E_INVAL                                                 # misaligned


def test_sparse_attn_workspace_and_validation(L):
    # few rows split their lists: 32 rows x 1024 entries x 64 heads -> 5 splits (224 entries
    # each, the last 128), each keeping a 512-dim fp32 partial and (max, sum) per head
    part = 64 * (512 * 4 + 8)
    assert L.idx_sparse_attn_workspace_size(32, 64, 1024) == 32 * 5 * part
    assert L.idx_sparse_attn_workspace_size(256, 64, 512) == 0      # enough rows: no split
    # lists longer than one workgroup's slot table (2048 entries, 1024 with 32 heads) are split
    assert L.idx_sparse_attn_workspace_size(300, 64, 3000) == 300 * 2 * part
    assert L.idx_sparse_attn_workspace_size(300, 64, 1500) == 0
    assert L.idx_sparse_attn_workspace_size(300, 32, 1500) == 300 * 2 * 32 * (512 * 4 + 8)
    assert L.idx_sparse_attn_workspace_size(8192, 128, 512) == 0
    assert L.idx_sparse_attn_workspace_size(32, 48, 1024) == 0      # unsupported head count
    F = ctypes.c_void_p(0x1000)
    MIS = ctypes.c_void_p(0x1008)                                  # not 16-byte aligned
    f = ctypes.c_float

    def call(q=F, kv=F, n_slots=10, slot=F, n_seq=1, max_keys=8, cu=F, idx=F, n_q=4, h=64,
             k=16, scale=0.1, out=F, ws=None, ws_bytes=0):
        return L.idx_sparse_attn(q, kv, n_slots, slot, n_seq, max_keys, cu, idx, n_q, h, k,
                                 f(scale), out, None, ws, ws_bytes, None)
    assert call(n_q=0) == E_OK
    assert call(h=48) == E_UNSUP
    assert call(k=0) == E_INVAL
    assert call(n_q=-1) == E_INVAL
    assert call(n_seq=0) == E_INVAL
    assert call(max_keys=0) == E_INVAL
    assert call(n_slots=-1) == E_INVAL
    assert call(scale=float("nan")) == E_INVAL
    assert call(scale=float("inf")) == E_INVAL
    assert call(scale=0.0) == E_INVAL
    assert call(scale=-0.5) == E_INVAL
    assert call(q=None) == E_INVAL
    assert call(idx=None) == E_INVAL
    assert call(out=None) == E_INVAL
    assert call(q=MIS) == E_INVAL
    assert call(kv=MIS) == E_INVAL
    assert call(out=MIS) == E_INVAL
    assert call(n_q=32, k=1024) == E_WS                              # split: needs a workspace
    assert call(n_q=32, k=1024, ws=F, ws_bytes=100) == E_WS
    assert call(n_q=32, k=1024, ws=MIS, ws_bytes=10 ** 9) == E_INVAL       # misaligned workspace


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        ix.store_keys(x, torch.ones(128), torch.zeros(4, dtype=torch.int32),
                      torch.zeros(1, 1, dtype=torch.int32), torch.zeros(8448, dtype=torch.uint8),
                      ix.FP8)
