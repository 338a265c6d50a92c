"""The allocation-free entry point (idx_logits_topk_noalloc) against idx_logits_topk.

Called through the C ABI (ctypes), twice in a row on one GPU, the second call with a smaller
batch, so the second reads a scratch the first has left full: both must equal the workspace
entry point's selection (index sets and values, bit for bit; the same kernels run).
"""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import by_index, dev_inputs, gpu_store, workload

pytestmark = pytest.mark.gpu


def _noalloc(wl, d, pool, dtype):
    L = ix.lib()
    n_q = wl.n_q
    out_idx = torch.full((n_q, wl.k), -7, dtype=torch.int32, device="cuda")
    out_val = torch.full((n_q, wl.k), 7.0, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = L.idx_logits_topk_noalloc(
        p(d["q"]), p(d["w"]), p(pool), dtype, wl.n_pages_pool, p(d["page_table"]), wl.n_seq,
        wl.max_pages, p(d["seq_lens"]), p(d["cu_q"]), n_q, 64, wl.k, p(out_idx), p(out_val),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.idx_status_string(st)
    return out_idx, out_val


def _reference(wl, d, pool, dtype):
    return ix.logits_topk(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"], d["cu_q"],
                          wl.k, want_values=True)


def test_noalloc_matches_workspace_entry_point():
    L = ix.lib()
    assert L.idx_logits_topk_noalloc_scratch_bytes() == 64 << 20
    cases = [(workload(4), W.FP8), (workload(2), W.BF16)]   # 32 x 32768 keys, then 64 x <= 5632
    for wl, dtype in cases:
        print(f"noalloc {wl.name} dtype={dtype} n_q={wl.n_q}", flush=True)
        d = dev_inputs(wl)
        pool = gpu_store(ix, wl, dtype, d)
        gi, gv = _noalloc(wl, d, pool, dtype)
        ri, rv = _reference(wl, d, pool, dtype)
        torch.cuda.synchronize()
        gi, gv = by_index(gi, gv)
        ri, rv = by_index(ri, rv)
        assert torch.equal(gi, ri)
        assert torch.equal(gv.view(torch.int32), rv.view(torch.int32))


def test_noalloc_chunks_a_batch_larger_than_its_scratch():
    """The long prefill chunk's full workspace (185 MB) exceeds the scratch: the call runs it in
    query chunks and still equals the workspace entry point on sampled rows."""
    wl = workload(3)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, W.BF16, d)
    rows, most = ix.topk_plan(wl.n_q, wl.n_seq, wl.max_pages, wl.k,
                              ix.lib().idx_logits_topk_noalloc_scratch_bytes())
    assert 1 <= rows < wl.n_q and most <= 64 << 20
    gi, gv = _noalloc(wl, d, pool, W.BF16)
    ri, rv = _reference(wl, d, pool, W.BF16)
    torch.cuda.synchronize()
    gi, gv = by_index(gi, gv)
    ri, rv = by_index(ri, rv)
    assert torch.equal(gi, ri)
    assert torch.equal(gv.view(torch.int32), rv.view(torch.int32))


def test_noalloc_validation():
    L = ix.lib()
    f = L.idx_logits_topk_noalloc
    fake = ctypes.c_void_p(0x1000)
    # host-side checks return before any HIP call
    assert f(fake, fake, fake, 1, 4, fake, 1, 2, fake, fake, 3, 32, 512, fake, None, None) == 2
    assert f(fake, fake, fake, 1, 4, fake, 1, 2, fake, fake, 3, 64, 0, fake, None, None) == 1
    assert f(None, None, None, 1, 4, None, 1, 2, None, None, 0, 64, 512, None, None, None) == 0
    # a single query row of 2^25 keys (128 MiB of scores) needs more than the scratch holds:
    # rejected before the scratch is looked up or anything is launched
    assert f(fake, fake, fake, 1, 4, fake, 1, 1 << 19, fake, fake, 1, 64, 512, fake, None,
             None) == 3
