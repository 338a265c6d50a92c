"""Prefill-shaped batches of several sequences (1024 or more query rows, at least 4 per sequence),
the shape the rows kernels serve: each workgroup scores 4 consecutive rows, and here its rows
belong to different sequences (query counts that are not multiples of 4), some rows see no key
(queries at the first tokens), one sequence has no query, and the page table has a hole and a
page beyond the pool.  Dense logits against the oracle on every row, through the bf16 DMA
kernel, the register-staged fp8 and fp4 kernels and the fp8 x fp8 kernel; top-k against the
oracle, and equal to dense-then-select.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import (by_index, check_logits, check_topk_sets, dev_inputs, gpu_store,
                           oracle_rows, query_positions, tolerance_ratio)

pytestmark = pytest.mark.gpu
FP8, BF16, FP4 = W.FP8, W.BF16, W.FP4

SEQ_LENS = [2, 0, 37, 900, 3000, 64, 1500, 5000, 130, 2200]
Q_LENS = [2, 0, 5, 301, 250, 3, 151, 197, 9, 110]     # 1028 rows in 10 sequences


def _workload(seed, k, dtypes):
    wl = W.make_workload("prefill-multiseq", seed, SEQ_LENS, Q_LENS, k, permute_pages=True,
                         extra_pages=3, dtypes=dtypes)
    assert wl.n_q >= 1024 and wl.n_q >= 4 * wl.n_seq      # prefill-shaped: the rows kernels
    wl.page_table[6, 5] = -1                              # keys 320..383 of sequence 6: -inf
    wl.page_table[7, 2] = wl.n_pages_pool + 4             # keys 128..191 of sequence 7: -inf
    return wl


def _pool(oracle_mod, wl, dtype):
    pool, _ = oracle_mod.store_workload(wl, dtype)
    return pool


@pytest.mark.parametrize("dtype", [BF16, FP8, FP4])
def test_multiseq_dense_logits(oracle_mod, dtype):
    wl = _workload(300 + dtype, 512, (dtype,))
    pool = _pool(oracle_mod, wl, dtype)
    d = dev_inputs(wl)
    g = ix.logits_dense(d["q"], d["w"], torch.from_numpy(pool).cuda(), dtype, d["page_table"],
                        d["seq_lens"], d["cu_q"], wl.max_keys).cpu().numpy()
    o, nv = oracle_rows(oracle_mod, wl, pool, dtype, None)
    check_logits(g, o, f"multiseq dtype={dtype}")
    assert nv.min() == 0 and nv.max() > 1000


def test_multiseq_dense_logits_fp8q(oracle_mod):
    wl = _workload(310, 512, (FP8,))
    pool = _pool(oracle_mod, wl, FP8)
    d = dev_inputs(wl)
    codes, scales = ix.quantize_q(d["q"])
    g = ix.logits_dense_fp8q(codes, scales, d["w"], torch.from_numpy(pool).cuda(),
                             d["page_table"], d["seq_lens"], d["cu_q"], wl.max_keys).cpu().numpy()
    oc, os_ = oracle_mod.quantize_q(wl.q_bits)
    o, _ = oracle_mod.logits_fp8q(oc, os_, wl.w, pool, wl.page_table, wl.seq_lens, wl.cu_q,
                                  row_len=wl.max_keys)
    check_logits(g, o, "multiseq fp8q")
    assert tolerance_ratio(g, o) < 1.0


@pytest.mark.parametrize("dtype,k", [(BF16, 512), (FP8, 64), (FP4, 512)])
def test_multiseq_topk(oracle_mod, dtype, k):
    """The whole path (GPU store, score, select) against the oracle, and equal to the selection
    over the GPU's own dense logits."""
    wl = _workload(320 + dtype, k, (dtype,))
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d)
    gi, gv = ix.logits_topk(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.k, want_values=True)
    o, nv = oracle_rows(oracle_mod, wl, _pool(oracle_mod, wl, dtype), dtype, None)
    mean, exact = check_topk_sets(gi.cpu().numpy(), o, nv, wl.k, f"multiseq dtype={dtype}")
    print(f"  overlap={mean:.6f} exact-gap rows={exact}", flush=True)
    dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.max_keys)
    # each row's causal length: the page holes are -inf keys inside that prefix, not past it
    t = query_positions(wl)
    nvis = torch.from_numpy(np.minimum((t + 1) // 4, wl.max_keys).astype(np.int32)).cuda()
    si, sv = ix.topk_rows(dense, wl.k, nvis)
    gi, gv = by_index(gi, gv)
    si, sv = by_index(si, sv)
    assert torch.equal(gi, si)
    assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))
    assert (nv < wl.k).any() and (nv > wl.k).any()        # padded and selected rows both occur


@pytest.mark.parametrize("k,want_values", [(512, False), (2048, True), (1, True), (100, False)])
def test_prefill_selection_ties_match_dense_then_select(k, want_values):
    """Prefill-shaped bf16 batches go through the rows scoring kernel and the whole-row
    selection (one wave per row).  Rows whose scores tie massively (a sequence of all-zero keys:
    every score 0, so the threshold bin holds the whole row, more than a wave lists in LDS; a
    sequence whose keys take three values), rows shorter than k, rows that see no key and long
    plain rows (5632 keys) must give the selection made over the dense logits, bit for bit, with
    and without values, for k from 1 to 2048."""
    seq_lens = [22528, 3000, 2500, 900, 40, 12000]
    q_lens = [420, 250, 301, 151, 9, 110]           # 1241 rows
    wl = W.make_workload("prefill-ties", 640 + k, seq_lens, q_lens, k, permute_pages=True,
                         extra_pages=2, dtypes=(BF16,))
    assert wl.n_q >= 1024 and wl.n_q >= 4 * wl.n_seq and wl.max_keys <= 6144
    x = wl.x.copy()
    x[wl.key_seq == 1] = 0.0
    rows2 = np.nonzero(wl.key_seq == 2)[0]
    x[rows2] = x[rows2[np.arange(rows2.size) % 3]]
    x[rows2, 64:] = 0.0
    d = dev_inputs(wl, x)
    pool = gpu_store(ix, wl, BF16, d)
    gi, gv = ix.logits_topk(d["q"], d["w"], pool, BF16, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.k, want_values=want_values)
    assert (gv is not None) == want_values
    dense = ix.logits_dense(d["q"], d["w"], pool, BF16, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.max_keys)
    t = query_positions(wl)
    nvis = torch.from_numpy(np.minimum((t + 1) // 4, wl.max_keys).astype(np.int32)).cuda()
    si, sv = ix.topk_rows(dense, wl.k, nvis)
    si, sv = by_index(si, sv)
    if want_values:
        gi, gv = by_index(gi, gv)
        assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))
    else:
        gi = by_index(gi)
    assert torch.equal(gi, si)
    # sequence 1 scores 0 everywhere: its rows take their first k keys (ties to the lower index)
    r1 = np.nonzero((np.arange(wl.n_q) >= wl.cu_q[1]) & (np.arange(wl.n_q) < wl.cu_q[2]))[0]
    nv1 = nvis[torch.from_numpy(r1).cuda()].cpu().numpy()
    full = r1[nv1 >= k]
    assert full.size > 0 or k > nv1.max()
    if full.size:
        want = torch.arange(k, dtype=torch.int32).expand(full.size, k)
        assert torch.equal(gi[torch.from_numpy(full).cuda(), :k].cpu(), want)
