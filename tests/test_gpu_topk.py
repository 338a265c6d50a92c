"""S3 parity.

1. The selection kernel alone against the oracle's full sort on identical fp32 inputs: index
   sets and their values must match exactly (ties broken toward the lower index, -0 == +0), for rows with
   heavy ties, short rows, rows longer than the LDS cache and every k the API allows.
2. The whole read path (score + select) against fp64 oracle logits: exact sets wherever the
   oracle's k-th / (k+1)-th gap exceeds the logit tolerance, near-tie validity everywhere and
   mean overlap >= 0.999.
3. GPU self-consistency: idx_logits_topk equals idx_topk_rows applied to idx_logits_dense, and
   chunking the queries through a small workspace changes nothing.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import (by_index, check_topk_sets, dev_inputs, gpu_store, oracle_rows,
                           query_positions, workload)

pytestmark = pytest.mark.gpu
FP8, BF16 = W.FP8, W.BF16


def _rows(seed, n_rows, stride, kind):
    r = np.random.default_rng(seed)
    if kind == "ties":
        v = r.integers(-3, 4, (n_rows, stride)).astype(np.float32)
        v[v == 0] = np.where(r.random((v == 0).sum()) < 0.5, -0.0, 0.0)
    elif kind == "ties3":   # three values: the threshold value fills more slots than LDS lists
        v = r.integers(-1, 2, (n_rows, stride)).astype(np.float32)
    elif kind == "normal":
        v = r.standard_normal((n_rows, stride)).astype(np.float32)
    else:   # few distinct values with -inf mixed in
        v = r.choice(np.array([-np.inf, -1.5, 0.25, 7.0], np.float32), (n_rows, stride))
    return v


@pytest.mark.parametrize("n_rows,stride,k,kind", [
    (64, 1024, 512, "ties"), (64, 1024, 512, "normal"), (8, 5632, 512, "mixed"),
    (4, 32768, 1024, "normal"), (3, 32768, 2048, "ties"), (2, 40000, 1024, "normal"),
    (2, 40000, 700, "ties"), (16, 100, 1, "ties"), (16, 100, 2048, "normal"),
    (5, 513, 512, "ties"), (5, 512, 512, "normal"),
    # more rows than the one-workgroup-per-row path takes: one wave per row or segment
    (160, 6000, 512, "normal"), (150, 40000, 1024, "normal"), (140, 20000, 2048, "ties"),
    (129, 9000, 64, "mixed"),
    # whole rows, one wave each, order unspecified: the threshold bin listed in LDS, or (ties3,
    # mixed) too full for the list and filtered in registers; the longest row one wave holds
    (200, 4000, 512, "ties"), (136, 6100, 1000, "mixed"), (150, 6000, 512, "ties3"),
    (130, 6144, 2048, "normal"), (131, 3000, 1, "normal"),
])
def test_topk_rows_bit_exact(oracle_mod, n_rows, stride, k, kind):
    v = _rows(n_rows * 1000003 + stride * 31 + k + 7 * len(kind), n_rows, stride, kind)
    row_len = np.random.default_rng(5).integers(0, stride + 1, n_rows).astype(np.int32)
    row_len[0] = stride
    row_len[-1] = min(k, stride)
    gi, gv = ix.topk_rows(torch.from_numpy(v).cuda(), k, torch.from_numpy(row_len).cuda())
    oi, ov = oracle_mod.topk(v, k, row_len=row_len)
    gi, gv = gi.cpu().numpy(), gv.cpu().numpy()
    for r in range(n_rows):
        m = min(k, int(row_len[r]))
        # the same set (the order within a row is unspecified: compared by index)
        g_order = np.argsort(gi[r, :m])
        o_order = np.argsort(oi[r, :m])
        assert np.array_equal(gi[r, :m][g_order], oi[r, :m][o_order]), f"row {r}"
        assert np.all(gi[r, m:] == -1)
        # values equal (a -0 score is returned as +0)
        assert np.array_equal(gv[r, :m][g_order], ov[r, :m][o_order].astype(np.float32))
        assert np.all(np.isneginf(gv[r, m:]))


def _gpu_topk(wl, d, pool, dtype, workspace=None, want_values=False):
    return ix.logits_topk(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"], d["cu_q"],
                          wl.k, workspace=workspace, want_values=want_values)


@pytest.mark.parametrize("cfg,dtype,stride", [(0, FP8, 1), (1, BF16, 1), (2, FP8, 1),
                                              (2, BF16, 1), (3, BF16, 8), (4, FP8, 1),
                                              (4, BF16, 1)])
def test_logits_topk_vs_oracle(oracle_mod, cfg, dtype, stride):
    """The full path as measured: keys stored by the GPU, then score + select on the GPU; the
    oracle checks every stride-th row and the last (1,025 of the long prefill chunk's 8,192)."""
    wl = workload(cfg)
    print(f"topk cfg{cfg} dtype={dtype}", flush=True)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d)
    gi, _ = _gpu_topk(wl, d, pool, dtype)
    gi = gi.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, wl.n_q, stride), [wl.n_q - 1]]))
    pool_o, _ = oracle_mod.store_workload(wl, dtype)
    o, nv = oracle_rows(oracle_mod, wl, pool_o, dtype, rows)
    mean, exact = check_topk_sets(gi[rows], o, nv, wl.k, f"cfg{cfg}")
    print(f"  rows={rows.size} overlap={mean:.6f} exact-gap rows={exact}", flush=True)


@pytest.mark.parametrize("dtype", [FP8, BF16])
def test_logits_topk_ragged(oracle_mod, dtype):
    wl = W.make_workload("ragged", 31 + dtype, [0, 3, 4, 130, 700, 1500, 2100],
                         [0, 2, 1, 7, 33, 70, 3], 64, permute_pages=True, extra_pages=2)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d)
    gi, gv = _gpu_topk(wl, d, pool, dtype, want_values=True)
    pool_o, _ = oracle_mod.store_workload(wl, dtype)
    o, nv = oracle_rows(oracle_mod, wl, pool_o, dtype, None)
    check_topk_sets(gi.cpu().numpy(), o, nv, wl.k, "ragged")
    gv = gv.cpu().numpy()
    gi = gi.cpu().numpy()
    for r in range(wl.n_q):
        m = min(wl.k, int(nv[r]))
        assert np.all(np.isneginf(gv[r, m:]))
        assert np.allclose(gv[r, :m], o[r, gi[r, :m]], rtol=2e-3, atol=1e-3)


@pytest.mark.parametrize("cfg,dtype", [(2, FP8), (2, BF16), (0, FP8), (3, BF16), (4, BF16)])
def test_topk_matches_dense_then_select(cfg, dtype):
    wl = workload(cfg)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d)
    gi, gv = _gpu_topk(wl, d, pool, dtype, want_values=True)
    dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.max_keys)
    nvis = torch.isfinite(dense).sum(dim=1).to(torch.int32)
    si, sv = ix.topk_rows(dense, wl.k, nvis)
    gi, gv = by_index(gi, gv)
    si, sv = by_index(si, sv)
    assert torch.equal(gi, si)
    assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))


def test_small_workspace_chunks_queries():
    wl = workload(0)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP8, d)
    full, _ = _gpu_topk(wl, d, pool, FP8)
    ws = torch.empty(ix.min_workspace(wl.n_seq, wl.max_pages, wl.k) * 3 + 100, dtype=torch.uint8,
                     device="cuda")
    part, _ = _gpu_topk(wl, d, pool, FP8, workspace=ws)
    assert torch.equal(by_index(full), by_index(part))


def test_too_small_workspace_raises():
    wl = workload(0)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP8, d)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ix.IndexerError):
        _gpu_topk(wl, d, pool, FP8, workspace=ws)


def test_logits_topk_repeatable():
    wl = workload(4)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP8, d)
    a, _ = _gpu_topk(wl, d, pool, FP8)
    b, _ = _gpu_topk(wl, d, pool, FP8)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,k", [(FP8, 512), (BF16, 1024), (FP8, 64)])
def test_decode_selection_matches_dense_then_select(dtype, k):
    """Decode-shaped batches (few long rows; one workgroup per row, or segments and a second pass
    for rows longer than a workgroup holds).  Rows shorter than k, rows just below and above k,
    and keys on an invalid page (-inf) included; the result must equal the selection over the
    dense logits, bit for bit."""
    r = np.random.default_rng(40 + k)
    lens = r.integers(8, 60000, 24).astype(np.int32)
    lens[:3] = [12, 4 * k - 4, 4 * k + 8]             # n_vis < k, just below and above k
    wl = W.make_workload("decode-ragged", 77 + k, lens, np.ones(lens.size, np.int32), k,
                         permute_pages=True, max_pages=240)
    wl.page_table[5, 3] = wl.n_pages_pool + 7           # keys 192..255 of row 5 score -inf
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d)
    gi, gv = _gpu_topk(wl, d, pool, dtype, want_values=True)
    dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.max_keys)
    t = query_positions(wl)
    nv = torch.from_numpy(np.minimum((t + 1) // 4, wl.max_keys).astype(np.int32)).cuda()
    si, sv = ix.topk_rows(dense, wl.k, nv)
    gi, gv = by_index(gi, gv)
    si, sv = by_index(si, sv)
    assert torch.equal(gi, si)
    assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))


@pytest.mark.parametrize("dtype,k", [(FP8, 64), (BF16, 512), (FP8, 1024), (BF16, 2048)])
def test_long_row_selection_matches_dense_then_select(dtype, k):
    """Rows of more than 16384 key columns, which are selected from each scoring workgroup's keys
    bucketed by histogram bin: the front of every list, or, when the threshold bin reaches past
    it (small k), the lists read in full.  Ragged rows up to 37,500 keys, rows shorter than k and
    just above it, and keys on an invalid page included; the result must equal the selection
    over the dense logits, bit for bit."""
    r = np.random.default_rng(90 + k)
    lens = r.integers(8, 150000, 12).astype(np.int32)
    lens[:3] = [12, 4 * k - 4, 4 * k + 8]             # n_vis < k, just below and above k
    lens[3] = 150000
    wl = W.make_workload("decode-long-ragged", 91 + k, lens, np.ones(lens.size, np.int32), k,
                         permute_pages=True, max_pages=600)
    wl.page_table[3, 40] = wl.n_pages_pool + 7          # keys 2560..2623 of row 3 score -inf
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d)
    gi, gv = _gpu_topk(wl, d, pool, dtype, want_values=True)
    dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.max_keys)
    t = query_positions(wl)
    nv = torch.from_numpy(np.minimum((t + 1) // 4, wl.max_keys).astype(np.int32)).cuda()
    si, sv = ix.topk_rows(dense, wl.k, nv)
    gi, gv = by_index(gi, gv)
    si, sv = by_index(si, sv)
    assert torch.equal(gi, si)
    assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))


@pytest.mark.parametrize("budget", ["min", 4 << 20, 11 << 20, "recommended"])
def test_workspace_guard_bytes(budget):
    """More than 128 rows of more than 6144 keys go through the segmented selection, whose
    candidate buffers a one-row chunk does not need: however the workspace budget cuts the
    batch into chunks, nothing is written outside it, and the selection equals the one made
    with a workspace for the whole batch in one pass."""
    wl = W.make_workload("guard", 909, [4 * 7100], [300], 512, permute_pages=True)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, BF16, d)
    full, _ = _gpu_topk(wl, d, pool, BF16)
    if budget == "min":
        nbytes = ix.min_workspace(wl.n_seq, wl.max_pages, wl.k)
    elif budget == "recommended":
        nbytes = ix.workspace_size(wl.n_q, wl.n_seq, wl.max_pages, wl.k)
    else:
        nbytes = budget
    rows, most = ix.topk_plan(wl.n_q, wl.n_seq, wl.max_pages, wl.k, nbytes)
    print(f"guard budget={nbytes} rows/chunk={rows} most={most}", flush=True)
    assert most <= nbytes
    guard = 1 << 16
    buf = torch.full((nbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = buf[guard:guard + nbytes]
    part, _ = _gpu_topk(wl, d, pool, BF16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(buf[:guard] == 0x5A), "bytes written before the workspace"
    assert torch.all(buf[guard + nbytes:] == 0x5A), "bytes written after the workspace"
    assert torch.equal(by_index(full), by_index(part))


@pytest.mark.parametrize("dtype,k", [(BF16, 1024), (FP8, 512), (BF16, 2048)])
def test_decode_selection_ties_match_dense_then_select(dtype, k):
    """Decode rows whose scores tie massively: a sequence of all-zero keys (every score 0, so
    the threshold bin holds the whole row, more than a workgroup lists in LDS), a sequence whose
    keys take three values (dims 64..127 zero, so the rotation leaves identical rows identical),
    a row shorter than k and long plain rows.  Ties go to the lower index; the selection must
    equal the one made over the dense logits, bit for bit."""
    lens = np.array([4 * 9000, 4 * 5000, 4 * 700, 4 * 20000, 4 * 4100, 4 * 33000], np.int32)
    wl = W.make_workload("decode-ties", 515 + k, lens, np.ones(lens.size, np.int32), k,
                         permute_pages=True)
    x = wl.x.copy()
    x[wl.key_seq == 0] = 0.0
    rows1 = np.nonzero(wl.key_seq == 1)[0]
    x[rows1] = x[rows1[np.arange(rows1.size) % 3]]
    x[rows1, 64:] = 0.0
    d = dev_inputs(wl, x)
    pool = gpu_store(ix, wl, dtype, d)
    gi, gv = _gpu_topk(wl, d, pool, dtype, want_values=True)
    dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                            d["cu_q"], wl.max_keys)
    t = query_positions(wl)
    nv = torch.from_numpy(np.minimum((t + 1) // 4, wl.max_keys).astype(np.int32)).cuda()
    si, sv = ix.topk_rows(dense, wl.k, nv)
    gi, gv = by_index(gi, gv)
    si, sv = by_index(si, sv)
    assert torch.equal(gi, si)
    assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))
    assert torch.equal(gi[0, :k].cpu(), torch.arange(k, dtype=torch.int32))   # all ties: 0..k-1
