"""Sparse attention over the selected keys against the fp64 oracle.

Tolerance, from the arithmetic: scores accumulate in fp32 from exact bf16 products (relative error
about 1e-6); each softmax weight is rounded to bf16 (relative 2^-9) and the weights are divided by
the sum of the rounded values, so the weighted sum moves by at most about 2 * 2^-9 of the largest
|v_d| among the listed latents; the output is rounded to bf16 (2^-9 of |o_d|).  Each element must
satisfy |gpu - oracle| <= 2^-7 * max_j |v_jd| + 2^-8 * |oracle| + 1e-6, and the log-sum-exp
(whose weight sum carries the same 2^-9) |gpu - oracle| <= 2^-8 + 1e-5 * |oracle|.  Rows with
nothing to attend to must give exactly 0 and -inf.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import workload

pytestmark = pytest.mark.gpu


def _bf16_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _run_gpu(a: W.AttnInputs, cu_q):
    q, kv, kv_slot, idx = a.torch_inputs()
    out, lse = ix.sparse_attn(q, kv, kv_slot, torch.from_numpy(cu_q).cuda(), idx, a.scale)
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return _bf16_f64(o), lse.cpu().numpy().astype(np.float64)


def _vmax(a: W.AttnInputs, cu_q, rows):
    """Per row and dim, the largest |v_d| among the latents the row lists."""
    out = np.zeros((rows.size, W.LATENT_DIM))
    n_seq, max_keys = a.kv_slot.shape
    for r, i in enumerate(rows):
        b = int(np.searchsorted(cu_q, i, side="right") - 1)
        if b < 0 or b >= n_seq:
            continue
        s = a.idx[i]
        s = s[(s >= 0) & (s < max_keys)]
        sl = a.kv_slot[b, s]
        sl = sl[(sl >= 0) & (sl < a.kv_bits.shape[0])]
        if sl.size:
            out[r] = np.abs(_bf16_f64(a.kv_bits[sl])).max(axis=0)
    return out


def _check(a, cu_q, g_out, g_lse, rows, oracle_mod, what):
    o, l = oracle_mod.sparse_attn(a.q_bits, a.kv_bits, a.kv_slot, cu_q, a.idx, a.scale, rows=rows)
    g_out, g_lse = g_out[rows], g_lse[rows]
    empty = np.isneginf(l)
    assert np.array_equal(np.isneginf(g_lse), empty), f"{what}: empty rows differ"
    assert np.all(g_out[empty] == 0), f"{what}: an empty row must be 0"
    tol = (2.0 ** -7) * _vmax(a, cu_q, rows)[:, None, :] + (2.0 ** -8) * np.abs(o) + 1e-6
    err = np.abs(g_out - o)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance; max err "
                           f"{err.max():.3g}, max err / tol {(err / tol).max():.3g}")
    fin = ~empty
    lerr = np.abs(g_lse[fin] - l[fin])
    assert np.all(lerr <= 2.0 ** -8 + 1e-5 * np.abs(l[fin])), f"{what}: lse max err {lerr.max()}"
    return float(err.max()), float((err / tol).max()), float(lerr.max()) if lerr.size else 0.0


def _rows(n_q, n, seed):
    if n is None or n >= n_q:
        return np.arange(n_q, dtype=np.int64)
    pick = np.random.default_rng(seed).choice(n_q, n - 2, replace=False)
    return np.unique(np.concatenate([[0, n_q - 1], pick])).astype(np.int64)


@pytest.mark.parametrize("cfg,n_heads,n_rows", [(0, 64, 48), (2, 64, None), (4, 64, None),
                                                (3, 64, 24), (0, 128, 24), (2, 32, None),
                                                (4, 128, None), (2, 128, None)])
def test_attn_vs_oracle(oracle_mod, cfg, n_heads, n_rows):
    """The measured shapes: prefill rows (one workgroup per row and head block) and decode rows
    (lists split over several workgroups, then merged), 32, 64 and 128 heads."""
    wl = workload(cfg) if cfg != 4 else W.cfg4(needles=False)
    a = W.attn_inputs(wl, n_heads=n_heads)
    cu_q = wl.cu_q
    print(f"attn cfg{cfg} heads={n_heads} rows={wl.n_q} k={a.idx.shape[1]} split_ws="
          f"{ix.sparse_attn_workspace_size(wl.n_q, n_heads, a.idx.shape[1])}", flush=True)
    g_out, g_lse = _run_gpu(a, cu_q)
    rows = _rows(wl.n_q, n_rows, cfg)
    e, r, le = _check(a, cu_q, g_out, g_lse, rows, oracle_mod, f"cfg{cfg}")
    print(f"  rows={rows.size} max err {e:.3g} (err/tol {r:.3f}), lse max err {le:.3g}", flush=True)


def _ragged_inputs(seed, n_heads=64, k=96):
    wl = W.make_workload("ragged", seed, [0, 3, 4, 130, 700, 1500, 2100],
                         [0, 2, 1, 7, 33, 70, 3], k, permute_pages=True)
    a = W.attn_inputs(wl, n_heads=n_heads, k=k, scale=0.3)
    r = np.random.default_rng(seed)
    idx = a.idx.copy()
    # duplicates, entries beyond max_keys, negative entries in the middle of a list
    idx[40, 5] = idx[40, 6]
    idx[41, 2] = wl.max_keys + 7
    idx[42, 0] = -3
    idx[43, :] = -1                                    # an explicitly empty row
    kv_slot = a.kv_slot.copy()
    kv_slot[5, :40] = -1                               # unmapped keys
    kv_slot[6, 10:20] = a.kv_bits.shape[0] + r.integers(0, 9, 10)   # rows beyond kv
    return wl, W.AttnInputs(a.q_bits, a.kv_bits, kv_slot, idx, a.scale)


@pytest.mark.parametrize("n_heads", [32, 64, 128])
def test_attn_ragged_and_invalid_entries(oracle_mod, n_heads):
    """Empty and short sequences (rows with no visible key), lists with duplicates, negative and
    too-large entries, unmapped keys and slots beyond the latents."""
    wl, a = _ragged_inputs(71, n_heads)
    cu_q = wl.cu_q
    g_out, g_lse = _run_gpu(a, cu_q)
    _check(a, cu_q, g_out, g_lse, np.arange(wl.n_q, dtype=np.int64), oracle_mod, "ragged")
    assert np.isneginf(g_lse[43]).all() and np.all(g_out[43] == 0)


def test_attn_rows_outside_the_sequences(oracle_mod):
    """Rows past cu_q[n_seq] belong to no sequence: they attend to nothing."""
    wl = workload(2)
    a = W.attn_inputs(wl, k=64)
    cu_q = wl.cu_q.copy()
    cu_q[-5:] = cu_q[-6]                               # the last 5 sequences get no rows, so
                                                       # the last 5 rows fall outside
    g_out, g_lse = _run_gpu(a, cu_q)
    assert np.all(g_out[-5:] == 0) and np.isneginf(g_lse[-5:]).all()
    _check(a, cu_q, g_out, g_lse, np.arange(wl.n_q, dtype=np.int64), oracle_mod, "outside")


def test_attn_single_key_rows_are_exact(oracle_mod):
    """One listed key: the weight is exactly 1, so the output is that latent, bit for bit."""
    wl = workload(2)
    a = W.attn_inputs(wl, k=64)
    a.idx[:, 1:] = -1
    g_out, _ = _run_gpu(a, wl.cu_q)
    for i in range(wl.n_q):
        b = int(np.searchsorted(wl.cu_q, i, side="right") - 1)
        v = _bf16_f64(a.kv_bits[a.kv_slot[b, a.idx[i, 0]]])
        assert np.array_equal(g_out[i], np.broadcast_to(v, g_out[i].shape))


def test_attn_list_order_does_not_matter():
    """The list is a set of terms: permuting every row's entries changes the result only by the
    order of fp32 additions."""
    wl = workload(2)
    a = W.attn_inputs(wl, k=256)
    g1, l1 = _run_gpu(a, wl.cu_q)
    r = np.random.default_rng(3)
    idx = np.stack([r.permutation(row) for row in a.idx]).astype(np.int32)
    g2, l2 = _run_gpu(W.AttnInputs(a.q_bits, a.kv_bits, a.kv_slot, idx, a.scale), wl.cu_q)
    assert np.allclose(g1, g2, atol=2.0 ** -7, rtol=2.0 ** -7)
    assert np.allclose(l1, l2, atol=2.0 ** -8)


def test_attn_on_the_oracle_selection(oracle_mod):
    """The path end to end on its own numbers: the oracle's top-k of the oracle's logits (the
    indexer's output) is the list the attention reads, on the 4K prefill rows."""
    wl = workload(0)
    pool, _ = oracle_mod.store_workload(wl, W.BF16)
    rows = np.arange(0, wl.n_q, 8, dtype=np.int64)
    lg, nv = oracle_mod.logits(wl.q_bits, wl.w, pool, W.BF16, wl.page_table, wl.seq_lens,
                               wl.cu_q, rows=rows)
    sel, _ = oracle_mod.topk(lg, wl.k, row_len=nv)
    a = W.attn_inputs(wl)
    idx = np.full_like(a.idx, -1)
    idx[rows] = sel
    a = W.AttnInputs(a.q_bits, a.kv_bits, a.kv_slot, idx, a.scale)
    g_out, g_lse = _run_gpu(a, wl.cu_q)
    _check(a, wl.cu_q, g_out, g_lse, rows, oracle_mod, "oracle selection")


def test_attn_long_lists_are_split(oracle_mod):
    """Lists longer than one workgroup's slot table (2048 entries) are split even when the batch
    has enough rows, and merged: 300 rows with k = 3000 over sequences of up to 4000 keys."""
    wl = W.make_workload("long-lists", 61, [16000, 12000], [150, 150], 3000, permute_pages=True)
    a = W.attn_inputs(wl, k=3000)
    assert ix.sparse_attn_workspace_size(wl.n_q, 64, 3000) > 0, "the lists must be split"
    g_out, g_lse = _run_gpu(a, wl.cu_q)
    rows = _rows(wl.n_q, 12, 61)
    _check(a, wl.cu_q, g_out, g_lse, rows, oracle_mod, "long lists")


def test_attn_repeatable():
    wl = workload(2)
    a = W.attn_inputs(wl)
    g1, l1 = _run_gpu(a, wl.cu_q)
    g2, l2 = _run_gpu(a, wl.cu_q)
    assert np.array_equal(g1, g2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("n_heads", [64, 128])
def test_attn_split_lists_with_empty_splits(oracle_mod, n_heads):
    """Few rows, so every list is split and merged (with 128 heads, in two head blocks per row):
    the first half of each list is padding, so the first splits hold no key (the merge starts
    from the later ones), some rows hold nothing at all, and one row's only valid entries sit in
    its last split."""
    wl = workload(4)                                   # 32 decode rows, 1024 listed keys
    a = W.attn_inputs(wl, n_heads=n_heads)
    assert ix.sparse_attn_workspace_size(wl.n_q, n_heads, a.idx.shape[1]) > 0, \
        "lists must be split"
    idx = a.idx.copy()
    k = idx.shape[1]
    idx[:, : k // 2] = -1
    idx[3, :] = -1                                     # nothing listed
    idx[7, :] = -1
    idx[7, -3:] = a.idx[7, -3:]                        # three keys, all in the last split
    a = W.AttnInputs(a.q_bits, a.kv_bits, a.kv_slot, idx, a.scale)
    g_out, g_lse = _run_gpu(a, wl.cu_q)
    assert np.isneginf(g_lse[3]).all() and np.all(g_out[3] == 0)
    _check(a, wl.cu_q, g_out, g_lse, np.arange(wl.n_q, dtype=np.int64), oracle_mod, "empty splits")
