"""S2 parity: head-reduced logits from the HIP scoring kernel against the fp64 oracle.

The GPU scores the oracle-written pool (so this isolates the scoring kernel from the store) and
must agree with the oracle's logits of the same stored bytes to |d| <= 1e-3 + 2e-3 |oracle|,
with -inf at exactly the positions the oracle marks invisible.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import by_index, check_logits, dev_inputs, gpu_store, oracle_rows, workload

pytestmark = pytest.mark.gpu
FP8, BF16 = W.FP8, W.BF16


def _oracle_pool(oracle_mod, wl, dtype):
    pool, _ = oracle_mod.store_workload(wl, dtype)
    return pool


def _dense(wl, d, pool_np, dtype, max_keys=None):
    pool = torch.from_numpy(pool_np).cuda()
    mk = wl.max_keys if max_keys is None else max_keys
    return ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"], d["cu_q"],
                           mk)


@pytest.mark.parametrize("cfg,dtype", [(0, FP8), (1, BF16), (1, FP8), (2, FP8), (2, BF16)])
def test_dense_logits_all_rows(oracle_mod, cfg, dtype):
    wl = workload(cfg)
    print(f"dense cfg{cfg} dtype={dtype} rows={wl.n_q}", flush=True)
    pool = _oracle_pool(oracle_mod, wl, dtype)
    g = _dense(wl, dev_inputs(wl), pool, dtype).cpu().numpy()
    o, _ = oracle_rows(oracle_mod, wl, pool, dtype, None)
    check_logits(g, o, f"cfg{cfg}")


@pytest.mark.parametrize("cfg,dtype,stride", [(3, BF16, 8), (4, FP8, 1), (4, BF16, 1)])
def test_dense_logits_sampled_rows(oracle_mod, cfg, dtype, stride):
    """Full-size batch on the GPU; the oracle recomputes every stride-th row and the last one
    (1,025 of the long prefill chunk's 8,192 rows; every row of the 32-row decode batch)."""
    wl = workload(cfg)
    rows = np.unique(np.concatenate([np.arange(0, wl.n_q, stride), [wl.n_q - 1]]))
    print(f"dense cfg{cfg} dtype={dtype} rows {rows.size} of {wl.n_q}", flush=True)
    pool = _oracle_pool(oracle_mod, wl, dtype)
    g = _dense(wl, dev_inputs(wl), pool, dtype)
    o, _ = oracle_rows(oracle_mod, wl, pool, dtype, rows)
    check_logits(g[torch.from_numpy(rows).cuda()].cpu().numpy(), o, f"cfg{cfg}")


def _ragged(seed, dtype):
    seq_lens = [0, 3, 4, 130, 700, 1500]
    q_lens = [0, 2, 1, 7, 33, 70]
    wl = W.make_workload("ragged", seed, seq_lens, q_lens, 16, permute_pages=True, extra_pages=3,
                         dtypes=(dtype,))
    return wl


@pytest.mark.parametrize("dtype", [FP8, BF16])
@pytest.mark.parametrize("max_keys_delta", [0, 37, -100])
def test_dense_ragged_batch(oracle_mod, dtype, max_keys_delta):
    """Several sequences with empty, tiny and ragged lengths, queries before the first key, a
    page-table hole and a page id beyond the pool (its keys score -inf), output width wider and
    narrower than the table."""
    wl = _ragged(900 + dtype, dtype)
    wl.page_table[4, 2] = -1
    wl.page_table[5, 3] = wl.n_pages_pool + 2
    pool = _oracle_pool(oracle_mod, wl, dtype)
    mk = wl.max_keys + max_keys_delta
    g = _dense(wl, dev_inputs(wl), pool, dtype, max_keys=mk).cpu().numpy()
    o, nv = oracle_rows(oracle_mod, wl, pool, dtype, None, row_len=mk)
    check_logits(g, o, "ragged")
    assert nv.min() == 0 and nv.max() > 64


def test_fp8_every_code(oracle_mod):
    """A pool of random e4m3 codes (all 254 finite codes, subnormals included) and random
    scales, zero included: widening to bf16 must be exact for every code."""
    r = np.random.default_rng(11)
    n_pages = 8
    pb = W.page_bytes(FP8)
    pool = np.zeros(n_pages * pb, np.uint8)
    codes = r.integers(0, 256, (n_pages, 64 * 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = np.exp(r.uniform(-8, 3, (n_pages, 64))).astype(np.float32)
    scales[0, :4] = 0.0
    for p in range(n_pages):
        pool[p * pb: p * pb + 8192] = codes[p]
        pool[p * pb + 8192: (p + 1) * pb] = scales[p].view(np.uint8)
    codes[0, :256] = np.arange(256, dtype=np.uint8)
    codes[0, 0x7F] = codes[0, 0xFF] = 0x01
    pool[0:256] = codes[0, :256]
    wl = W.make_workload("codes", 12, [4 * 512], [5], 8, permute_pages=True, dtypes=(FP8,))
    assert wl.n_pages_pool == n_pages
    g = _dense(wl, dev_inputs(wl), pool, FP8).cpu().numpy()
    o, _ = oracle_rows(oracle_mod, wl, pool, FP8, None)
    check_logits(g, o, "fp8 codes")


def test_dense_repeatable(oracle_mod):
    wl = workload(2)
    pool = _oracle_pool(oracle_mod, wl, FP8)
    d = dev_inputs(wl)
    a = _dense(wl, d, pool, FP8)
    b = _dense(wl, d, pool, FP8)
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape,dtype", [("decode", FP8), ("decode", BF16), ("decode", W.FP4),
                                         ("prefill", BF16), ("prefill", FP8)])
def test_page_placement_invariance(shape, dtype):
    """The same keys stored through two page tables, one a random relabelling of the other's
    pages, give bit-identical logits and selections: a score depends on the key's bytes, never on
    where its page sits in the pool.  Decode rows go through the split kernel, the 1100-row
    prefill batch through the rows kernels."""
    if shape == "decode":
        wl = W.make_workload("placement-decode", 70, [20000, 9000, 33000, 4100], [1, 1, 1, 1],
                             512, permute_pages=True, extra_pages=2, dtypes=(dtype,))
    else:
        wl = W.make_workload("placement-prefill", 71, [9000, 6000], [700, 400], 512,
                             permute_pages=True, extra_pages=2, dtypes=(dtype,))
    d1 = dev_inputs(wl)
    relabel = np.random.default_rng(72).permutation(wl.n_pages_pool).astype(np.int32)
    pt2 = wl.page_table.copy()
    ok = (pt2 >= 0) & (pt2 < wl.n_pages_pool)
    pt2[ok] = relabel[pt2[ok]]
    assert not np.array_equal(pt2, wl.page_table)
    d2 = dict(d1)
    d2["page_table"] = torch.from_numpy(pt2).cuda()
    out = []
    for d in (d1, d2):
        pool = gpu_store(ix, wl, dtype, d)
        dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                                d["cu_q"], wl.max_keys)
        gi, gv = ix.logits_topk(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                                d["cu_q"], wl.k, want_values=True)
        out.append((dense, *by_index(gi, gv)))
    (a, ai, av), (b, bi, bv) = out
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(ai, bi)
    assert torch.equal(av.view(torch.int32), bv.view(torch.int32))
