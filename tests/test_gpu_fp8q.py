"""fp8 x fp8 scoring: q quantised per (query, head) and the fp8 matrix cores.

1. idx_quantize_q equals the oracle's quantisation bit for bit (codes and scales), zero vectors
   and extreme magnitudes included.
2. Dense logits against the oracle's fp64 logits of the same codes (R18), on every fp8 workload
   (the 8192-query prefill batch on sampled rows), ragged batches and out-of-pool pages.
3. Top-k against the oracle under R19, and equal to the selection over the dense logits.
"""
import json
import os

import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import (by_index, check_logits, check_topk_sets, dev_inputs, gpu_store,
                           tolerance_ratio, workload)

pytestmark = pytest.mark.gpu
FP8 = W.FP8


def _q8(wl, d):
    codes, scales = ix.quantize_q(d["q"])
    return codes, scales


def test_quantize_q_bit_exact(oracle_mod):
    wl = workload(0)
    codes, scales = ix.quantize_q(wl.q_torch().cuda())
    oc, os_ = oracle_mod.quantize_q(wl.q_bits)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)
    r = np.random.default_rng(9)
    v = (r.standard_normal((300, 128)) * r.choice([1e-30, 1e-3, 1.0, 1e30], (300, 1)))
    v = v.astype(np.float32)
    v[5] = 0.0
    v[6, :] = -0.0
    qb = torch.from_numpy(v).to(torch.bfloat16)
    bits = qb.view(torch.int16).numpy().view(np.uint16).copy()
    codes, scales = ix.quantize_q(qb.cuda())
    oc, os_ = oracle_mod.quantize_q(bits)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), os_)


@pytest.mark.parametrize("cfg,n_rows", [(0, None), (2, None), (3, 1024), (4, None)])
def test_dense_fp8q_vs_oracle(oracle_mod, cfg, n_rows):
    wl = workload(cfg)
    print(f"fp8q dense cfg{cfg}", flush=True)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP8, d)
    codes, scales = _q8(wl, d)
    dense = ix.logits_dense_fp8q(codes, scales, d["w"], pool, d["page_table"], d["seq_lens"],
                                 d["cu_q"], wl.max_keys).cpu().numpy()
    rows = np.arange(wl.n_q) if n_rows is None else np.unique(np.concatenate(
        [[0, wl.n_q - 1], np.random.default_rng(cfg).choice(wl.n_q, n_rows - 2, replace=False)]))
    pool_o, _ = oracle_mod.store_workload(wl, FP8)
    oc, os_ = oracle_mod.quantize_q(wl.q_bits)
    o, _ = oracle_mod.logits_fp8q(oc, os_, wl.w, pool_o, wl.page_table, wl.seq_lens, wl.cu_q,
                                  rows=rows, row_len=wl.max_keys)
    err = check_logits(dense[rows], o, f"fp8q cfg{cfg}")
    ratio = tolerance_ratio(dense[rows], o)
    # the fp8 matrix cores add a product error the bf16 path does not have (about 8e-4 absolute
    # on logits up to 45); report how much of the tolerance it uses
    print(f"  max abs err {err:.3g}, max err / tolerance {ratio:.3f}", flush=True)
    _report(f"cfg{cfg}", {"rows": int(rows.size), "max_abs_err": err, "max_err_over_tol": ratio})
    assert ratio < 1.0


def _report(key, value):
    """Append to fp8q_error.json under INDEXER_REPORT_DIR (when set)."""
    path = os.environ.get("INDEXER_REPORT_DIR")
    if not path:
        return
    os.makedirs(path, exist_ok=True)
    f = os.path.join(path, "fp8q_error.json")
    data = json.load(open(f)) if os.path.exists(f) else {}
    data[key] = value
    json.dump(data, open(f, "w"), indent=1)


def test_dense_fp8q_ragged_and_bad_pages(oracle_mod):
    wl = W.make_workload("ragged-fp8q", 57, [0, 3, 4, 130, 700, 1500, 2100],
                         [0, 2, 1, 7, 33, 70, 3], 64, permute_pages=True, extra_pages=2)
    wl.page_table[4, 1] = wl.n_pages_pool + 3          # keys 64..127 of sequence 4: -inf
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP8, d)
    codes, scales = _q8(wl, d)
    dense = ix.logits_dense_fp8q(codes, scales, d["w"], pool, d["page_table"], d["seq_lens"],
                                 d["cu_q"], wl.max_keys).cpu().numpy()
    pool_o, _ = oracle_mod.store_workload(wl, FP8)
    oc, os_ = oracle_mod.quantize_q(wl.q_bits)
    o, _ = oracle_mod.logits_fp8q(oc, os_, wl.w, pool_o, wl.page_table, wl.seq_lens, wl.cu_q,
                                  row_len=wl.max_keys)
    check_logits(dense, o, "fp8q ragged")


@pytest.mark.parametrize("cfg", [0, 2, 4])
def test_topk_fp8q_vs_oracle(oracle_mod, cfg):
    wl = workload(cfg)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP8, d)
    codes, scales = _q8(wl, d)
    gi, gv = ix.logits_topk_fp8q(codes, scales, d["w"], pool, d["page_table"], d["seq_lens"],
                                 d["cu_q"], wl.k, want_values=True)
    pool_o, _ = oracle_mod.store_workload(wl, FP8)
    oc, os_ = oracle_mod.quantize_q(wl.q_bits)
    o, nv = oracle_mod.logits_fp8q(oc, os_, wl.w, pool_o, wl.page_table, wl.seq_lens, wl.cu_q)
    mean, exact = check_topk_sets(gi.cpu().numpy(), o, nv, wl.k, f"fp8q cfg{cfg}")
    print(f"  overlap={mean:.6f} exact-gap rows={exact}", flush=True)
    dense = ix.logits_dense_fp8q(codes, scales, d["w"], pool, d["page_table"], d["seq_lens"],
                                 d["cu_q"], wl.max_keys)
    nvis = torch.isfinite(dense).sum(dim=1).to(torch.int32)
    si, sv = ix.topk_rows(dense, wl.k, nvis)
    gi, gv = by_index(gi, gv)
    si, sv = by_index(si, sv)
    assert torch.equal(gi, si)
    assert torch.equal(gv.view(torch.int32), sv.view(torch.int32))
