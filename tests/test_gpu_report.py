"""Accuracy figures of the whole path, per workload and cache dtype (reported, with sanity bars).

For each workload: the largest logit error against the fp64 oracle on the same stored bytes
(dense logits, every row or a row sample), the fraction of rows whose top-k set equals the
oracle's exactly and the mean overlap with it, and the "background" overlap of the top-k from
the quantised cache with the top-k of the unquantised ranking (oracle logits over the canonical
fp32 keys): the storage-precision effect, measured without a model.  Written to
$INDEXER_REPORT_DIR/accuracy_report.json when that is set.
"""
import json
import os

import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import dev_inputs, gpu_store, workload

pytestmark = pytest.mark.gpu
FP8, BF16, FP4 = W.FP8, W.BF16, W.FP4
REPORT = {}


def _write():
    path = os.environ.get("INDEXER_REPORT_DIR")
    if path:
        os.makedirs(path, exist_ok=True)
        with open(os.path.join(path, "accuracy_report.json"), "w") as f:
            json.dump(REPORT, f, indent=1)


def _topk_sets(scores, nv, k, oracle_mod):
    idx, _ = oracle_mod.topk(scores, k, row_len=nv)
    return [set(int(v) for v in row if v >= 0) for row in idx]


@pytest.mark.parametrize("cfg", [0, 2, 3, 4])
def test_accuracy_report(oracle_mod, cfg):
    wl = workload(cfg)
    print(f"accuracy cfg{cfg} ({wl.name})", flush=True)
    rows = np.arange(wl.n_q) if wl.n_q <= 256 else np.unique(np.concatenate(
        [[0, wl.n_q - 1], np.random.default_rng(cfg).choice(wl.n_q, 62, replace=False)]))
    d = dev_inputs(wl)
    _, k32 = oracle_mod.store_workload(wl, BF16, want_k32=True)
    ref = np.zeros((wl.n_seq, wl.max_keys, 128), np.float32)
    ref[wl.key_seq, wl.key_idx] = k32
    o32, nv = oracle_mod.logits(wl.q_bits, wl.w, None, BF16, wl.page_table, wl.seq_lens, wl.cu_q,
                                rows=rows, keys_ref=ref, ref_stride=wl.max_keys)
    top32 = _topk_sets(o32, nv, wl.k, oracle_mod)
    rt = torch.from_numpy(rows).cuda()
    for dtype, name in ((BF16, "bf16"), (FP8, "fp8"), (FP4, "fp4")):
        pool = gpu_store(ix, wl, dtype, d)
        dense = ix.logits_dense(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                                d["cu_q"], wl.max_keys)[rt].cpu().numpy()
        gi, _ = ix.logits_topk(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                               d["cu_q"], wl.k)
        gi = gi.cpu().numpy()[rows]
        pool_o, _ = oracle_mod.store_workload(wl, dtype)
        o, _ = oracle_mod.logits(wl.q_bits, wl.w, pool_o, dtype, wl.page_table, wl.seq_lens,
                                 wl.cu_q, rows=rows)
        fin = np.isfinite(o)
        err = np.abs(dense[fin].astype(np.float64) - o[fin])
        rel = err / np.maximum(np.abs(o[fin]), 1e-30)
        top_o = _topk_sets(o, nv, wl.k, oracle_mod)
        same, ov, ov32 = 0, [], []
        for j in range(rows.size):
            m = min(wl.k, int(nv[j]))
            g = set(int(v) for v in gi[j, :m])
            same += g == top_o[j]
            ov.append(len(g & top_o[j]) / max(m, 1))
            ov32.append(len(g & top32[j]) / max(m, 1))
        out = {"workload": wl.name, "kv_dtype": name, "rows": int(rows.size),
               "logit_max_abs_err": float(err.max()), "logit_max_rel_err": float(rel.max()),
               "logit_max_abs": float(np.abs(o[fin]).max()),
               "topk_exact_set_fraction": same / rows.size,
               "topk_mean_overlap_vs_oracle": float(np.mean(ov)),
               "topk_mean_overlap_vs_fp32_ranking": float(np.mean(ov32))}
        REPORT[f"{wl.name}-{name}"] = out
        print("  " + json.dumps(out), flush=True)
        _write()
        assert np.mean(ov) >= 0.999
        assert np.mean(ov32) >= {BF16: 0.99, FP8: 0.95, FP4: 0.5}[dtype]
