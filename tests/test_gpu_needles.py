"""Needle recall of the top-k under fp8 vs bf16 key storage.

Needles are keys planted along a query-derived direction (3 * unit(direction) + N(0, 0.1)),
written through the same store path as every other key.  Two directions are used: the head-mean
of the query ('literal') and the w-weighted head sum ('weighted'); only the latter has a positive
expected score under a signed head weighting, so only it is a ranking invariant.

Eligible needles are the ones in the top-k of the unquantised ranking (oracle logits over the
canonical fp32 keys).  recall(X) = |eligible and in the GPU top-k with X-stored keys| / |eligible|.

Must-rank (bf16): bf16 rounding moves each key element by at most 2^-9 of itself, and ReLU is
1-Lipschitz, so a key's logit moves by at most B(s) = 2^-9 * sum_i u_i |k32_{s,i}| with
u = sum_h |w_h| |q_h|.  A needle whose unquantised logit minus 2B beats every other key's
unquantised logit plus 2B (the doubling covers fp32 accumulation) by rank k must be selected.
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
FP8, BF16 = W.FP8, W.BF16
REPORT = {}


def _bf16_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(oracle_mod, cfg, construction):
    wl = workload(cfg)
    nd = wl.needles
    x = oracle_mod.plant_needles(wl, construction)
    d = dev_inputs(wl, x)
    _, k32 = oracle_mod.store_keys(x, wl.gamma, wl.eps, wl.key_idx, wl.key_seq, wl.page_table,
                                   BF16, oracle_mod.new_pool(wl.n_pages_pool, BF16), want_k32=True)
    # canonical keys laid out [n_seq, max_keys, 128] for the unquantised ranking
    ref = np.zeros((wl.n_seq, wl.max_keys, 128), np.float32)
    ref[wl.key_seq, wl.key_idx] = k32
    rows = np.unique(nd["qrow"])
    o32, nv = oracle_mod.logits(wl.q_bits, wl.w, None, BF16, wl.page_table, wl.seq_lens, wl.cu_q,
                                rows=rows, keys_ref=ref, ref_stride=wl.max_keys)
    top32 = {}
    for j, r in enumerate(rows):
        idx, _ = oracle_mod.topk(o32[j:j + 1], wl.k, row_len=nv[j:j + 1])
        top32[int(r)] = set(int(v) for v in idx[0] if v >= 0)
    got = {}
    for dtype in (BF16, FP8):
        pool = gpu_store(ix, wl, dtype, d)
        gi, _ = ix.logits_topk(d["q"], d["w"], pool, dtype, d["page_table"], d["seq_lens"],
                               d["cu_q"], wl.k)
        got[dtype] = gi.cpu().numpy()
    elig = [(int(r), int(s)) for r, s in zip(nd["qrow"], nd["s"]) if int(s) in top32[int(r)]]
    rec = {}
    for dtype, name in ((BF16, "bf16"), (FP8, "fp8")):
        hit = sum(1 for r, s in elig if s in set(got[dtype][r].tolist()))
        rec[name] = hit / len(elig) if elig else float("nan")
    out = {"config": wl.name, "construction": construction, "needles": int(nd["s"].size),
           "eligible": len(elig), "recall_bf16": rec["bf16"], "recall_fp8": rec["fp8"],
           "gap": rec["bf16"] - rec["fp8"]}
    REPORT[f"cfg{cfg}-{construction}"] = out
    print(json.dumps(out), flush=True)
    _write_report()
    return wl, rows, o32, nv, ref, got, out


def _write_report():
    path = os.environ.get("INDEXER_REPORT_DIR")
    if path:
        os.makedirs(path, exist_ok=True)
        with open(os.path.join(path, "needle_recall.json"), "w") as f:
            json.dump(REPORT, f, indent=1)


def _must_rank_check(wl, rows, o32, nv, ref, gi_bf16):
    nd = wl.needles
    checked = 0
    for j, r in enumerate(rows):
        b = int(np.searchsorted(wl.cu_q, r, side="right") - 1)
        n = int(nv[j])
        u = np.abs(wl.w[r]).astype(np.float64) @ np.abs(_bf16_f64(wl.q_bits[r]))   # [128]
        bound = 2.0 * 2.0 ** -9 * (np.abs(ref[b, :n]).astype(np.float64) @ u)
        lo = o32[j, :n] - bound
        hi = o32[j, :n] + bound
        sel = set(gi_bf16[r].tolist())
        for s in nd["s"][nd["qrow"] == r]:
            s = int(s)
            others = np.delete(hi, s)
            if np.sum(others >= lo[s]) < wl.k:
                assert s in sel, f"needle ({r}, {s}) must be in the bf16 top-{wl.k}"
                checked += 1
    return checked


@pytest.mark.parametrize("cfg", [1, 4])
def test_needles_weighted(oracle_mod, cfg):
    wl, rows, o32, nv, ref, got, out = _run(oracle_mod, cfg, "weighted")
    checked = _must_rank_check(wl, rows, o32, nv, ref, got[BF16])
    print(f"  must-rank needles checked: {checked}", flush=True)
    assert checked > 0


@pytest.mark.parametrize("cfg", [1, 4])
def test_needles_literal(oracle_mod, cfg):
    _, _, _, _, _, _, out = _run(oracle_mod, cfg, "literal")
    assert 0.0 <= out["recall_fp8"] <= 1.0 or out["eligible"] == 0
