"""Shared test helpers: moving seeded workloads to the GPU, running both sides, comparing."""
from __future__ import annotations

import functools
import re
import os

import numpy as np
import torch

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")

# logit tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle| (fp32 accumulation vs fp64)
RTOL, ATOL = 2e-3, 1e-3


def header_functions():
    """Names of the functions include/dsa_indexer.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", text)))


def query_positions(wl) -> np.ndarray:
    """Token position t of every query row: the queries of sequence b are its last q_len_b
    tokens, t = L_b - q_len_b + i."""
    t = np.empty(wl.n_q, dtype=np.int64)
    cu = wl.cu_q
    for b in range(wl.n_seq):
        ql = int(wl.q_lens[b])
        t[cu[b]:cu[b + 1]] = int(wl.seq_lens[b]) - ql + np.arange(ql)
    return t


@functools.lru_cache(maxsize=None)
def workload(cfg: int):
    return W.CONFIGS[cfg]()


def dev_inputs(wl, x=None, device="cuda"):
    """Upload a workload's arrays (x may be replaced, e.g. by a needle-planted copy)."""
    x = wl.x if x is None else x
    return {
        "x": torch.from_numpy(np.ascontiguousarray(x)).to(device),
        "gamma": torch.from_numpy(wl.gamma).to(device),
        "key_idx": torch.from_numpy(wl.key_idx).to(device),
        "key_seq": torch.from_numpy(wl.key_seq).to(device),
        "page_table": torch.from_numpy(wl.page_table).to(device),
        "seq_lens": torch.from_numpy(wl.seq_lens).to(device),
        "cu_q": torch.from_numpy(wl.cu_q).to(device),
        "q": wl.q_torch().to(device),
        "w": torch.from_numpy(wl.w).to(device),
    }


def gpu_store(ix, wl, dtype, d, mask=None, pool=None, rotate=False):
    if pool is None:
        pool = ix.new_cache(wl.n_pages_pool, dtype)
    if mask is None:
        ix.store_keys(d["x"], d["gamma"], d["key_idx"], d["page_table"], pool, dtype,
                      eps=wl.eps, key_seq=d["key_seq"], rotate=rotate)
    else:
        m = torch.from_numpy(np.nonzero(mask)[0]).to(d["x"].device)
        ix.store_keys(d["x"][m].contiguous(), d["gamma"], d["key_idx"][m].contiguous(),
                      d["page_table"], pool, dtype, eps=wl.eps,
                      key_seq=d["key_seq"][m].contiguous(), rotate=rotate)
    return pool


def check_logits(gpu_rows: np.ndarray, ora_rows: np.ndarray, what: str):
    """Elementwise: finite pattern identical, finite values within tolerance."""
    fin_o = np.isfinite(ora_rows)
    fin_g = np.isfinite(gpu_rows)
    assert np.array_equal(fin_o, fin_g), f"{what}: visibility pattern differs"
    assert np.all(np.isneginf(gpu_rows[~fin_g])), f"{what}: invisible entries must be -inf"
    g = gpu_rows[fin_o].astype(np.float64)
    o = ora_rows[fin_o]
    err = np.abs(g - o)
    bad = err > ATOL + RTOL * np.abs(o)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} logits out of tolerance, "
                           f"max err {err.max():.3g}")
    return float(err.max()) if err.size else 0.0


def tolerance_ratio(gpu_rows: np.ndarray, ora_rows: np.ndarray) -> float:
    """Largest |gpu - oracle| / (ATOL + RTOL |oracle|) over the finite entries: how much of the
    logit tolerance the worst entry uses (check_logits requires it to stay within 1)."""
    fin = np.isfinite(ora_rows)
    if not fin.any():
        return 0.0
    o = ora_rows[fin]
    return float(np.max(np.abs(gpu_rows[fin].astype(np.float64) - o) / (ATOL + RTOL * np.abs(o))))


def check_topk_sets(gpu_idx: np.ndarray, ora_logits: np.ndarray, n_vis: np.ndarray, k: int,
                    what: str, min_overlap: float = 0.999):
    """Top-k sets against fp64 oracle logits.

    Per row: padding is exact and the indices distinct; where the oracle's k-th / (k+1)-th gap exceeds the
    logit tolerance the set matches exactly; everywhere, each selected key is within twice the
    tolerance of the oracle's k-th value and no unselected key beats the selection by more than
    that.  Over all rows the mean overlap with the oracle's set is >= min_overlap.
    """
    overlaps = []
    n_exact_rows = 0
    for r in range(gpu_idx.shape[0]):
        nv = int(n_vis[r])
        row = ora_logits[r, :nv]
        g = gpu_idx[r]
        m = min(k, nv)
        assert np.all(g[m:] == -1), f"{what} row {r}: padding"
        sel = np.sort(g[:m])   # the order within a row is unspecified
        assert np.all(np.diff(sel) > 0), f"{what} row {r}: indices must be distinct"
        assert sel.size == 0 or (sel.min() >= 0 and sel.max() < nv), f"{what} row {r}: range"
        if nv <= k:
            assert np.array_equal(sel, np.arange(nv)), f"{what} row {r}: short row"
            overlaps.append(1.0)
            continue
        order = np.lexsort((np.arange(nv), -row))
        o_set = np.sort(order[:k])
        sk, sk1 = row[order[k - 1]], row[order[k]]
        tol = ATOL + RTOL * abs(sk)
        if sk - sk1 > tol:
            assert np.array_equal(sel, o_set), f"{what} row {r}: set differs despite a clear gap"
            n_exact_rows += 1
        assert row[sel].min() >= sk - 2 * tol, f"{what} row {r}: a selected key is too low"
        mask = np.ones(nv, bool)
        mask[sel] = False
        if mask.any():
            assert row[mask].max() <= sk1 + 2 * tol, f"{what} row {r}: an unselected key is too high"
        overlaps.append(np.intersect1d(sel, o_set).size / k)
    mean = float(np.mean(overlaps)) if overlaps else 1.0
    assert mean >= min_overlap, f"{what}: mean overlap {mean:.5f}"
    return mean, n_exact_rows


def oracle_rows(oracle, wl, pool, dtype, rows, row_len=None, q_bits=None):
    return oracle.logits(wl.q_bits if q_bits is None else q_bits, wl.w, pool, dtype,
                         wl.page_table, wl.seq_lens, wl.cu_q, rows=rows, row_len=row_len)


def by_index(idx: torch.Tensor, val: torch.Tensor = None):
    """Top-k rows reordered by index, padding (-1) last: the order within a row is unspecified,
    so two selections are compared in this form."""
    key = torch.where(idx < 0, torch.iinfo(torch.int32).max, idx)
    order = torch.sort(key, dim=1, stable=True).indices
    si = torch.gather(idx, 1, order)
    return si if val is None else (si, torch.gather(val, 1, order))
