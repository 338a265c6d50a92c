"""The fp4 (e2m1) index-key cache: 4-bit codes, one fp32 scale per key, 68 B per key.

1. Stored bytes equal the oracle's, bit for bit: the measured workloads, plain and rotated, and
   ragged, out-of-range inputs (sentinel-filled pools compared whole).
2. Every e2m1 rounding decision: a scale-1 construction puts each code, each midpoint between
   neighbouring codes and the fp32 values next to those midpoints through the store.
3. Scoring: dense logits of oracle-written fp4 pools (every code, random scales, ragged batches)
   against the oracle's fp64 logits of the same bytes, through both scoring kernels.
4. The whole path (GPU store, score, select) against the oracle's top-k sets, and the overlap of
   the fp4 top-k with the unquantised fp32 ranking, plain and rotated (reported).
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import (check_logits, check_topk_sets, dev_inputs, gpu_store, oracle_rows,
                           workload)

pytestmark = pytest.mark.gpu
FP4 = W.FP4
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _diff_report(pool_g, pool_o):
    bad = np.nonzero(pool_g != pool_o)[0]
    pb = W.page_bytes(FP4)
    first = [(int(b // pb), int(b % pb), int(pool_g[b]), int(pool_o[b])) for b in bad[:8]]
    return f"{bad.size} bytes differ; (page, offset, gpu, oracle): {first}"


def test_fp4_page_bytes(oracle_mod):
    assert ix.page_bytes(FP4) == W.page_bytes(FP4) == oracle_mod.page_bytes(FP4) == 64 * 68


@pytest.mark.parametrize("cfg", [0, 2, 3, 4])
@pytest.mark.parametrize("rotate", [False, True])
def test_fp4_store_bit_exact(oracle_mod, cfg, rotate):
    wl = workload(cfg)
    print(f"fp4 store cfg{cfg} rotate={rotate} keys={wl.n_keys}", flush=True)
    d = dev_inputs(wl)
    pool_g = gpu_store(ix, wl, FP4, d, rotate=rotate).cpu().numpy()
    pool_o, _ = oracle_mod.store_workload(wl, FP4, hadamard=rotate)
    assert np.array_equal(pool_g, pool_o), _diff_report(pool_g, pool_o)


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("n", [1, 9, 131])
def test_fp4_store_ragged_and_out_of_range(oracle_mod, rotate, n):
    r = np.random.default_rng([57, n, int(rotate)])
    n_seq, max_pages, n_pool = 3, 3, 12
    pt = r.permutation(n_pool)[:n_seq * max_pages].astype(np.int32).reshape(n_seq, max_pages)
    pt[1, 2] = -1
    pt[2, 1] = n_pool + 5
    x = (r.standard_normal((n, 128)) * r.choice([1e-3, 1.0, 50.0], (n, 1))).astype(np.float32)
    x[0] = 0.0                                            # an all-zero key: scale 0, codes 0
    gamma = (1 + 0.1 * r.standard_normal(128)).astype(np.float32)
    key_seq = r.integers(-1, n_seq + 1, n).astype(np.int32)
    key_idx = r.integers(-2, max_pages * 64 + 3, n).astype(np.int32)
    _, first = np.unique(np.stack([key_seq, key_idx]), axis=1, return_index=True)
    keep = np.zeros(n, bool)
    keep[first] = True
    x, key_seq, key_idx = x[keep], key_seq[keep], key_idx[keep]
    dev = "cuda"
    pool = ix.new_cache(n_pool, FP4)
    ix.store_keys(torch.from_numpy(x).to(dev), torch.from_numpy(gamma).to(dev),
                  torch.from_numpy(key_idx).to(dev), torch.from_numpy(pt).to(dev), pool, FP4,
                  eps=1e-6, key_seq=torch.from_numpy(key_seq).to(dev), rotate=rotate)
    pool_o = oracle_mod.new_pool(n_pool, FP4)
    oracle_mod.store_keys(x, gamma, 1e-6, key_idx, key_seq, pt, FP4, pool_o, hadamard=rotate)
    pool_g = pool.cpu().numpy()
    assert np.array_equal(pool_g, pool_o), _diff_report(pool_g, pool_o)


def _e2m1_rounding_rows():
    """fp32 values at every e2m1 code, every midpoint and the fp32 neighbours of each midpoint,
    both signs, tiny values and signed zeros; dim 127 is +-6 so that each key's absmax is 6 and
    its scale exactly 1."""
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    m32 = np.concatenate([E2M1, mids]).astype(np.float32)
    v = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)),
                        np.nextafter(m32, np.float32(0)), [2.0 ** -30, 1e-38, 5.999999]])
    v = np.concatenate([v, -v, [0.0, -0.0]]).astype(np.float32)
    v = v[np.abs(v) <= 6]                                 # absmax stays 6
    r = np.random.default_rng(4)
    v = np.concatenate([v, r.uniform(-6, 6, 900).astype(np.float32)])
    n_rows = (v.size + 126) // 127
    flat = np.zeros(n_rows * 127, np.float32)
    flat[:v.size] = v
    rows = np.zeros((n_rows, 128), np.float32)
    rows[:, :127] = flat.reshape(n_rows, 127)
    rows[:, 127] = np.where(np.arange(n_rows) % 2 == 0, 6.0, -6.0)
    return rows


def test_fp4_store_rounding_exhaustive(oracle_mod):
    """eps = 2^80 and gamma = 2^40 make the canonical key x itself (as for the fp8 rounding test),
    so with |x|max = 6 the scale is 1 and the stored codes are e2m1(x) directly."""
    x = _e2m1_rounding_rows()
    n = x.shape[0]
    pt = np.arange(n, dtype=np.int32)[:, None]
    gamma = np.full(128, 2.0 ** 40, np.float32)
    key_idx = np.zeros(n, np.int32)
    key_seq = np.arange(n, dtype=np.int32)
    dev = "cuda"
    pool = ix.new_cache(n, FP4)
    ix.store_keys(torch.from_numpy(x).to(dev), torch.from_numpy(gamma).to(dev),
                  torch.from_numpy(key_idx).to(dev), torch.from_numpy(pt).to(dev), pool, FP4,
                  eps=2.0 ** 80, key_seq=torch.from_numpy(key_seq).to(dev))
    pool_g = pool.cpu().numpy()
    pool_o = oracle_mod.new_pool(n, FP4)
    _, k32 = oracle_mod.store_keys(x, gamma, 2.0 ** 80, key_idx, key_seq, pt, FP4, pool_o,
                                   want_k32=True)
    assert np.array_equal(pool_g, pool_o), _diff_report(pool_g, pool_o)
    assert np.array_equal(k32, x)
    pb = W.page_bytes(FP4)
    scales = np.array([pool_o[p * pb + 4096: p * pb + 4100].view(np.float32)[0] for p in range(n)])
    assert np.all(scales == 1.0), "the construction must give scale 1"
    # codes are the nearest e2m1 value, ties to the even code: checked independently of the
    # encoder, by distance to the 8 magnitudes
    codes = np.stack([pool_o[p * pb: p * pb + 64] for p in range(n)])
    nib = np.stack([codes & 15, codes >> 4], axis=2).reshape(n, 128)
    mag = E2M1[nib & 7]
    a = np.minimum(np.abs(x.astype(np.float64)), 6.0)
    dist = np.abs(a[..., None] - E2M1)
    best = dist.min(axis=2)
    assert np.array_equal(np.abs(a - mag), best)
    tie = (dist == best[..., None]).sum(axis=2) > 1
    assert np.all((nib[tie] & 1) == 0), "ties go to the even code"
    assert np.array_equal(nib >> 3, np.signbit(k32).astype(nib.dtype))


def _pool_from_codes(r, n_pages, zero_scales=4):
    pb = W.page_bytes(FP4)
    pool = np.zeros(n_pages * pb, np.uint8)
    for p in range(n_pages):
        codes = r.integers(0, 256, 64 * 64).astype(np.uint8)
        if p == 0:
            codes[:256] = np.arange(256, dtype=np.uint8)    # every pair of codes, -0 included
        scales = np.exp(r.uniform(-6, 3, 64)).astype(np.float32)
        if p == 0:
            scales[:zero_scales] = 0.0
        pool[p * pb: p * pb + 4096] = codes
        pool[p * pb + 4096: (p + 1) * pb] = scales.view(np.uint8)
    return pool


@pytest.mark.parametrize("q_len", [5, 1100])
def test_fp4_every_code(oracle_mod, q_len):
    """Random code bytes (every code in both nibbles) and random scales, zero included: the
    widening to bf16 must be exact for every code, through the decode-shaped kernel (few rows)
    and the prefill-shaped one (1024 rows or more)."""
    r = np.random.default_rng([13, q_len])
    wl = W.make_workload("codes", 14, [4 * 512], [q_len], 8, permute_pages=True, dtypes=(FP4,))
    pool = _pool_from_codes(r, wl.n_pages_pool)
    d = dev_inputs(wl)
    g = ix.logits_dense(d["q"], d["w"], torch.from_numpy(pool).cuda(), FP4, d["page_table"],
                        d["seq_lens"], d["cu_q"], wl.max_keys).cpu().numpy()
    o, _ = oracle_rows(oracle_mod, wl, pool, FP4, None)
    check_logits(g, o, "fp4 codes")


@pytest.mark.parametrize("cfg,n_rows", [(0, None), (2, None), (3, 24), (4, 8)])
def test_fp4_dense_logits(oracle_mod, cfg, n_rows):
    wl = workload(cfg)
    print(f"fp4 dense cfg{cfg}", flush=True)
    pool, _ = oracle_mod.store_workload(wl, FP4)
    d = dev_inputs(wl)
    g = ix.logits_dense(d["q"], d["w"], torch.from_numpy(pool).cuda(), FP4, d["page_table"],
                        d["seq_lens"], d["cu_q"], wl.max_keys)
    if n_rows is None:
        rows = np.arange(wl.n_q)
    else:
        rows = np.unique(np.concatenate([[0, wl.n_q - 1], np.random.default_rng(cfg).choice(
            wl.n_q, n_rows - 2, replace=False)]))
    o, _ = oracle_rows(oracle_mod, wl, pool, FP4, rows)
    check_logits(g[torch.from_numpy(rows).cuda()].cpu().numpy(), o, f"fp4 cfg{cfg}")


@pytest.mark.parametrize("max_keys_delta", [0, 37, -100])
def test_fp4_dense_ragged_batch(oracle_mod, max_keys_delta):
    wl = W.make_workload("ragged", 902, [0, 3, 4, 130, 700, 1500], [0, 2, 1, 7, 33, 70], 16,
                         permute_pages=True, extra_pages=3, dtypes=(FP4,))
    wl.page_table[4, 2] = -1
    wl.page_table[5, 3] = wl.n_pages_pool + 2
    pool, _ = oracle_mod.store_workload(wl, FP4)
    mk = wl.max_keys + max_keys_delta
    d = dev_inputs(wl)
    g = ix.logits_dense(d["q"], d["w"], torch.from_numpy(pool).cuda(), FP4, d["page_table"],
                        d["seq_lens"], d["cu_q"], mk).cpu().numpy()
    o, nv = oracle_rows(oracle_mod, wl, pool, FP4, None, row_len=mk)
    check_logits(g, o, "fp4 ragged")
    assert nv.min() == 0 and nv.max() > 64


@pytest.mark.parametrize("cfg,n_rows", [(0, None), (2, None), (3, 48), (4, None)])
def test_fp4_logits_topk_vs_oracle(oracle_mod, cfg, n_rows):
    """The whole path on an fp4 cache: GPU store, then score + select on the GPU."""
    wl = workload(cfg)
    print(f"fp4 topk cfg{cfg}", flush=True)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP4, d)
    gi, _ = ix.logits_topk(d["q"], d["w"], pool, FP4, d["page_table"], d["seq_lens"], d["cu_q"],
                           wl.k)
    gi = gi.cpu().numpy()
    if n_rows is None:
        rows = np.arange(wl.n_q)
    else:
        rows = np.unique(np.concatenate([[0, wl.n_q - 1], np.random.default_rng(cfg).choice(
            wl.n_q, n_rows - 2, replace=False)]))
    pool_o, _ = oracle_mod.store_workload(wl, FP4)
    o, nv = oracle_rows(oracle_mod, wl, pool_o, FP4, rows)
    mean, exact = check_topk_sets(gi[rows], o, nv, wl.k, f"fp4 cfg{cfg}")
    print(f"  rows={rows.size} overlap={mean:.6f} exact-gap rows={exact}", flush=True)


def test_fp4_logits_topk_ragged(oracle_mod):
    wl = W.make_workload("ragged", 33, [0, 3, 4, 130, 700, 1500, 2100], [0, 2, 1, 7, 33, 70, 3],
                         64, permute_pages=True, extra_pages=2, dtypes=(FP4,))
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, FP4, d)
    gi, gv = ix.logits_topk(d["q"], d["w"], pool, FP4, d["page_table"], d["seq_lens"], d["cu_q"],
                            wl.k, want_values=True)
    pool_o, _ = oracle_mod.store_workload(wl, FP4)
    o, nv = oracle_rows(oracle_mod, wl, pool_o, FP4, None)
    gi, gv = gi.cpu().numpy(), gv.cpu().numpy()
    check_topk_sets(gi, o, nv, wl.k, "fp4 ragged")
    for r in range(wl.n_q):
        m = min(wl.k, int(nv[r]))
        assert np.all(np.isneginf(gv[r, m:]))
        assert np.allclose(gv[r, :m], o[r, gi[r, :m]], rtol=2e-3, atol=1e-3)


@pytest.mark.parametrize("cfg", [2, 4])
def test_fp4_overlap_with_fp32_ranking(oracle_mod, cfg):
    """Storage-precision effect of the fp4 cache, plain and rotated: the mean overlap of its
    top-k with the top-k of the unquantised fp32 ranking (rotation keeps q.k, so one ranking
    serves both).  Reported; the bar only rules out a broken path (chance overlap is k / keys,
    at most 0.13 here)."""
    wl = workload(cfg)
    d = dev_inputs(wl)
    _, k32 = oracle_mod.store_workload(wl, FP4, want_k32=True)
    ref = np.zeros((wl.n_seq, wl.max_keys, 128), np.float32)
    ref[wl.key_seq, wl.key_idx] = k32
    o_ref, nv = oracle_mod.logits(wl.q_bits, wl.w, None, FP4, wl.page_table, wl.seq_lens,
                                  wl.cu_q, keys_ref=ref, ref_stride=wl.max_keys)
    qr = ix.rotate_q(d["q"])
    overlaps = {}
    for rot in (False, True):
        pool = gpu_store(ix, wl, FP4, d, rotate=rot)
        gi, _ = ix.logits_topk(qr if rot else d["q"], d["w"], pool, FP4, d["page_table"],
                               d["seq_lens"], d["cu_q"], wl.k)
        gi = gi.cpu().numpy()
        ov = []
        for r in range(wl.n_q):
            m = min(wl.k, int(nv[r]))
            ref_set = np.argsort(-o_ref[r, :nv[r]], kind="stable")[:m]
            ov.append(np.intersect1d(gi[r, :m], ref_set).size / max(m, 1))
        overlaps[rot] = float(np.mean(ov))
    print(f"  fp4 top-{wl.k} overlap with the fp32 ranking ({wl.name}): plain "
          f"{overlaps[False]:.5f}, rotated {overlaps[True]:.5f}", flush=True)
    assert overlaps[False] > 0.5 and overlaps[True] > 0.5
