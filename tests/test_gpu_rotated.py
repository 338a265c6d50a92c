"""The rotated store (normalised 128-point Walsh-Hadamard transform after RoPE) and q rotation.

1. Stored bytes of the rotated store equal the oracle's, bit for bit, on the measured workloads
   and on ragged, out-of-range inputs (sentinel-filled pools compared whole).
2. q rotation equals the oracle's bit for bit, also in place.
3. The whole rotated path (rotated store, rotated q, score + select) against the oracle's fp64
   logits of the same rotated cache, as for the plain path.
4. Rotation keeps q.k: rotated logits match the plain ones within the bf16 roundings, and the
   top-k overlap of the fp8 cache with the unquantised ranking is reported with and without it.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import check_topk_sets, dev_inputs, gpu_store, oracle_rows, workload

pytestmark = pytest.mark.gpu
FP8, BF16 = W.FP8, W.BF16


def _diff_report(pool_g, pool_o):
    bad = np.nonzero(pool_g != pool_o)[0]
    return f"{bad.size} bytes differ, first at {bad[:6].tolist()}"


@pytest.mark.parametrize("cfg,dtype", [(0, FP8), (0, BF16), (2, FP8), (2, BF16), (4, FP8),
                                       (4, BF16)])
def test_rotated_store_bit_exact(oracle_mod, cfg, dtype):
    wl = workload(cfg)
    print(f"rotated store cfg{cfg} dtype={dtype} keys={wl.n_keys}", flush=True)
    d = dev_inputs(wl)
    pool_g = gpu_store(ix, wl, dtype, d, rotate=True).cpu().numpy()
    pool_o, _ = oracle_mod.store_workload(wl, dtype, hadamard=True)
    assert np.array_equal(pool_g, pool_o), _diff_report(pool_g, pool_o)
    # the rotation changes the bytes: the plain store differs
    pool_p = gpu_store(ix, wl, dtype, d).cpu().numpy()
    assert not np.array_equal(pool_p, pool_g)


@pytest.mark.parametrize("dtype", [FP8, BF16])
def test_rotated_store_ragged_and_out_of_range(oracle_mod, dtype):
    r = np.random.default_rng([91, dtype])
    n, n_seq, max_pages, n_pool = 77, 3, 3, 12
    pt = r.permutation(n_pool)[:n_seq * max_pages].astype(np.int32).reshape(n_seq, max_pages)
    pt[1, 2] = -1
    pt[2, 1] = n_pool + 5
    x = (r.standard_normal((n, 128)) * r.choice([1e-3, 1.0, 50.0], (n, 1))).astype(np.float32)
    x[3] = 0.0                                            # an all-zero key
    gamma = (1 + 0.1 * r.standard_normal(128)).astype(np.float32)
    key_seq = r.integers(-1, n_seq + 1, n).astype(np.int32)
    key_idx = r.integers(-2, max_pages * 64 + 3, n).astype(np.int32)
    _, first = np.unique(np.stack([key_seq, key_idx]), axis=1, return_index=True)
    keep = np.zeros(n, bool)
    keep[first] = True
    x, key_seq, key_idx = x[keep], key_seq[keep], key_idx[keep]
    dev = "cuda"
    pool = ix.new_cache(n_pool, dtype)
    ix.store_keys(torch.from_numpy(x).to(dev), torch.from_numpy(gamma).to(dev),
                  torch.from_numpy(key_idx).to(dev), torch.from_numpy(pt).to(dev), pool, dtype,
                  eps=1e-6, key_seq=torch.from_numpy(key_seq).to(dev), rotate=True)
    pool_o = oracle_mod.new_pool(n_pool, dtype)
    oracle_mod.store_keys(x, gamma, 1e-6, key_idx, key_seq, pt, dtype, pool_o, hadamard=True)
    pool_g = pool.cpu().numpy()
    assert np.array_equal(pool_g, pool_o), _diff_report(pool_g, pool_o)


@pytest.mark.parametrize("cfg", [0, 3])
def test_rotate_q_bit_exact(oracle_mod, cfg):
    wl = workload(cfg)
    q = wl.q_torch().cuda()
    got = ix.rotate_q(q).view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle_mod.rotate_q(wl.q_bits)
    assert np.array_equal(got, want)
    # in place, and q's dims of large and tiny magnitude
    r = np.random.default_rng(5)
    v = (r.standard_normal((300, 128)) * r.choice([1e-20, 1.0, 1e20], (300, 1))).astype(np.float32)
    qb = torch.from_numpy(v).to(torch.bfloat16)
    bits = qb.view(torch.int16).numpy().view(np.uint16).copy()
    qd = qb.cuda()
    ix.rotate_q(qd, out=qd)
    assert np.array_equal(qd.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle_mod.rotate_q(bits))


@pytest.mark.parametrize("cfg,dtype", [(0, FP8), (1, BF16), (2, FP8), (4, BF16)])
def test_rotated_path_vs_oracle(oracle_mod, cfg, dtype):
    wl = workload(cfg)
    print(f"rotated path cfg{cfg} dtype={dtype}", flush=True)
    d = dev_inputs(wl)
    pool = gpu_store(ix, wl, dtype, d, rotate=True)
    qr = ix.rotate_q(d["q"])
    gi, _ = ix.logits_topk(qr, d["w"], pool, dtype, d["page_table"], d["seq_lens"], d["cu_q"],
                           wl.k)
    pool_o, _ = oracle_mod.store_workload(wl, dtype, hadamard=True)
    o, nv = oracle_rows(oracle_mod, wl, pool_o, dtype, None, q_bits=oracle_mod.rotate_q(wl.q_bits))
    mean, exact = check_topk_sets(gi.cpu().numpy(), o, nv, wl.k, f"rotated cfg{cfg}")
    print(f"  overlap={mean:.6f} exact-gap rows={exact}", flush=True)


def test_rotation_keeps_logits_and_fp8_overlap(oracle_mod):
    """bf16 cache: rotated logits = plain logits up to the bf16 roundings of q and k.  fp8 cache:
    the top-k overlap with the unquantised fp32 ranking, plain and rotated (reported)."""
    wl = workload(0)
    d = dev_inputs(wl)
    qr = ix.rotate_q(d["q"])
    dense = {}
    for rot in (False, True):
        pool = gpu_store(ix, wl, BF16, d, rotate=rot)
        dense[rot] = ix.logits_dense(qr if rot else d["q"], d["w"], pool, BF16, d["page_table"],
                                     d["seq_lens"], d["cu_q"], wl.max_keys).cpu().numpy()
    fin = np.isfinite(dense[False])
    assert np.array_equal(fin, np.isfinite(dense[True]))
    a, b = dense[False][fin], dense[True][fin]
    assert np.max(np.abs(a - b)) <= 0.05 * np.max(np.abs(a)), "rotation must keep q.k"
    _, k32 = oracle_mod.store_workload(wl, BF16, want_k32=True)
    ref = np.zeros((wl.n_seq, wl.max_keys, 128), np.float32)
    ref[wl.key_seq, wl.key_idx] = k32
    o_ref, nv = oracle_mod.logits(wl.q_bits, wl.w, None, BF16, wl.page_table, wl.seq_lens,
                                  wl.cu_q, keys_ref=ref, ref_stride=wl.max_keys)
    overlaps = {}
    for rot in (False, True):
        pool = gpu_store(ix, wl, FP8, d, rotate=rot)
        gi, _ = ix.logits_topk(qr if rot else d["q"], d["w"], pool, FP8, d["page_table"],
                               d["seq_lens"], d["cu_q"], wl.k)
        gi = gi.cpu().numpy()
        ov = []
        for r in range(wl.n_q):
            m = min(wl.k, int(nv[r]))
            ref_set = np.argsort(-o_ref[r, :nv[r]], kind="stable")[:m]
            ov.append(np.intersect1d(gi[r, :m], ref_set).size / max(m, 1))
        overlaps[rot] = float(np.mean(ov))
    print(f"  fp8 top-{wl.k} overlap with the fp32 ranking: plain {overlaps[False]:.5f}, "
          f"rotated {overlaps[True]:.5f}", flush=True)
    assert overlaps[True] > 0.95 and overlaps[False] > 0.95
