"""S1 parity: stored cache bytes from the HIP store kernel equal the oracle's, bit for bit.

Pools start filled with a 0xA5 sentinel on both sides and are compared whole, so a stray write
anywhere in the pool fails the test as well as a wrong byte in a stored key.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_rmsnorm_amd as ix
import workloads as W
from tests.helpers import dev_inputs, gpu_store, workload

pytestmark = pytest.mark.gpu
FP8, BF16 = W.FP8, W.BF16


def _compare(pool_g: np.ndarray, pool_o: np.ndarray, dtype: int, what: str):
    bad = np.nonzero(pool_g != pool_o)[0]
    if bad.size:
        pb = W.page_bytes(dtype)
        first = [(int(b // pb), int(b % pb), int(pool_g[b]), int(pool_o[b])) for b in bad[:8]]
        raise AssertionError(f"{what}: {bad.size} bytes differ; (page, offset, gpu, oracle): {first}")


def _x_for(wl, oracle_mod):
    return oracle_mod.plant_needles(wl, "weighted") if wl.needles else wl.x


@pytest.mark.parametrize("cfg,dtype", [(0, FP8), (1, BF16), (1, FP8), (2, FP8), (2, BF16),
                                       (3, BF16), (4, FP8), (4, BF16)])
def test_store_bit_exact(oracle_mod, cfg, dtype):
    wl = workload(cfg)
    x = _x_for(wl, oracle_mod)
    print(f"store cfg{cfg} dtype={dtype} keys={wl.n_keys}", flush=True)
    d = dev_inputs(wl, x)
    if wl.step_keys is not None:
        # as measured: the earlier keys are stored first, the chunk's keys inside the step
        pool = gpu_store(ix, wl, dtype, d, mask=~wl.step_keys)
        gpu_store(ix, wl, dtype, d, mask=wl.step_keys, pool=pool)
    else:
        pool = gpu_store(ix, wl, dtype, d)
    pool_g = pool.cpu().numpy()
    pool_o = oracle_mod.new_pool(wl.n_pages_pool, dtype)
    oracle_mod.store_keys(x, wl.gamma, wl.eps, wl.key_idx, wl.key_seq, wl.page_table, dtype, pool_o)
    _compare(pool_g, pool_o, dtype, f"cfg{cfg}")


def _run_both(oracle_mod, x, gamma, eps, key_idx, key_seq, pt, dtype, n_pool):
    dev = "cuda"
    pool = ix.new_cache(n_pool, dtype)
    ix.store_keys(torch.from_numpy(x).to(dev), torch.from_numpy(gamma).to(dev),
                  torch.from_numpy(key_idx).to(dev), torch.from_numpy(pt).to(dev), pool, dtype,
                  eps=eps, key_seq=None if key_seq is None else torch.from_numpy(key_seq).to(dev))
    pool_o = oracle_mod.new_pool(n_pool, dtype)
    oracle_mod.store_keys(x, gamma, eps, key_idx, key_seq, pt, dtype, pool_o)
    return pool.cpu().numpy(), pool_o


@pytest.mark.parametrize("dtype", [FP8, BF16])
@pytest.mark.parametrize("n", [1, 7, 9, 64, 131])
def test_store_ragged_and_out_of_range(oracle_mod, dtype, n):
    r = np.random.default_rng([55, n, dtype])
    n_seq, max_pages, n_pool = 3, 3, 12
    pt = r.permutation(n_pool)[:n_seq * max_pages].astype(np.int32).reshape(n_seq, max_pages)
    pt[1, 2] = -1                      # a hole in the table
    pt[2, 1] = n_pool + 5              # a page beyond the pool
    x = (r.standard_normal((n, 128)) * r.choice([1e-3, 1.0, 50.0], (n, 1))).astype(np.float32)
    gamma = (1 + 0.1 * r.standard_normal(128)).astype(np.float32)
    key_seq = r.integers(-1, n_seq + 1, n).astype(np.int32)        # some out of range
    key_idx = r.integers(-2, max_pages * 64 + 3, n).astype(np.int32)
    # distinct slots so that no two rows race on one slot
    _, first = np.unique(np.stack([key_seq, key_idx]), axis=1, return_index=True)
    keep = np.zeros(n, bool)
    keep[first] = True
    x, key_seq, key_idx = x[keep], key_seq[keep], key_idx[keep]
    pg, po = _run_both(oracle_mod, x, gamma, 1e-6, key_idx, key_seq, pt, dtype, n_pool)
    assert np.array_equal(pg, po)


@pytest.mark.parametrize("dtype", [FP8, BF16])
def test_store_zero_keys_and_null_seq(oracle_mod, dtype):
    x = np.zeros((3, 128), np.float32)
    x[1] = np.random.default_rng(1).standard_normal(128)
    pt = np.array([[1, 0]], np.int32)
    pg, po = _run_both(oracle_mod, x, np.ones(128, np.float32), 1e-6,
                       np.array([0, 70, 5], np.int32), None, pt, dtype, 2)
    assert np.array_equal(pg, po)
    pool = ix.new_cache(2, dtype)
    ix.store_keys(torch.zeros((0, 128), device="cuda"), torch.ones(128, device="cuda"),
                  torch.zeros(0, dtype=torch.int32, device="cuda"),
                  torch.from_numpy(pt).cuda(), pool, dtype)
    assert bool((pool == 0xA5).all())


def _rounding_rows():
    """fp32 values that probe every e4m3 rounding decision and many bf16 ties: all codes, all
    midpoints between neighbouring codes and the fp32 values next to them, both signs."""
    mags = np.array([oracle_dec(c) for c in range(127)])
    mids = (mags[:-1] + mags[1:]) / 2
    vals = [mags, mids]
    m32 = mids.astype(np.float32)
    vals += [np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))]
    v = np.concatenate([np.asarray(a, np.float64) for a in vals])
    v = np.concatenate([v, -v, [-0.0, 2.0 ** -12, -(2.0 ** -12), 447.9, -447.9]])
    v = v[np.abs(v) <= 448].astype(np.float32)
    r = np.random.default_rng(3)
    # bf16 ties (low 16 bits exactly 0x8000) in a range that keeps |v| <= 448
    ties = ((r.integers(0x3A00, 0x43E0, 600).astype(np.uint32) << 16) | 0x8000)
    ties |= (r.integers(0, 2, 600).astype(np.uint32) << 31)
    v = np.concatenate([v, ties.view(np.float32)])
    n_rows = (v.size + 126) // 127
    rows = np.zeros((n_rows, 128), np.float32)
    flat = np.zeros(n_rows * 127, np.float32)
    flat[:v.size] = v
    rows[:, :127] = flat.reshape(n_rows, 127)
    rows[:, 127] = np.where(np.arange(n_rows) % 2 == 0, 448.0, -448.0)   # amax 448 => scale 1
    return rows


def oracle_dec(c):
    e, m = (c >> 3) & 15, c & 7
    return 2.0 ** -6 * m / 8 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)


@pytest.mark.parametrize("dtype", [FP8, BF16])
def test_store_rounding_exhaustive(oracle_mod, dtype):
    """With eps = 2^80 the mean square vanishes next to eps in fp64, so the RMSNorm factor is
    exactly 2^-40; gamma = 2^40 undoes it and key 0 has no rotation, so the canonical key is x
    itself.  With |x|max = 448 the fp8 scale is exactly 1 and the codes are e4m3(x)."""
    x = _rounding_rows()
    n = x.shape[0]
    pt = np.arange(n, dtype=np.int32)[:, None]            # one page per sequence
    gamma = np.full(128, 2.0 ** 40, np.float32)
    key_idx = np.zeros(n, np.int32)
    key_seq = np.arange(n, dtype=np.int32)
    pg, po = _run_both(oracle_mod, x, gamma, 2.0 ** 80, key_idx, key_seq, pt, dtype, n)
    assert np.array_equal(pg, po)
    # the canonical key equals x in value (a zero in the rotated half may change sign:
    # -0 * cos 0 - (negative * sin 0) = +0)
    _, k32 = oracle_mod.store_keys(x, gamma, 2.0 ** 80, key_idx, key_seq, pt, dtype,
                                   oracle_mod.new_pool(n, dtype), want_k32=True)
    assert np.array_equal(k32, x)
    pb = W.page_bytes(dtype)
    if dtype == FP8:
        scales = np.array([po[p * pb + 8192: p * pb + 8196].view(np.float32)[0] for p in range(n)])
        assert np.all(scales == 1.0), "the construction must give scale 1"
        codes = np.concatenate([po[p * pb: p * pb + 127] for p in range(n)])
        want = torch.from_numpy(np.ascontiguousarray(k32[:, :127]).ravel()).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, want)
    else:
        bits = np.concatenate([po[p * pb: p * pb + 256].view(np.uint16)[:127] for p in range(n)])
        want = torch.from_numpy(np.ascontiguousarray(k32[:, :127]).ravel()).to(
            torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(bits, want.view(np.uint16))


def test_store_repeatable():
    wl = workload(2)
    d = dev_inputs(wl)
    a = gpu_store(ix, wl, FP8, d)
    b = gpu_store(ix, wl, FP8, d)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,rotate", [(FP8, False), (BF16, False), (W.FP4, False),
                                          (FP8, True)])
def test_store_far_positions(oracle_mod, dtype, rotate):
    """Keys at positions that reach every part of the RoPE angle (key index s = m0 + 256 m1 +
    65536 m2, each part's cosine and sine combined by angle addition) and past 2^24 keys (the
    direct sincos): the boundaries of every part, and 3000 keys spread up to 2^24 + 2^15, stored
    bit-identical to the oracle's cos and sin of the whole angle."""
    r = np.random.default_rng([77, dtype, int(rotate)])
    edges = [0, 1, 2, 255, 256, 257, 511, 65535, 65536, 65537, 131071, 1 << 20, (1 << 20) + 77,
             (1 << 23) + 5, (1 << 24) - 1, 1 << 24, (1 << 24) + 1, (1 << 24) + 300]
    key_idx = np.unique(np.concatenate([edges, r.integers(0, (1 << 24) + (1 << 15), 3000)]))
    key_idx = key_idx.astype(np.int32)
    max_pages = ((1 << 24) + (1 << 15)) // 64
    pages = np.unique(key_idx // 64)
    pt = np.full((1, max_pages), -1, np.int32)
    pt[0, pages] = r.permutation(pages.size).astype(np.int32)
    x = (r.standard_normal((key_idx.size, 128)) * r.choice([1e-2, 1.0, 30.0],
                                                           (key_idx.size, 1))).astype(np.float32)
    gamma = (1 + 0.1 * r.standard_normal(128)).astype(np.float32)
    dev = "cuda"
    pool = ix.new_cache(pages.size, dtype)
    ix.store_keys(torch.from_numpy(x).to(dev), torch.from_numpy(gamma).to(dev),
                  torch.from_numpy(key_idx).to(dev), torch.from_numpy(pt).to(dev), pool, dtype,
                  eps=1e-6, rotate=rotate)
    pool_o = oracle_mod.new_pool(pages.size, dtype)
    oracle_mod.store_keys(x, gamma, 1e-6, key_idx, None, pt, dtype, pool_o, hadamard=rotate)
    _compare(pool.cpu().numpy(), pool_o, dtype, f"far positions dtype={dtype} rotate={rotate}")
