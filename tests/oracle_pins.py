"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each pin raises AssertionError on failure.  They use closed forms, library routines (torch's CPU
float8_e4m3fn / bfloat16 casts, numpy complex arithmetic, matrix products, stable argsort) on
special cases that reduce to them, invariants of the method (scale invariance of RMSNorm, rotation
by RoPE, ReLU(d) + ReLU(-d) = |d|), brute force on tiny inputs, and the sizes the DSA indexer pages
print (tests/golden/layout.txt).  ``ALL_PINS`` is also run with planted mistakes in the oracle to
show that each mistake trips at least one pin.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle

D, H, PAGE = 128, 64, 64
FP8, BF16 = oracle.FP8, oracle.BF16
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(i):
    return np.random.default_rng([7777, i])


def _torch_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _store_rows(x, s, gamma=None, eps=1e-6, dtype=BF16):
    """Store rows of x at logical positions s of one sequence; return (pool, k32, page_table)."""
    x = np.asarray(x, np.float32)
    s = np.asarray(s, np.int32)
    gamma = np.ones(D, np.float32) if gamma is None else np.asarray(gamma, np.float32)
    max_pages = int(s.max()) // PAGE + 1
    pt = np.arange(max_pages, dtype=np.int32)[None, :]
    pool = oracle.new_pool(max_pages, dtype)
    skipped, k32 = oracle.store_keys(x, gamma, eps, s, None, pt, dtype, pool, want_k32=True)
    assert skipped == 0
    return pool, k32, pt


def _pool_keys(pool, pt, dtype, b, n):
    """Decode keys 0..n-1 of sequence b from a pool with torch's casts (an independent decoder)."""
    pb = oracle.page_bytes(dtype)
    out = np.zeros((n, D))
    for s in range(n):
        page = pt[b, s // PAGE]
        base = page * pb
        slot = s % PAGE
        if dtype == BF16:
            raw = pool[base + slot * 256: base + slot * 256 + 256].view(np.uint16)
            out[s] = _bf16_to_f64(raw)
        else:
            codes = pool[base + slot * D: base + slot * D + D]
            scale = pool[base + PAGE * D + 4 * slot: base + PAGE * D + 4 * slot + 4].view(np.float32)[0]
            out[s] = _torch_e4m3_to_f64(codes) * float(scale)
    return out


# ------------------------------------------------------------------------------------------------
# Layout sizes printed on the pages
# ------------------------------------------------------------------------------------------------

def pin_layout_sizes():
    vals = {}
    with open(os.path.join(GOLDEN, "layout.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    assert oracle.page_bytes(FP8) == vals["page_keys"] * vals["fp8_bytes_per_token"] == 8448
    assert oracle.page_bytes(BF16) == vals["page_keys"] * vals["bf16_bytes_per_token"] == 16384
    assert vals["bf16_bytes_per_token"] == 2 * vals["head_dim"]
    assert vals["fp8_bytes_per_token"] == vals["head_dim"] + 4


# ------------------------------------------------------------------------------------------------
# Number formats
# ------------------------------------------------------------------------------------------------

def pin_e4m3_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = _torch_e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def pin_e4m3_roundtrip_and_midpoints():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    dec = oracle.e4m3_decode(np.array(finite, np.uint8)).astype(np.float32)
    enc = oracle.e4m3_encode(dec)
    # -0.0 decodes to -0.0 and must come back as 0x80; everything else round-trips
    assert np.array_equal(enc, np.array(finite, np.uint8))
    mags = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(mags) > 0)
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)        # exact: <= 5 significant bits
    assert np.array_equal(mid.astype(np.float64), (mags[:-1] + mags[1:]) / 2)
    got = oracle.e4m3_encode(mid)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want), "midpoints must round to the even code"
    got_neg = oracle.e4m3_encode(-mid)
    assert np.array_equal(got_neg, want | 0x80)
    # just off the midpoints the nearest value wins
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    assert np.array_equal(oracle.e4m3_encode(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.e4m3_encode(dn), lo.astype(np.uint8))


def pin_e4m3_vs_torch_sweep():
    r = _rng(1)
    v = np.concatenate([
        r.uniform(-448, 448, 4000),
        r.standard_normal(4000) * 10.0,
        np.exp(r.uniform(np.log(1e-4), np.log(448), 4000)) * r.choice([-1, 1], 4000),
        np.linspace(-0.02, 0.02, 2001),                  # subnormal region, exact ties included
    ]).astype(np.float32)
    ours = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def pin_e4m3_saturation_and_zero():
    big = np.array([448.0, 448.001, 463.9, 464.0, 500.0, 1e6, 3.4e38], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    tiny = np.array([2.0 ** -11, 1e-10, 0.0], np.float32)    # round to zero
    assert np.all(oracle.e4m3_encode(tiny) == 0x00)
    assert np.all(oracle.e4m3_encode(-tiny) == 0x80)
    assert oracle.e4m3_encode(np.array([2.0 ** -9], np.float32))[0] == 0x01
    assert oracle.e4m3_encode(np.array([2.0 ** -6], np.float32))[0] == 0x08


def pin_bf16_vs_torch():
    r = _rng(2)
    v = np.concatenate([
        r.standard_normal(20000),
        np.exp(r.uniform(-80, 80, 20000)) * r.choice([-1, 1], 20000),
    ]).astype(np.float32)
    # exact ties: fp32 patterns whose low 16 bits are 0x8000
    ties = (r.integers(0, 2 ** 15, 4000, dtype=np.uint32) << 16 | 0x8000
            | (r.integers(0, 2, 4000, dtype=np.uint32) << 31)) & 0xFE7FFFFF
    v = np.concatenate([v, ties.astype(np.uint32).view(np.float32)])
    v = v[np.isfinite(v)]
    assert np.array_equal(oracle.bf16_encode(v), _torch_bf16_bits(v))


# ------------------------------------------------------------------------------------------------
# S1: RMSNorm, RoPE, quantisation
# ------------------------------------------------------------------------------------------------

def pin_rmsnorm_unit_rms():
    x = _rng(3).standard_normal((16, D)).astype(np.float32)
    _, k32, _ = _store_rows(x, np.zeros(16), eps=0.0)
    rms = np.sqrt(np.mean(k32.astype(np.float64) ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) < 2e-7), rms


def pin_rmsnorm_scale_and_gamma():
    r = _rng(4)
    x = r.standard_normal((8, D)).astype(np.float32)
    g = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    s = np.array([0, 1, 5, 100, 999, 4000, 20000, 32767])
    _, a, _ = _store_rows(x, s, gamma=g, eps=0.0)
    _, b, _ = _store_rows(2 * x, s, gamma=g, eps=0.0)
    _, c, _ = _store_rows(x, s, gamma=2 * g, eps=0.0)
    assert np.array_equal(a, b), "RMSNorm output must not depend on the scale of x"
    assert np.array_equal(c, 2 * a), "the output must be linear in gamma"


def _inv_freq_np():
    return np.power(10000.0, -np.arange(0, 64, 2) / 64.0).astype(np.float32)


def pin_rope_inv_freq():
    assert np.array_equal(oracle.rope_inv_freq(), _inv_freq_np())


def pin_rope_complex_rotation():
    r = _rng(5)
    x = np.repeat(r.standard_normal((1, D)).astype(np.float32), 6, axis=0)
    s = np.array([0, 1, 7, 1000, 20000, 32767])
    _, k32, _ = _store_rows(x, s)
    k = k32.astype(np.float64)
    assert np.array_equal(k32[1:, :64], np.repeat(k32[:1, :64], 5, axis=0)), \
        "dims 0..63 are not rotated"
    z0 = k[0, 64::2] + 1j * k[0, 65::2]
    for row, pos in enumerate(s):
        ang = 4.0 * pos * _inv_freq_np().astype(np.float64)
        z = z0 * np.exp(1j * ang)
        got = k[row, 64::2] + 1j * k[row, 65::2]
        assert np.all(np.abs(got - z) <= 4e-7 * np.abs(z0) + 1e-12), (pos, np.abs(got - z).max())


def pin_rope_relative_position():
    """<R_m a, R_n b> depends only on m - n (rotated halves)."""
    r = _rng(6)
    a = r.standard_normal(D).astype(np.float32)
    b = r.standard_normal(D).astype(np.float32)
    x = np.stack([a, b, a, b])
    s = np.array([10, 3, 1010, 1003])
    _, k32, _ = _store_rows(x, s, eps=0.0)
    k = k32.astype(np.float64)
    d1 = k[0, 64:] @ k[1, 64:]
    d2 = k[2, 64:] @ k[3, 64:]
    assert abs(d1 - d2) < 2e-5 * (1 + abs(d1)), (d1, d2)


def pin_bf16_store_vs_torch():
    x = _rng(7).standard_normal((40, D)).astype(np.float32)
    s = np.arange(40) * 3
    pool, k32, pt = _store_rows(x, s, dtype=BF16)
    pb = oracle.page_bytes(BF16)
    for i, si in enumerate(s):
        base = pt[0, si // PAGE] * pb + (si % PAGE) * 256
        assert np.array_equal(pool[base:base + 256].view(np.uint16), _torch_bf16_bits(k32[i]))


def pin_fp8_store_scale_and_bound():
    x = _rng(8).standard_normal((40, D)).astype(np.float32)
    s = np.arange(40) * 2 + 1
    pool, k32, pt = _store_rows(x, s, dtype=FP8)
    pb = oracle.page_bytes(FP8)
    for i, si in enumerate(s):
        base = pt[0, si // PAGE] * pb
        codes = pool[base + (si % PAGE) * D: base + (si % PAGE) * D + D]
        scale = float(pool[base + PAGE * D + 4 * (si % PAGE):][:4].view(np.float32)[0])
        amax = float(np.abs(k32[i]).max())
        assert abs(scale * 448.0 - amax) <= amax * 2 ** -23
        assert np.max(codes & 0x7F) == 0x7E, "the largest element must map to +-448"
        deq = _torch_e4m3_to_f64(codes) * scale
        err = np.abs(deq - k32[i].astype(np.float64))
        bound = 2.0 ** -4 * np.abs(k32[i]) + 2.0 ** -10 * scale + 1e-7 * amax
        assert np.all(err <= bound)
        assert np.array_equal(np.signbit(deq) | (deq == 0), np.signbit(k32[i]) | (deq == 0))


# eps = 2^80 swamps the mean square of any row with |x| < 2^12 (half an fp64 ulp of 2^80 is
# 2^27), so 1 / sqrt(ms + eps) = 2^-40 exactly; gamma = 2^40 undoes it and position 0 rotates by
# nothing: the canonical key is x itself, bit for bit.  With eps outside the root the factor would
# be 2^-80 instead.
_EPS_HUGE, _GAMMA_HUGE = 2.0 ** 80, np.full(D, 2.0 ** 40, np.float32)


def _store_rows_pos0(x, dtype):
    """Store each row of x at key index 0 of its own sequence (position 0, no rotation) with the
    eps / gamma pair above; returns (pool, k32, page_table)."""
    n = x.shape[0]
    pt = np.arange(n, dtype=np.int32)[:, None]
    pool = oracle.new_pool(n, dtype)
    skipped, k32 = oracle.store_keys(x, _GAMMA_HUGE, _EPS_HUGE, np.zeros(n, np.int32),
                                     np.arange(n, dtype=np.int32), pt, dtype, pool, want_k32=True)
    assert skipped == 0
    return pool, k32, pt


def pin_rmsnorm_eps_placement():
    """eps sits inside the square root, 1 / sqrt(mean(x^2) + eps), in two closed forms."""
    r = _rng(60)
    # (1) eps comparable to the mean square: x = c * ones with c = 2^-3 has mean square c^2, and
    # eps = 3 c^2 makes the factor 1 / sqrt(4 c^2) = 1 / (2c) = 4, so the key is gamma / 2.
    g = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    x = np.full((3, D), 0.125, np.float32)
    x[1] *= -1.0
    x[2, ::2] *= -1.0                      # signs do not change the mean square
    _, k32, _ = _store_rows(x, np.zeros(3, np.int32), gamma=g, eps=3.0 / 64.0)
    assert np.array_equal(k32, np.sign(x) * (g / 2)), "eps must enter under the square root"
    # (2) eps = 2^80 with gamma = 2^40 returns x unchanged
    x = (r.standard_normal((5, D)) * 2.0 ** r.integers(-20, 10, (5, 1))).astype(np.float32)
    _, k32, _ = _store_rows_pos0(x, BF16)
    assert np.array_equal(k32, x)


def _e4m3_positive_midpoints():
    """Midpoints between adjacent non-negative e4m3 values (by torch's decoding), and the values."""
    vals = np.unique(_torch_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8)))
    return (vals[:-1] + vals[1:]) / 2.0, vals


def pin_fp8_store_bytes():
    """fp8 store bytes rebuilt in numpy and torch from the canonical keys: the scale is numpy's
    correctly rounded fp32 division absmax / 448, the codes torch's e4m3fn cast of numpy's fp32
    quotients k / scale.  Keys equal x exactly (eps = 2^80, gamma = 2^40, position 0), so the
    rows are built to put quotients on and next to every e4m3 midpoint, over scales of many
    magnitudes, where any other rounding of the quotient (a product with the fp32 reciprocal of
    the scale, say) picks the other code."""
    r = _rng(61)
    mids, _ = _e4m3_positive_midpoints()
    rows = []
    for n in range(96):
        amax = np.float32(r.uniform(1.0, 2.0) * 2.0 ** r.integers(-24, 11))
        scale = amax / np.float32(448.0)
        m = r.choice(mids, D - 1)
        t = (m * np.float64(scale)).astype(np.float32)
        step = r.integers(-3, 4, D - 1)
        v = t.copy()
        for _ in range(3):                 # walk a few fp32 ulps from the rounded target
            v = np.where(step > 0, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(step < 0, np.nextafter(v, np.float32(-np.inf)), v)
            step = step - np.sign(step)
        v = np.minimum(v, amax)            # the absmax stays the key's largest magnitude
        sign = np.where(r.random(D - 1) < 0.5, -1.0, 1.0).astype(np.float32)
        row = np.concatenate([[amax if n % 2 else -amax], sign * v]).astype(np.float32)
        rows.append(row[r.permutation(D)])
    # plain Gaussian keys with a heavy channel, and a key with a zero
    g = r.standard_normal((32, D)) * 2.0 ** r.integers(-20, 10, (32, 1))
    g[:, 5] *= 40.0
    g[3, 7] = 0.0
    x = np.concatenate([np.stack(rows), g]).astype(np.float32)
    pool, k32, pt = _store_rows_pos0(x, FP8)
    assert np.array_equal(k32, x)
    pb = oracle.page_bytes(FP8)
    amax = np.abs(x).max(axis=1).astype(np.float32)
    scale = amax / np.float32(448.0)                                   # fp32 division
    q = (x / scale[:, None]).astype(np.float32)                        # fp32 division
    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    recip = (x * (np.float32(1.0) / scale)[:, None]).astype(np.float32)
    other = torch.from_numpy(recip).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.sum(other != want) > 20, "the rows must tell the two quotient roundings apart"
    for n in range(x.shape[0]):
        base = int(pt[n, 0]) * pb
        assert np.array_equal(pool[base: base + D], want[n]), n
        got_s = pool[base + PAGE * D: base + PAGE * D + 4].view(np.float32)[0]
        assert got_s == scale[n], n


def pin_paging_invariance():
    r = _rng(9)
    n = 150
    x = r.standard_normal((n, D)).astype(np.float32)
    s = np.arange(n, dtype=np.int32)
    for dtype in (FP8, BF16):
        pt_id = np.arange(3, dtype=np.int32)[None, :]
        pt_perm = np.array([[4, 0, 2]], dtype=np.int32)
        p1 = oracle.new_pool(3, dtype)
        p2 = oracle.new_pool(5, dtype)
        oracle.store_keys(x, np.ones(D, np.float32), 1e-6, s, None, pt_id, dtype, p1)
        oracle.store_keys(x, np.ones(D, np.float32), 1e-6, s, None, pt_perm, dtype, p2)
        k1 = _pool_keys(p1, pt_id, dtype, 0, n)
        k2 = _pool_keys(p2, pt_perm, dtype, 0, n)
        assert np.array_equal(k1, k2)
        pb = oracle.page_bytes(dtype)
        assert np.all(p2[1 * pb:2 * pb] == 0xA5) and np.all(p2[3 * pb:4 * pb] == 0xA5), \
            "pages outside the table stay untouched"


# ------------------------------------------------------------------------------------------------
# S2: visibility and scores
# ------------------------------------------------------------------------------------------------

def pin_visibility_brute_force():
    for t in range(-5, 600):
        n = sum(1 for s in range(0, 200) if 4 * s + 3 <= t)
        assert oracle.n_visible(t, 100) == n, t
    assert oracle.n_visible(10 ** 6, 2) == 128, "visibility is capped by the page-table width"


def _tiny_pool(dtype, n_keys=140, seed=10):
    r = _rng(seed)
    x = r.standard_normal((n_keys, D)).astype(np.float32)
    g = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    s = np.arange(n_keys, dtype=np.int32)
    max_pages = (n_keys + PAGE - 1) // PAGE
    pt = r.permutation(max_pages + 1)[:max_pages].astype(np.int32)[None, :]
    pool = oracle.new_pool(max_pages + 1, dtype)
    oracle.store_keys(x, g, 1e-6, s, None, pt, dtype, pool)
    return pool, pt


def _q_bits(n_q, seed):
    q = _rng(seed).standard_normal((n_q, H, D)).astype(np.float32)
    return _torch_bf16_bits(q.ravel()).reshape(n_q, H, D)


def pin_visibility_in_logits():
    pool, pt = _tiny_pool(BF16)
    L, q_len = 4 * 140, 40
    qb = _q_bits(q_len, 11)
    w = np.full((q_len, H), 1.0 / 64, np.float32)
    out, nv = oracle.logits(qb, w, pool, BF16, pt, [L], [0, q_len])
    for i in range(q_len):
        t = L - q_len + i
        vis = np.array([4 * s + 3 <= t for s in range(out.shape[1])])
        assert np.array_equal(np.isfinite(out[i]), vis), i
        assert nv[i] == vis.sum()


def pin_scores_onehot_head():
    for dtype in (FP8, BF16):
        pool, pt = _tiny_pool(dtype, seed=12)
        n_q, L = 6, 4 * 140
        qb = _q_bits(n_q, 13)
        keys = _pool_keys(pool, pt, dtype, 0, 140)
        for h0 in (0, 17, 63):
            w = np.zeros((n_q, H), np.float32)
            w[:, h0] = 1.0
            out, nv = oracle.logits(qb, w, pool, dtype, pt, [L], [0, n_q])
            qf = _bf16_to_f64(qb)
            for i in range(n_q):
                ref = np.maximum(0.0, keys[:nv[i]] @ qf[i, h0])
                assert np.allclose(out[i, :nv[i]], ref, rtol=1e-12, atol=1e-12), (dtype, h0, i)


def pin_scores_relu_pairs():
    pool, pt = _tiny_pool(BF16, seed=14)
    n_q, L = 4, 4 * 140
    half = _q_bits(n_q, 15)[:, :32]
    qb = np.concatenate([half, half ^ np.uint16(0x8000)], axis=1)       # q[h+32] = -q[h]
    wh = (_rng(16).standard_normal((n_q, 32)) / 8).astype(np.float32)
    w = np.concatenate([wh, wh], axis=1)
    out, nv = oracle.logits(qb, w, pool, BF16, pt, [L], [0, n_q])
    keys = _pool_keys(pool, pt, BF16, 0, 140)
    qf = _bf16_to_f64(half)
    for i in range(n_q):
        d = keys[:nv[i]] @ qf[i].T                                       # [n, 32]
        ref = np.abs(d) @ wh[i].astype(np.float64)
        assert np.allclose(out[i, :nv[i]], ref, rtol=1e-10, atol=1e-10)


def pin_scores_positive_linear():
    r = _rng(17)
    n_q, n_keys, L = 3, 60, 4 * 60
    keys = np.abs(r.standard_normal((1, n_keys, D))).astype(np.float32)
    qb = _torch_bf16_bits(np.abs(r.standard_normal(n_q * H * D)).astype(np.float32)).reshape(n_q, H, D)
    w = (r.standard_normal((n_q, H)) / 8).astype(np.float32)
    pt = np.zeros((1, 1), np.int32)
    out, nv = oracle.logits(qb, w, None, BF16, pt, [L], [0, n_q], keys_ref=keys, ref_stride=n_keys)
    qf = _bf16_to_f64(qb)
    for i in range(n_q):
        v = w[i].astype(np.float64) @ qf[i]                              # sum_h w_h q_h
        ref = keys[0, :nv[i]].astype(np.float64) @ v
        assert np.allclose(out[i, :nv[i]], ref, rtol=1e-10, atol=1e-10)


# ------------------------------------------------------------------------------------------------
# S3: top-k
# ------------------------------------------------------------------------------------------------

def pin_topk_brute_force():
    r = _rng(18)
    for trial in range(60):
        n = int(r.integers(1, 50))
        k = int(r.choice([1, 2, 5, 16, 64]))
        v = r.integers(0, 6, size=(3, n)).astype(np.float64)            # many ties
        v[0, ::3] = -0.0
        idx, val = oracle.topk(v, k)
        for row in range(3):
            vr = np.where(v[row] == 0, 0.0, v[row])
            sel = [i for i in range(n)
                   if sum(1 for j in range(n) if vr[j] > vr[i] or (vr[j] == vr[i] and j < i)) < k]
            got = [i for i in idx[row] if i >= 0]
            assert sorted(got) == sel, (trial, row)
            assert list(idx[row, :len(sel)]) == list(np.argsort(-vr, kind="stable")[:len(sel)])
            assert np.all(idx[row, len(sel):] == -1) and np.all(np.isneginf(val[row, len(sel):]))


def pin_topk_row_len():
    v = np.array([[5.0, 4.0, 3.0, 9.0, 9.0, 1.0]])
    idx, _ = oracle.topk(v, 3, row_len=np.array([3]))
    assert list(idx[0]) == [0, 1, 2]
    idx, _ = oracle.topk(v, 2, row_len=np.array([6]))
    assert list(idx[0]) == [3, 4]


# ------------------------------------------------------------------------------------------------
# Needle planting (harness helper built on the oracle's RoPE)
# ------------------------------------------------------------------------------------------------

def pin_needle_planting():
    r = _rng(19)
    kstar = r.standard_normal((5, D))
    s = np.array([0, 3, 77, 900, 32000], np.int32)
    g = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    xo = np.empty((5, D), np.float32)
    oracle.lib().oracle_plant_keys(oracle._ptr(kstar), oracle._ptr(s), 5, oracle._ptr(g),
                                   oracle._ptr(xo))
    _, k32, _ = _store_rows(xo, s, gamma=g)
    for i in range(5):
        c = k32[i].astype(np.float64) @ kstar[i] / (np.linalg.norm(k32[i]) * np.linalg.norm(kstar[i]))
        assert c > 1 - 1e-6, c


def pin_needle_must_rank_bf16():
    """A needle planted along the query's weighted head sum must be selected under bf16 storage,
    on the oracle alone (store, logits, top-k), on inputs small enough for brute force.

    Bound (the must-rank reading of the pages' recall test): bf16 rounding moves each key element
    by at most 2^-9 of itself and ReLU is 1-Lipschitz, so a logit moves by at most
    B(s) = 2^-9 sum_i u_i |k32_i|, u = sum_h |w_h| |q_h|.  A needle whose unquantised logit minus
    2B beats all but fewer than k other keys' unquantised logits plus 2B must be in the top-k.
    The bf16 logits are also recomputed by brute force from the stored bytes."""
    import workloads as W
    wl = W.make_workload("needle-pin", 4242, [1024, 1024, 1536, 2048], [1, 1, 1, 1], 16,
                         permute_pages=True, extra_pages=1)
    wl.needles = W.draw_needles(wl, 4)
    x = oracle.plant_needles(wl, "weighted")
    pool = oracle.new_pool(wl.n_pages_pool, BF16)
    _, k32 = oracle.store_keys(x, wl.gamma, wl.eps, wl.key_idx, wl.key_seq, wl.page_table, BF16,
                               pool, want_k32=True)
    ref = np.zeros((wl.n_seq, wl.max_keys, D), np.float32)
    ref[wl.key_seq, wl.key_idx] = k32
    o16, nv = oracle.logits(wl.q_bits, wl.w, pool, BF16, wl.page_table, wl.seq_lens, wl.cu_q)
    o32, _ = oracle.logits(wl.q_bits, wl.w, None, BF16, wl.page_table, wl.seq_lens, wl.cu_q,
                           keys_ref=ref, ref_stride=wl.max_keys)
    top, _ = oracle.topk(o16, wl.k, row_len=nv)
    nd = wl.needles
    checked = 0
    for r in range(wl.n_q):
        n = int(nv[r])
        assert n == wl.seq_lens[r] // 4     # one query at the last token sees every key
        q = _bf16_to_f64(wl.q_bits[r])                          # [64, 128]
        w = wl.w[r].astype(np.float64)
        keys = _pool_keys(pool, wl.page_table, BF16, r, n)      # decoded from the bytes
        brute = np.maximum(keys @ q.T, 0.0) @ w
        assert np.allclose(brute, o16[r, :n], rtol=1e-12, atol=1e-12)
        u = np.abs(w) @ np.abs(q)
        bound = 2.0 * 2.0 ** -9 * (np.abs(ref[r, :n]).astype(np.float64) @ u)
        lo, hi = o32[r, :n] - bound, o32[r, :n] + bound
        sel = set(int(v) for v in top[r] if v >= 0)
        for sn in nd["s"][nd["qrow"] == r]:
            sn = int(sn)
            if np.sum(np.delete(hi, sn) >= lo[sn]) < wl.k:
                assert sn in sel, f"needle ({r}, {sn}) must be in the bf16 top-{wl.k}"
                checked += 1
    assert checked >= 12, checked


# ---- rotated store: the normalised Walsh-Hadamard transform -------------------------------------

def _sylvester_matrix(n=D) -> np.ndarray:
    """H[i][j] = (-1)^popcount(i & j): the Sylvester-Hadamard matrix from its bit definition."""
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    pop = np.zeros_like(bits)
    for b in range(7):
        pop += (bits >> b) & 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def _exact_two_pow_minus_3_5() -> float:
    """The fp64 nearest to 2^-3.5, from 60-digit decimal arithmetic (float() of a Decimal rounds
    correctly)."""
    import decimal
    ctx = decimal.Context(prec=60)
    return float(ctx.sqrt(ctx.divide(decimal.Decimal(1), decimal.Decimal(128))))


def pin_hadamard_scale_is_nearest():
    c = oracle.hadamard_scale()
    assert c == _exact_two_pow_minus_3_5()
    assert abs(c * c * 128.0 - 1.0) < 4e-16


def pin_hadamard_vs_bit_definition():
    Hm = _sylvester_matrix()
    assert np.array_equal(Hm @ Hm.T, 128.0 * np.eye(D))
    x = _rng(30).standard_normal((12, D))
    got = oracle.hadamard128(x)
    want = (x @ Hm.T) * _exact_two_pow_minus_3_5()
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(x))


def pin_hadamard_unit_vectors_exact():
    """A unit vector's transform is a column of H times the scale, exactly (every butterfly sum
    is of +-1 and 0); the all-ones vector maps to sqrt(128) e_0."""
    c = _exact_two_pow_minus_3_5()
    Hm = _sylvester_matrix()
    e = np.eye(D)
    got = oracle.hadamard128(e)
    assert np.array_equal(got, Hm.T * c)
    ones = oracle.hadamard128(np.ones(D))[0]
    assert ones[0] == 128.0 * c and np.all(ones[1:] == 0.0)


def pin_hadamard_orthogonal_involution():
    r = _rng(31)
    a, b = r.standard_normal(D), r.standard_normal(D) * 1e3
    ha, hb = oracle.hadamard128(a)[0], oracle.hadamard128(b)[0]
    assert abs(np.dot(ha, hb) - np.dot(a, b)) <= 1e-12 * np.linalg.norm(a) * np.linalg.norm(b)
    assert abs(np.linalg.norm(ha) - np.linalg.norm(a)) <= 1e-14 * np.linalg.norm(a)
    assert np.max(np.abs(oracle.hadamard128(ha)[0] - a)) <= 1e-14 * np.max(np.abs(a))


def pin_rotate_q_vs_matrix_and_torch():
    """bf16 q: the matrix product is exact in fp64 here (sums of 128 bf16 values of similar
    magnitude), times the scale, then torch's fp32 and bf16 casts (round-to-nearest-even)."""
    q = _torch_bf16_bits(_rng(32).standard_normal((6, 64, D)).astype(np.float32))
    got = oracle.rotate_q(q)
    v = (_bf16_to_f64(q).reshape(-1, D) @ _sylvester_matrix().T) * _exact_two_pow_minus_3_5()
    want = _torch_bf16_bits(v.astype(np.float32)).reshape(q.shape)
    assert np.array_equal(got, want)


def pin_rotated_store_composes():
    """The rotated store's canonical key is the unrotated one rotated (up to the fp32 rounding of
    each), its bf16 bytes are torch's casts of it, and rotated q . rotated k = q . k."""
    r = _rng(33)
    x = (r.standard_normal((30, D)) * r.choice([0.1, 1.0, 30.0], (30, 1))).astype(np.float32)
    s = np.arange(30, dtype=np.int32) * 5 + 2
    _, k_plain, _ = _store_rows(x, s, dtype=BF16)
    gamma = np.ones(D, np.float32)
    max_pages = int(s.max()) // PAGE + 1
    pt = np.arange(max_pages, dtype=np.int32)[None, :]
    pool = oracle.new_pool(max_pages, BF16)
    _, k_rot = oracle.store_keys(x, gamma, 1e-6, s, None, pt, BF16, pool, want_k32=True,
                                 hadamard=True)
    c = _exact_two_pow_minus_3_5()
    want = (k_plain.astype(np.float64) @ _sylvester_matrix().T) * c
    amax = np.abs(k_plain).max(axis=1, keepdims=True)
    assert np.all(np.abs(k_rot - want) <= 2.0 ** -21 * amax)
    pb = oracle.page_bytes(BF16)
    for i, si in enumerate(s):
        base = pt[0, si // PAGE] * pb + (si % PAGE) * 256
        assert np.array_equal(pool[base:base + 256].view(np.uint16), _torch_bf16_bits(k_rot[i]))
    q = _bf16_to_f64(_torch_bf16_bits(r.standard_normal((4, D)).astype(np.float32)))
    qr = _bf16_to_f64(oracle.rotate_q(_torch_bf16_bits(q.astype(np.float32))))
    d_plain = q @ k_plain.astype(np.float64).T
    d_rot = qr @ k_rot.astype(np.float64).T
    scale = np.abs(q).sum(axis=1, keepdims=True) * amax.T
    assert np.all(np.abs(d_rot - d_plain) <= 2.0 ** -6 * scale)


# ---- fp8 x fp8 scoring: q quantised per (query, head) ----------------------------------------

def pin_quantize_q_vs_torch():
    """The scale is numpy's correctly rounded fp32 division absmax / 448; the codes are torch's
    e4m3 cast of numpy's fp32 quotients; an all-zero vector gives scale 0 and codes 0."""
    r = _rng(40)
    v = (r.standard_normal((50, D)) * r.choice([1e-4, 1.0, 300.0], (50, 1))).astype(np.float32)
    v[7] = 0.0
    q = _torch_bf16_bits(v)
    codes, scales = oracle.quantize_q(q)
    qf = _bf16_to_f64(q).astype(np.float32)
    amax = np.abs(qf).max(axis=1)
    want_s = (amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(scales, want_s)
    for n in range(50):
        if want_s[n] == 0:
            assert scales[n] == 0 and np.all(codes[n] == 0)
            continue
        quot = (qf[n] / want_s[n]).astype(np.float32)
        want = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[n], want), n


def pin_quantize_q_error_bound():
    q = _torch_bf16_bits(_rng(41).standard_normal((40, D)).astype(np.float32))
    codes, scales = oracle.quantize_q(q)
    deq = _torch_e4m3_to_f64(codes) * scales[:, None].astype(np.float64)
    qf = _bf16_to_f64(q)
    # half an e4m3 step (2^-4 relative) plus half the subnormal step, times the scale
    assert np.all(np.abs(deq - qf) <= 2.0 ** -4 * np.abs(qf) + 2.0 ** -10 * scales[:, None])
    # the largest element maps to the code 448 (up to the scale's own fp32 rounding)
    amax = np.abs(qf).max(axis=1)
    assert np.all(np.abs(np.abs(deq).max(axis=1) - amax) <= 2.0 ** -23 * amax)
    assert np.all((codes & 0x7F).max(axis=1) == 0x7E)


def _fp8q_case(seed):
    r = _rng(seed)
    n_keys, n_q = 130, 3
    x = r.standard_normal((n_keys, D)).astype(np.float32)
    pool, _, pt = _store_rows(x, np.arange(n_keys), dtype=FP8)
    seq_lens = np.array([4 * n_keys + 3], np.int32)
    cu_q = np.array([0, n_q], np.int32)
    w = (r.standard_normal((n_q, H)) / 8).astype(np.float32)
    return r, pool, pt, seq_lens, cu_q, w


def pin_logits_fp8q_equals_bf16_path_on_exact_q():
    """With power-of-two q scales, code * scale is a bf16 value: the fp8-q logits must equal the
    bf16-q logits of those values exactly (same fp64 products, same order)."""
    r, pool, pt, seq_lens, cu_q, w = _fp8q_case(42)
    codes = r.integers(0, 0x7F, (3, H, D)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes |= (r.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    scales = (2.0 ** r.integers(-6, 2, (3, H))).astype(np.float32)
    qv = _torch_e4m3_to_f64(codes) * scales[:, :, None]
    q_bits = _torch_bf16_bits(qv.astype(np.float32))
    assert np.array_equal(_bf16_to_f64(q_bits), qv)
    a, nva = oracle.logits(q_bits, w, pool, FP8, pt, seq_lens, cu_q)
    b, nvb = oracle.logits_fp8q(codes, scales, w, pool, pt, seq_lens, cu_q)
    assert np.array_equal(nva, nvb)
    assert np.array_equal(a, b)


def pin_logits_fp8q_scale_linear():
    """Doubling every q scale doubles every logit exactly; a head with scale 0 drops out."""
    r, pool, pt, seq_lens, cu_q, w = _fp8q_case(43)
    q = _torch_bf16_bits(r.standard_normal((3, H, D)).astype(np.float32))
    codes, scales = oracle.quantize_q(q)
    a, _ = oracle.logits_fp8q(codes, scales, w, pool, pt, seq_lens, cu_q)
    b, _ = oracle.logits_fp8q(codes, scales * 2, w, pool, pt, seq_lens, cu_q)
    fin = np.isfinite(a)
    assert np.array_equal(b[fin], 2 * a[fin])
    w0 = w.copy()
    w0[:, 5] = 0.0
    s0 = scales.copy()
    s0[:, 5] = 0.0
    c, _ = oracle.logits_fp8q(codes, s0, w, pool, pt, seq_lens, cu_q)
    d, _ = oracle.logits_fp8q(codes, scales, w0, pool, pt, seq_lens, cu_q)
    assert np.allclose(c[fin], d[fin], rtol=1e-12, atol=1e-9)


def pin_logits_fp8q_close_to_bf16_q():
    """Quantising q moves each logit by at most the e4m3 rounding of q (2^-4 relative per
    element), bounded per head by 2^-4 * sum_i |q_i| |k_i|."""
    r, pool, pt, seq_lens, cu_q, w = _fp8q_case(44)
    q = _torch_bf16_bits(r.standard_normal((3, H, D)).astype(np.float32))
    codes, scales = oracle.quantize_q(q)
    a, _ = oracle.logits(q, w, pool, FP8, pt, seq_lens, cu_q)
    b, _ = oracle.logits_fp8q(codes, scales, w, pool, pt, seq_lens, cu_q)
    kd = _pool_keys(pool, pt, FP8, 0, 130)
    qf = np.abs(_bf16_to_f64(q))
    bound = 2.0 ** -4 * np.einsum("nhd,sd->nhs", qf, np.abs(kd)) + 1e-6
    bound = np.einsum("nh,nhs->ns", np.abs(w.astype(np.float64)), bound)
    a, b = a[:, :130], b[:, :130]
    fin = np.isfinite(a)
    assert fin.sum() > 300
    assert np.all(np.abs(a - b)[fin] <= bound[fin])


# ---- fp4 keys (e2m1 codes, one fp32 scale per key) -------------------------------------------

FP4 = oracle.FP4
# The FP4 E2M1 magnitudes as tabulated in the OCP Microscaling Formats (MX) specification v1.0,
# section 5.3.3 (codes 0..7; bit 3 is the sign).
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_brute(v: np.ndarray) -> np.ndarray:
    """Nearest magnitude by exhaustive distance, ties to the even code, saturating at 6."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[:, None] - _E2M1_MAG[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (code | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def pin_e2m1_table():
    got = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(got[:8], _E2M1_MAG)
    assert np.array_equal(got[8:], -_E2M1_MAG)


def pin_e2m1_encode_brute_force():
    mids = (_E2M1_MAG[:-1] + _E2M1_MAG[1:]) / 2
    m32 = mids.astype(np.float32)
    v = np.concatenate([_E2M1_MAG, mids, np.nextafter(m32, np.float32(9)),
                        np.nextafter(m32, np.float32(0)), [6.5, 7.0, 100.0, 1e-30],
                        np.linspace(-8, 8, 4001)]).astype(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.e2m1_encode(v), _e2m1_brute(v))


def pin_fp4_store_bytes():
    """The stored bytes of fp4 keys, rebuilt in numpy from the canonical keys: scale = numpy's
    fp32 division absmax / 6, codes by the brute-force encoder, low nibble = even dim."""
    r = _rng(50)
    x = (r.standard_normal((70, D)) * r.choice([1e-3, 1.0, 40.0], (70, 1))).astype(np.float32)
    x[9] = 0.0
    s = np.arange(70, dtype=np.int32) * 2
    pool, k32, pt = _store_rows(x, s, dtype=FP4)
    pb = oracle.page_bytes(FP4)
    assert pb == 64 * 68
    for n, sn in enumerate(s):
        base = pt[0, sn // PAGE] * pb
        slot = sn % PAGE
        amax = np.abs(k32[n]).max()
        scale = np.float32(amax) / np.float32(6.0)
        if scale > 0:
            codes = _e2m1_brute((k32[n] / scale).astype(np.float32))
        else:
            codes = np.zeros(D, np.uint8)
        want = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        assert np.array_equal(pool[base + 64 * slot: base + 64 * slot + 64], want), n
        got_s = pool[base + 4096 + 4 * slot: base + 4096 + 4 * slot + 4].view(np.float32)[0]
        assert got_s == scale


def pin_fp4_logits_vs_numpy():
    r = _rng(51)
    n_keys = 100
    x = r.standard_normal((n_keys, D)).astype(np.float32)
    pool, _, pt = _store_rows(x, np.arange(n_keys), dtype=FP4)
    pb = oracle.page_bytes(FP4)
    keys = np.zeros((n_keys, D))
    for sn in range(n_keys):
        base = pt[0, sn // PAGE] * pb
        slot = sn % PAGE
        by = pool[base + 64 * slot: base + 64 * slot + 64]
        sc = float(pool[base + 4096 + 4 * slot: base + 4096 + 4 * slot + 4].view(np.float32)[0])
        codes = np.empty(D, np.uint8)
        codes[0::2], codes[1::2] = by & 15, by >> 4
        keys[sn] = np.where(codes & 8, -1.0, 1.0) * _E2M1_MAG[codes & 7] * sc
    q = _torch_bf16_bits(r.standard_normal((2, H, D)).astype(np.float32))
    w = (r.standard_normal((2, H)) / 8).astype(np.float32)
    seq_lens = np.array([4 * n_keys + 1], np.int32)
    cu_q = np.array([0, 2], np.int32)
    got, nv = oracle.logits(q, w, pool, FP4, pt, seq_lens, cu_q)
    d = np.einsum("nhd,sd->nhs", _bf16_to_f64(q), keys)
    want = np.einsum("nh,nhs->ns", w.astype(np.float64), np.maximum(d, 0.0))
    for row in range(2):
        m = int(nv[row])
        assert np.allclose(got[row, :m], want[row, :m], rtol=1e-12, atol=1e-9)
        assert np.all(np.isneginf(got[row, m:]))


# ---- sparse attention over the selected keys --------------------------------------------------

def _attn_case(seed, n_seq=2, max_keys=9, n_slots=20, q_lens=(3, 2), n_heads=3, k=6):
    """Small random attention inputs: bf16 q and kv, a permuted slot table with a hole, lists of
    k entries per row drawn from the sequence's keys."""
    r = _rng(seed)
    n_q = int(sum(q_lens))
    q = _torch_bf16_bits(r.standard_normal((n_q, n_heads, 512)).astype(np.float32))
    kv = _torch_bf16_bits(r.standard_normal((n_slots, 512)).astype(np.float32))
    kv_slot = r.permutation(n_slots)[:n_seq * max_keys].astype(np.int32).reshape(n_seq, max_keys)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    idx = np.stack([r.choice(max_keys, k, replace=False) for _ in range(n_q)]).astype(np.int32)
    return q, kv, kv_slot, cu_q, idx


def _attn_numpy(q, kv, kv_slot, cu_q, idx, scale):
    """The same attention from scipy's softmax and logsumexp over numpy's matrix products."""
    from scipy.special import logsumexp, softmax  # noqa: PLC0415
    n_q, n_heads, _ = q.shape
    out = np.zeros((n_q, n_heads, 512))
    lse = np.full((n_q, n_heads), -np.inf)
    qd, kvd = _bf16_to_f64(q), _bf16_to_f64(kv)
    for i in range(n_q):
        b = int(np.searchsorted(cu_q, i, side="right") - 1)
        sl = [kv_slot[b, s] for s in idx[i] if 0 <= s < kv_slot.shape[1]]
        sl = [x for x in sl if 0 <= x < kv.shape[0]]
        if not sl:
            continue
        v = kvd[sl]                                    # [n, 512]
        lg = scale * (qd[i] @ v.T)                     # [heads, n]
        out[i] = softmax(lg, axis=1) @ v
        lse[i] = logsumexp(lg, axis=1)
    return out, lse


def pin_attn_vs_scipy():
    """Two sequences, permuted slots, distinct lists: equal to scipy's softmax of numpy's
    products, times the same rows."""
    q, kv, kv_slot, cu_q, idx = _attn_case(1)
    scale = 512 ** -0.5
    o, l = oracle.sparse_attn(q, kv, kv_slot, cu_q, idx, scale)
    ro, rl = _attn_numpy(q, kv, kv_slot, cu_q, idx, scale)
    assert np.allclose(o, ro, rtol=1e-12, atol=1e-13)
    assert np.allclose(l, rl, rtol=1e-12, atol=1e-13)


def pin_attn_single_key():
    """One listed key: the weight is exactly 1, so the output is that latent exactly and the
    log-sum-exp is its scaled logit."""
    q, kv, kv_slot, cu_q, idx = _attn_case(2)
    idx[:, 1:] = -1
    scale = 0.37
    o, l = oracle.sparse_attn(q, kv, kv_slot, cu_q, idx, scale)
    for i in range(q.shape[0]):
        b = int(np.searchsorted(cu_q, i, side="right") - 1)
        v = _bf16_to_f64(kv[kv_slot[b, idx[i, 0]]])
        assert np.array_equal(o[i], np.broadcast_to(v, o[i].shape))
        assert np.allclose(l[i], scale * (_bf16_to_f64(q[i]) @ v), rtol=1e-13, atol=1e-13)


def pin_attn_uniform_weights():
    """q = 0: every logit is 0, the output is the plain mean of the listed latents and the
    log-sum-exp is log n."""
    q, kv, kv_slot, cu_q, idx = _attn_case(3)
    q[:] = 0
    o, l = oracle.sparse_attn(q, kv, kv_slot, cu_q, idx, 1.0)
    for i in range(q.shape[0]):
        b = int(np.searchsorted(cu_q, i, side="right") - 1)
        mean = _bf16_to_f64(kv[kv_slot[b, idx[i]]]).mean(axis=0)
        assert np.allclose(o[i], mean, rtol=1e-13, atol=1e-14)
        assert np.allclose(l[i], np.log(idx.shape[1]), rtol=1e-14)


def pin_attn_list_order_and_skipped_entries():
    """The list is a set of terms: shuffling it changes nothing, and entries that are -1, beyond
    max_keys, or whose slot is -1 or beyond the kv rows add nothing."""
    q, kv, kv_slot, cu_q, idx = _attn_case(4, k=5)
    kv_slot = kv_slot.copy()
    kv_slot[:, 7] = -1
    kv_slot[:, 8] = kv.shape[0] + 3
    base = np.where(np.isin(idx, [7, 8]), 0, idx)      # lists without the bad keys
    o0, l0 = oracle.sparse_attn(q, kv, kv_slot, cu_q, base, 0.5)
    r = _rng(40)
    junk = np.array([-1, 9, 12, -5, 7, 8], np.int32)
    ext = np.concatenate([base, np.tile(junk, (base.shape[0], 1))], axis=1)
    ext = np.stack([r.permutation(row) for row in ext]).astype(np.int32)
    o1, l1 = oracle.sparse_attn(q, kv, kv_slot, cu_q, ext, 0.5)
    assert np.allclose(o0, o1, rtol=1e-12, atol=1e-13)
    assert np.allclose(l0, l1, rtol=1e-12, atol=1e-13)


def pin_attn_duplicate_entry_counts_twice():
    """A key listed twice gets twice the weight: with logits a, a, b the weights are
    2e^a / (2e^a + e^b) and e^b / (2e^a + e^b)."""
    q, kv, kv_slot, cu_q, idx = _attn_case(5, k=3)
    idx[:, 1] = idx[:, 0]
    scale = 0.11
    o, _ = oracle.sparse_attn(q, kv, kv_slot, cu_q, idx, scale)
    for i in range(q.shape[0]):
        b = int(np.searchsorted(cu_q, i, side="right") - 1)
        va = _bf16_to_f64(kv[kv_slot[b, idx[i, 0]]])
        vb = _bf16_to_f64(kv[kv_slot[b, idx[i, 2]]])
        for h in range(q.shape[1]):
            qh = _bf16_to_f64(q[i, h])
            a, c = scale * (qh @ va), scale * (qh @ vb)
            wa = 2 / (2 + np.exp(c - a))
            assert np.allclose(o[i, h], wa * va + (1 - wa) * vb, rtol=1e-12, atol=1e-13)


def pin_attn_hardmax_limit():
    """A huge scale turns the softmax into the argmax: the output is the latent with the largest
    q . v (numpy's argmax of numpy's products)."""
    q, kv, kv_slot, cu_q, idx = _attn_case(6)
    o, _ = oracle.sparse_attn(q, kv, kv_slot, cu_q, idx, 1e6)
    for i in range(q.shape[0]):
        b = int(np.searchsorted(cu_q, i, side="right") - 1)
        v = _bf16_to_f64(kv[kv_slot[b, idx[i]]])
        for h in range(q.shape[1]):
            best = int(np.argmax(v @ _bf16_to_f64(q[i, h])))
            assert np.array_equal(o[i, h], v[best])


def pin_attn_empty_list():
    """No valid entry: output 0 and log-sum-exp -inf."""
    q, kv, kv_slot, cu_q, idx = _attn_case(7)
    idx[:] = -1
    idx[0, 0] = 99                                       # beyond max_keys
    o, l = oracle.sparse_attn(q, kv, kv_slot, cu_q, idx, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(l))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
