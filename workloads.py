"""Seeded synthetic inputs for the DSA indexer hot path (store -> score -> top-k).

Harness code, outside the library: the tests, the benchmark and the smoke check draw their inputs
here.  It draws random numbers and builds integer structure only: sequence lengths, query
counts, page tables and needle positions.  None of the indexer's arithmetic (normalisation, rotary
embedding, quantisation, scoring, selection) lives here, so the kernels and the CPU oracle can both
consume these arrays without sharing any of the method's code.

Every tensor comes from its own generator, ``numpy.random.default_rng([workload_seed, tensor_id])``,
so each input is independent of the order in which the others are drawn:

    0 x (pre-norm key activations)   1 gamma            2 q        3 w
    4 context lengths                5 page permutation 6 needle positions
    7 needle noise                   8 needle query choice
    20 attention q                   21 latents         22 latent slot permutation
    23 listed keys

Distributions (the DeepSeek Sparse Attention indexer as the four blog pages describe it, with the
shapes of their 4.5K / 10.5K / 22K-token tests and the 128K context length of the serving config):
x ~ N(0, 1) fp32; gamma ~ N(1, 0.1) fp32; q ~ N(0, 1) rounded to bf16; w ~ N(0, 1) / 8 fp32
(that is N(0,1)/sqrt(64) for 64 heads); eps = 1e-6.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

HEAD_DIM = 128
N_HEADS = 64
PAGE_KEYS = 64
COMPRESS = 4
FP8 = 0
BF16 = 1
FP4 = 2
EPS = 1e-6

T_X, T_GAMMA, T_Q, T_W, T_LENS, T_PERM, T_NEEDLE_POS, T_NEEDLE_NOISE, T_NEEDLE_Q = range(9)
T_ATTN_Q, T_ATTN_KV, T_ATTN_SLOT, T_ATTN_SEL = 20, 21, 22, 23
LATENT_DIM = 512


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tensor_id)])


def page_bytes(dtype: int) -> int:
    """Bytes of one cache page: 64 keys x (128 codes + 4 B scale) for fp8, 64 x 256 B for bf16,
    64 keys x (64 B of packed 4-bit codes + 4 B scale) for fp4."""
    if dtype == FP8:
        return PAGE_KEYS * (HEAD_DIM + 4)
    if dtype == FP4:
        return PAGE_KEYS * (HEAD_DIM // 2 + 4)
    return PAGE_KEYS * HEAD_DIM * 2


@dataclass
class Workload:
    """One batch of synthetic indexer inputs, all host-side (numpy / CPU torch)."""

    name: str
    seed: int
    seq_lens: np.ndarray          # [n_seq] int32, context tokens L_b
    q_lens: np.ndarray            # [n_seq] int32, queries are the last q_len_b tokens of seq b
    max_pages: int
    page_table: np.ndarray        # [n_seq, max_pages] int32, -1 = unused
    n_pages_pool: int
    key_seq: np.ndarray           # [n_keys] int32
    key_idx: np.ndarray           # [n_keys] int32, logical compressed-key index s (rope pos 4s)
    x: np.ndarray                 # [n_keys, 128] fp32 pre-norm activations
    gamma: np.ndarray             # [128] fp32
    q_bits: np.ndarray            # [n_q, 64, 128] uint16 bf16 bit patterns
    w: np.ndarray                 # [n_q, 64] fp32
    k: int
    eps: float = EPS
    dtypes: tuple = (FP8, BF16)
    # keys that belong to the measured store step (the prefill chunk stores its own keys inside
    # the step, a decode step the newest compressed key of each sequence; everything else is
    # stored beforehand).  Boolean mask over the key rows.
    step_keys: Optional[np.ndarray] = None
    # needles: per needle (seq b, query row i, key row n, logical s)
    needles: dict = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def n_q(self) -> int:
        return int(self.q_bits.shape[0])

    @property
    def n_keys(self) -> int:
        return int(self.x.shape[0])

    @property
    def max_keys(self) -> int:
        return self.max_pages * PAGE_KEYS

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    def q_torch(self) -> torch.Tensor:
        return torch.from_numpy(self.q_bits.view(np.int16)).view(torch.bfloat16)


def bf16_bits_from_normal(a: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 with torch's CPU cast; returns the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _page_table(seed: int, n_seq: int, n_keys_per_seq: np.ndarray, max_pages: int,
                permute: bool, extra_pages: int = 0):
    pages_per_seq = (n_keys_per_seq + PAGE_KEYS - 1) // PAGE_KEYS
    n_pool = int(pages_per_seq.sum()) + int(extra_pages)
    order = rng(seed, T_PERM).permutation(n_pool) if permute else np.arange(n_pool)
    pt = np.full((n_seq, max_pages), -1, dtype=np.int32)
    cur = 0
    for b in range(n_seq):
        p = int(pages_per_seq[b])
        pt[b, :p] = order[cur:cur + p]
        cur += p
    return pt, n_pool


def make_workload(name: str, seed: int, seq_lens, q_lens, k: int, *, permute_pages: bool,
                  max_pages: Optional[int] = None, stored_keys=None, extra_pages: int = 0,
                  dtypes=(FP8, BF16)) -> Workload:
    """Build a workload from per-sequence context lengths and query counts.

    ``stored_keys[b]`` is the number of compressed keys of sequence b that get stored (default
    floor(L_b / 4), every complete group of 4 tokens).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    n_seq = seq_lens.shape[0]
    n_keys_per_seq = (seq_lens // COMPRESS if stored_keys is None
                      else np.asarray(stored_keys, dtype=np.int64)).astype(np.int64)
    if max_pages is None:
        max_pages = int(max(1, ((n_keys_per_seq.max() if n_seq else 0) + PAGE_KEYS - 1) // PAGE_KEYS))
    pt, n_pool = _page_table(seed, n_seq, n_keys_per_seq, max_pages, permute_pages, extra_pages)
    key_seq = np.repeat(np.arange(n_seq, dtype=np.int32), n_keys_per_seq)
    key_idx = np.concatenate([np.arange(n, dtype=np.int32) for n in n_keys_per_seq]) \
        if n_seq else np.zeros(0, np.int32)
    n_keys = int(n_keys_per_seq.sum())
    x = rng(seed, T_X).standard_normal((n_keys, HEAD_DIM)).astype(np.float32)
    gamma = (1.0 + 0.1 * rng(seed, T_GAMMA).standard_normal(HEAD_DIM)).astype(np.float32)
    n_q = int(q_lens.sum())
    q32 = rng(seed, T_Q).standard_normal((n_q, N_HEADS, HEAD_DIM), dtype=np.float32)
    q_bits = bf16_bits_from_normal(q32)
    del q32
    w = (rng(seed, T_W).standard_normal((n_q, N_HEADS)) / 8.0).astype(np.float32)
    return Workload(name=name, seed=seed, seq_lens=seq_lens, q_lens=q_lens, max_pages=max_pages,
                    page_table=pt, n_pages_pool=n_pool, key_seq=key_seq, key_idx=key_idx, x=x,
                    gamma=gamma, q_bits=q_bits, w=w, k=k, dtypes=tuple(dtypes))


def draw_needles(wl: Workload, per_seq: int, s_hi: Optional[int] = None) -> dict:
    """Choose needle positions: for each needle, a query row of its sequence and a key index s
    below s_hi (default: every stored key of the sequence, which a decode query at the last token
    sees), without replacement within the sequence.  The caller picks s_hi so that every query of
    the sequence sees the needle.  Returns integer arrays plus the N(0, 0.1) noise each needle
    adds; the needle vectors themselves are built by the test harness."""
    g_pos, g_noise, g_q = rng(wl.seed, T_NEEDLE_POS), rng(wl.seed, T_NEEDLE_NOISE), rng(wl.seed, T_NEEDLE_Q)
    cu = wl.cu_q
    seq, qrow, s_arr, krow = [], [], [], []
    key_base = np.concatenate([[0], np.cumsum(np.bincount(wl.key_seq, minlength=wl.n_seq))])
    for b in range(wl.n_seq):
        ql = int(wl.q_lens[b])
        if ql == 0:
            continue
        rows = cu[b] + g_q.integers(0, ql, size=per_seq)
        hi = int(key_base[b + 1] - key_base[b])
        hi = hi if s_hi is None else min(s_hi, hi)
        ss = g_pos.choice(hi, size=per_seq, replace=False)
        for r, s in zip(rows, ss):
            seq.append(b)
            qrow.append(int(r))
            s_arr.append(int(s))
            krow.append(int(key_base[b] + s))
    noise = 0.1 * g_noise.standard_normal((len(seq), HEAD_DIM))
    return {"seq": np.array(seq, np.int32), "qrow": np.array(qrow, np.int64),
            "s": np.array(s_arr, np.int32), "krow": np.array(krow, np.int64), "noise": noise}


# ---------------------------------------------------------------------------------------------
# The five measured shapes.
# ---------------------------------------------------------------------------------------------

def cfg0(seed: int = 100) -> Workload:
    """Single-sequence prefill: 256 queries at t = 3840..4095 of a 4096-token context, 1024 keys,
    fp8 keys, identity page table, top-512."""
    return make_workload("prefill-4k-fp8", seed, [4096], [256], 512, permute_pages=False,
                         dtypes=(FP8,))


def cfg1(seed: int = 101) -> Workload:
    """cfg0's shapes with bf16 keys (fp8 too, for the recall gap) and 16 planted needles."""
    wl = make_workload("prefill-4k-bf16-needles", seed, [4096], [256], 512, permute_pages=False,
                       dtypes=(BF16, FP8))
    wl.needles = draw_needles(wl, 16, s_hi=960)
    return wl


def newest_keys(wl: Workload) -> np.ndarray:
    """Mask of each sequence's last compressed key (the key a decode step adds)."""
    last = wl.seq_lens[wl.key_seq] // 4 - 1
    return wl.key_idx == last


def cfg2(seed: int = 102) -> Workload:
    """Decode batch: 64 sequences, L_b ~ U{4096..22528}, one query each at t = L_b - 1, top-512,
    random page permutation over a shared pool, max 88 pages per sequence."""
    lens = rng(seed, T_LENS).integers(4096, 22528, size=64, endpoint=True).astype(np.int32)
    wl = make_workload("decode-64x4k-22k", seed, lens, np.ones(64, np.int32), 512,
                       permute_pages=True, max_pages=88)
    wl.step_keys = newest_keys(wl)
    return wl


def cfg3(seed: int = 103) -> Workload:
    """Long prefill chunk: the last 8192 queries of a 22528-token context (5632 keys), bf16 keys,
    top-512.  Keys 0..3583 are stored beforehand; the measured step stores keys 3584..5631 first."""
    wl = make_workload("prefill-22k-chunk8192-bf16", seed, [22528], [8192], 512,
                       permute_pages=False, dtypes=(BF16,))
    wl.step_keys = wl.key_idx >= 3584
    return wl


def cfg4(seed: int = 104, needles: bool = True) -> Workload:
    """Long-context decode: 32 sequences of 131072 tokens (32768 keys), one query each, top-1024,
    512 pages per sequence in a 16384-page randomly permuted pool, 32 needles per sequence."""
    wl = make_workload("decode-32x128k", seed, np.full(32, 131072, np.int32), np.ones(32, np.int32),
                       1024, permute_pages=True, max_pages=512)
    if needles:
        wl.needles = draw_needles(wl, 32)
    wl.step_keys = newest_keys(wl)
    return wl


CONFIGS = {0: cfg0, 1: cfg1, 2: cfg2, 3: cfg3, 4: cfg4}


# ---- inputs of the sparse attention over the selected keys --------------------------------------

@dataclass
class AttnInputs:
    """Host-side inputs of the sparse attention on a workload's sequences and query rows."""
    q_bits: np.ndarray       # [n_q, n_heads, 512] uint16 bf16 bit patterns
    kv_bits: np.ndarray      # [n_slots, 512] uint16
    kv_slot: np.ndarray      # [n_seq, max_keys] int32
    idx: np.ndarray          # [n_q, k] int32, -1 = none
    scale: float

    @property
    def n_heads(self) -> int:
        return int(self.q_bits.shape[1])

    def torch_inputs(self, device="cuda"):
        bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)  # noqa: E731
        return (bf(self.q_bits), bf(self.kv_bits), torch.from_numpy(self.kv_slot).to(device),
                torch.from_numpy(self.idx).to(device))


def _bf16_normal_rows(g: np.random.Generator, n: int, width: int, chunk: int = 1 << 16):
    out = np.empty((n, width), np.uint16)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        out[r0:r1] = bf16_bits_from_normal(g.standard_normal((r1 - r0, width), dtype=np.float32))
    return out


def attn_inputs(wl: Workload, n_heads: int = 64, k: Optional[int] = None,
                scale: Optional[float] = None) -> AttnInputs:
    """q and the latents ~ N(0, 1) rounded to bf16; one latent row per (sequence, key), on a
    random permutation of the rows; per query row a random subset of min(k, n) of the n keys
    stored for its sequence, in random order, then -1 padding (the shape of a top-k list, whose
    order is unspecified; the attention reads whatever keys a list names); softmax scale
    1 / sqrt(512) unless given."""
    k = wl.k if k is None else int(k)
    n_seq, max_keys = wl.n_seq, wl.max_keys
    q = _bf16_normal_rows(rng(wl.seed, T_ATTN_Q), wl.n_q * n_heads, LATENT_DIM)
    n_slots = n_seq * max_keys
    kv = _bf16_normal_rows(rng(wl.seed, T_ATTN_KV), n_slots, LATENT_DIM)
    kv_slot = rng(wl.seed, T_ATTN_SLOT).permutation(n_slots).astype(np.int32).reshape(
        n_seq, max_keys)
    n_stored = np.bincount(wl.key_seq, minlength=n_seq)
    row_seq = np.repeat(np.arange(n_seq), wl.q_lens)
    g = rng(wl.seed, T_ATTN_SEL)
    idx = np.full((wl.n_q, k), -1, np.int32)
    for r in range(wl.n_q):
        n = int(n_stored[row_seq[r]])
        m = min(k, n)
        if m:
            idx[r, :m] = g.permutation(n)[:m]
    return AttnInputs(q_bits=q.reshape(wl.n_q, n_heads, LATENT_DIM), kv_bits=kv, kv_slot=kv_slot,
                      idx=idx, scale=LATENT_DIM ** -0.5 if scale is None else float(scale))
