#!/usr/bin/env python3
"""Throughput of the DSA indexer hot path on one MI355X.

One step = the whole path over one batch: store the step's keys (RMSNorm + RoPE + quantise +
paged store), then score every query against its visible keys and select the top-k.

Default workload: the long prefill chunk -- the last 8192 queries of a 22528-token context (5632
compressed keys, 37,746,688 visible (query, key) pairs), bf16 keys, top-512, with the chunk's 2048
keys stored inside the step and keys 0..3583 stored beforehand.  Other shapes are selectable with
--workload for the design notes; they are not the headline line.

Prints one JSON line: keys scored per second (whole job), top-k queries per second, the scoring
kernel's roofline figures (HIP events around that kernel, on the stream it runs on) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

WORKLOADS = {
    # name: (config id, kv dtype)
    "prefill-22k-chunk8192-bf16": (3, 1),
    "prefill-22k-chunk8192-fp8": (3, 0),
    "prefill-4k-fp8": (0, 0),
    "prefill-4k-bf16-needles": (1, 1),
    "decode-64x4k-22k-fp8": (2, 0),
    "decode-64x4k-22k-bf16": (2, 1),
    "decode-32x128k-fp8": (4, 0),
    "decode-32x128k-bf16": (4, 1),
    "decode-32x128k-fp4": (4, 2),
    "decode-64x4k-22k-fp4": (2, 2),
    "prefill-22k-chunk8192-fp4": (3, 2),
}
KV_NAMES = {0: "fp8", 1: "bf16", 2: "fp4"}
KEY_BYTES = {0: 132, 1: 256, 2: 68}     # stored bytes per key: codes + scale, or bf16 values
DEFAULT = "prefill-22k-chunk8192-bf16"


# Sources that determine each kernel's machine code: a committed counter summary for a kernel is
# used only while its digest over these files still matches.
KERNEL_SOURCES = {
    "score_rows_bf16_kernel": ["csrc/score.hip", "csrc/internal.h", "build.py"],
    "score_rows_kernel": ["csrc/score.hip", "csrc/internal.h", "build.py"],
    # decode calls: the roofline and its traffic cover the scoring and the selection kernel
    "score_kernel": ["csrc/score.hip", "csrc/topk.hip", "csrc/internal.h", "build.py"],
    "store_keys_kernel": ["csrc/store.hip", "csrc/internal.h", "build.py"],
    "score_rows_fp8q_kernel": ["csrc/score.hip", "csrc/internal.h", "build.py"],
    "sparse_attn_kernel": ["csrc/attn.hip", "csrc/attn.h", "build.py"],
}


def sources_digest(kernel: str) -> str:
    import hashlib  # noqa: PLC0415
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, "sparse_attention_indexer_rmsnorm_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload`, from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary committed under profiles/ (already scaled by the copy-kernel calibration), or None if
    there is none or the kernel's sources have changed since the counters were taken."""
    path = os.path.join(HERE, "profiles", f"{kernel}-{workload}.md")
    if not os.path.exists(path):
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]+)`", open(path).read(), re.M))
    if fields.get("sources_digest") != sources_digest(kernel) or "traffic_bytes" not in fields:
        return None
    return int(fields["traffic_bytes"])


def _pairs(wl) -> int:
    """(query, visible key) pairs of a batch: the queries of sequence b are its last q_len_b
    tokens, and the query at token t sees floor((t + 1) / 4) compressed keys."""
    t = np.concatenate([int(L) - int(ql) + np.arange(int(ql), dtype=np.int64)
                        for L, ql in zip(wl.seq_lens, wl.q_lens)]) if wl.n_q else \
        np.zeros(0, np.int64)
    nv = np.minimum((t + 1) // 4, wl.max_keys)
    nv[t < 0] = 0
    return int(nv.sum()), nv


def cpu_baseline(wl, dtype, x_step_mask, n_sample_rows: int, rotate: bool = False,
                 fp8q: bool = False) -> dict:
    """The oracle as it stands, on every (n_q / n_sample_rows)-th query row of the same batch,
    plus the store of the step's keys (and, rotated, the rotation of q) scaled to the same
    fraction of the batch."""
    import oracle  # noqa: PLC0415  (test infrastructure; only this leg uses it)
    oracle.lib()
    stride = max(1, wl.n_q // n_sample_rows)
    rows = np.arange(0, wl.n_q, stride, dtype=np.int64)
    frac = rows.size / wl.n_q
    pool = oracle.new_pool(wl.n_pages_pool, dtype)
    if x_step_mask is not None:
        oracle.store_workload(wl, dtype, pool=pool, mask=~x_step_mask, hadamard=rotate)
    t0 = time.perf_counter()
    oracle.store_workload(wl, dtype, pool=pool, mask=x_step_mask, hadamard=rotate)
    q_bits = oracle.rotate_q(wl.q_bits) if rotate else wl.q_bits
    q8 = oracle.quantize_q(wl.q_bits) if fp8q else None
    t_store = time.perf_counter() - t0
    t0 = time.perf_counter()
    if fp8q:
        lg, nv = oracle.logits_fp8q(q8[0], q8[1], wl.w, pool, wl.page_table, wl.seq_lens,
                                    wl.cu_q, rows=rows)
    else:
        lg, nv = oracle.logits(q_bits, wl.w, pool, dtype, wl.page_table, wl.seq_lens, wl.cu_q,
                               rows=rows)
    oracle.topk(lg, wl.k, row_len=nv)
    t_read = time.perf_counter() - t0
    secs = t_store * frac + t_read
    return {"value": float(nv.sum() / secs), "unit": "keys/s", "cores": oracle.num_threads(),
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{rows.size} of {wl.n_q} query rows (every {stride}th) scored and "
                      f"selected, plus the step's store scaled by {frac:.4f}; "
                      f"{secs:.2f} s of wall time"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def ev_stats(pairs) -> dict:
    """Median, min and mean in ms of a list of (start, end) timing events."""
    t = np.array([a.elapsed_time(b) for a, b in pairs], dtype=np.float64)
    return {"median": round(float(np.median(t)), 5), "min": round(float(t.min()), 5),
            "mean": round(float(t.mean()), 5)}


def spin_cycles(torch, us: float) -> int:
    """Cycles of torch's spin kernel that keep the GPU busy for about `us` microseconds: queued
    before a short timed call, the spin lets the host enqueue the call and its events before the
    GPU reaches them, so the events bracket device work only (otherwise they also catch the
    host's launch of the call whenever the GPU waits for it)."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 200000
    torch.cuda._sleep(n)
    e0.record(stream)
    torch.cuda._sleep(n)
    e1.record(stream)
    torch.cuda.synchronize()
    per_us = n / max(e0.elapsed_time(e1) * 1e3, 1.0)
    return max(1000, int(per_us * us))


def ceilings(args, torch) -> int:
    """Context for the rooflines: the MFMA rate torch's GEMM reaches on this GPU, and the HBM read
    rate of a plain reduction, each the best of --steps runs."""
    dev = torch.device("cuda:0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        a @ b
    best = 1e9
    for _ in range(args.steps):
        e0.record()
        a @ b
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    gemm = 2 * 8192 ** 3 / (best * 1e-3) / 1e12
    del a, b
    x = torch.ones(128 << 20, dtype=torch.float32, device=dev)       # 512 MiB
    other = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    best_r = 1e9
    for _ in range(args.steps):
        other.sum()                        # evicts x from the MALL without dirtying it
        e0.record()
        x.sum()
        e1.record()
        torch.cuda.synchronize()
        best_r = min(best_r, e0.elapsed_time(e1))
    read = (512 << 20) / (best_r * 1e-3) / 1e9
    print(json.dumps({"metric": "device ceilings for library code",
                      "bf16_gemm_8192_tflops": round(gemm, 1),
                      "bf16_gemm_frac_of_peak": round(gemm / PEAK_BF16_TFLOPS, 4),
                      "hbm_read_512mib_gbs": round(read, 1),
                      "hbm_read_frac_of_peak": round(read / PEAK_HBM_GBS, 4)}), flush=True)
    return 0


def store_population(args, wl, dtype, d, pool, ix, torch) -> int:
    """S1 alone: store every key of the workload, --steps times; keys stored per second and the
    store kernel's HBM roofline (per key: 512 B of activations and 8 B of indices read, 132,
    256 or 68 B written for fp8, bf16 or fp4)."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def step():
        ix.store_keys(d["x"], d["gamma"], d["key_idx"], d["page_table"], pool, dtype, eps=wl.eps,
                      key_seq=d["key_seq"], rotate=args.rotate)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    key_bytes = KEY_BYTES[dtype]
    algo = wl.n_keys * (512 + 8 + key_bytes)
    achieved = algo / (kms * 1e-3) / 1e9
    name = args.workload + ("-rotated" if args.rotate else "") + "-store-population"
    print(json.dumps({
        "metric": "keys stored/s (S1: RMSNorm + RoPE + " + ("Hadamard + " if args.rotate else "")
                  + "quantise + paged store)",
        "value": wl.n_keys / (ms * 1e-3), "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": name, "keys": wl.n_keys, "kv_dtype": KV_NAMES[dtype]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": committed_traffic("store_keys_kernel", name),
                     "kernel": "store_keys_kernel", "kernel_ms": round(kms, 4)},
        "cpu_baseline": None}), flush=True)
    return 0


def attn_bench(args, cfg, ix, torch, W) -> int:
    """The sparse attention over the selected keys alone, on a workload's rows: q of
    --attn-heads heads x 512 dims (bf16) against each row's listed 512-dim bf16 latents (a random
    subset of min(k, visible) keys per row, workloads.attn_inputs).  Roofline: bf16 MFMA for
    prefill-shaped batches (4 flops per (row, head, listed key, dim): q.v and p.v), HBM for
    decode-shaped ones (1024 B per listed latent, plus q and the output)."""
    wl = W.CONFIGS[cfg]() if cfg != 4 else W.cfg4(needles=False)
    a = W.attn_inputs(wl, n_heads=args.attn_heads)
    dev = torch.device("cuda:0")
    q, kv, kv_slot, idx = a.torch_inputs(dev)
    cu_q = torch.from_numpy(wl.cu_q).to(dev)
    n_list = int((a.idx >= 0).sum())
    H, k = a.n_heads, a.idx.shape[1]
    out = torch.empty((wl.n_q, H, 512), dtype=torch.bfloat16, device=dev)
    ws_bytes = ix.sparse_attn_workspace_size(wl.n_q, H, k)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def call():
        ix.sparse_attn(q, kv, kv_slot, cu_q, idx, a.scale, out=out, workspace=ws)

    decode = cfg in (2, 4)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    # events in a second pass; decode calls are shorter than the host's launch of them, so a GPU
    # spin before each puts the host ahead and the events bracket device work only
    spin = spin_cycles(torch, 150.0) if decode else 0
    for e0, e1 in evs:
        if spin:
            torch.cuda._sleep(spin)
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    kt = ev_stats(evs)
    kms = kt["median"] if decode else kt["mean"]
    flops = 4.0 * H * 512 * n_list
    algo_bytes = n_list * 1024.0 + q.numel() * 2 + out.numel() * 2 + wl.n_q * H * 4 + idx.numel() * 4
    if decode:
        ach = algo_bytes / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        ach = flops / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None}
    name = wl.name.rsplit("-", 1)[0] if wl.name.endswith(("-fp8", "-bf16")) else wl.name
    name = f"{name}-attn-h{H}"
    roof["traffic"] = committed_traffic("sparse_attn_kernel", name)
    roof["kernel"] = "sparse_attn_kernel" + (" + sparse_attn_merge_kernel" if ws_bytes else "")
    roof["kernel_ms"] = kt
    roof["region"] = ("attention call (kernel and merge), median of HIP events" if decode else
                      "attention call, mean of HIP events")
    line = {
        "metric": "sparse attention listed keys/s ((query, listed key) pairs, all heads)",
        "value": n_list / (ms * 1e-3), "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "queries": wl.n_q, "heads": H, "latent_dim": 512, "k": k,
                   "listed": n_list, "workspace_bytes": ws_bytes},
        "roofline": roof, "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle  # noqa: PLC0415  (test infrastructure; only this leg uses it)
        oracle.lib()
        stride = max(1, wl.n_q // min(wl.n_q, args.cpu_sample_rows // 4))
        rows = np.arange(0, wl.n_q, stride, dtype=np.int64)
        c0 = time.perf_counter()
        oracle.sparse_attn(a.q_bits, a.kv_bits, a.kv_slot, wl.cu_q, a.idx, a.scale, rows=rows)
        secs = time.perf_counter() - c0
        n_s = int((a.idx[rows] >= 0).sum())
        line["cpu_baseline"] = {"value": n_s / secs, "unit": "keys/s", "cores": oracle.num_threads(),
                                "affinity_cores": len(os.sched_getaffinity(0)),
                                "cpu_model": cpu_model(), "kind": "oracle",
                                "sample": f"{rows.size} of {wl.n_q} rows (every {stride}th), "
                                          f"{n_s} listed keys, {secs:.2f} s of wall time"}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=1024)
    ap.add_argument("--cold", action="store_true",
                    help="read a 512 MiB buffer before every step so that the step's keys come "
                         "from HBM, not the 256 MB MALL; steps are then timed with HIP events "
                         "around each step (the flush excluded)")
    ap.add_argument("--store-population", action="store_true",
                    help="time only the store of the workload's whole key population (S1 alone): "
                         "keys stored per second and the store kernel's HBM roofline")
    ap.add_argument("--rotate", action="store_true",
                    help="the rotated store (Hadamard transform after RoPE): keys stored rotated "
                         "and the batch's q rotated inside every step")
    ap.add_argument("--fp8q", action="store_true",
                    help="fp8 x fp8 scoring (fp8 cache only): the batch's q quantised per head "
                         "inside every step, scored on the fp8 matrix cores; roofline against the "
                         "fp8 peak")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure what this GPU delivers to plain library code: torch's bf16 "
                         "GEMM at 8192^3 (TFLOP/s) and torch's read of a 512 MiB tensor (GB/s), "
                         "the latter from HBM after a read of another 512 MiB")
    ap.add_argument("--attn", action="store_true",
                    help="only time the sparse attention over the selected keys on the "
                         "workload's rows (the consumer of the top-k lists)")
    ap.add_argument("--attn-heads", type=int, default=64, choices=(32, 64, 128))
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB --steps times (the "
                         "reference for scaling HBM byte counters); prints its bytes per copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the indexer path "
              "shards by sequence or query chunk with no collective on the hot path, and this "
              "build runs one GPU.", file=sys.stderr)
        return 2

    import torch  # noqa: PLC0415
    import sparse_attention_indexer_rmsnorm_amd as ix  # noqa: PLC0415
    import workloads as W  # noqa: PLC0415

    if args.ceilings:
        return ceilings(args, torch)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": args.steps}))
        return 0

    ix.lib()
    cfg, dtype = WORKLOADS[args.workload]
    if args.attn:
        return attn_bench(args, cfg, ix, torch, W)
    if args.fp8q and (dtype != 0 or args.rotate):
        print("--fp8q needs an fp8 workload and no --rotate", file=sys.stderr)
        return 2
    wl = W.CONFIGS[cfg]() if cfg != 4 else W.cfg4(needles=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {
        "x": torch.from_numpy(wl.x).to(dev), "gamma": torch.from_numpy(wl.gamma).to(dev),
        "key_idx": torch.from_numpy(wl.key_idx).to(dev),
        "key_seq": torch.from_numpy(wl.key_seq).to(dev),
        "page_table": torch.from_numpy(wl.page_table).to(dev),
        "seq_lens": torch.from_numpy(wl.seq_lens).to(dev),
        "cu_q": torch.from_numpy(wl.cu_q).to(dev), "q": wl.q_torch().to(dev),
        "w": torch.from_numpy(wl.w).to(dev),
    }
    pool = ix.new_cache(wl.n_pages_pool, dtype, device=dev)
    if args.store_population:
        return store_population(args, wl, dtype, d, pool, ix, torch)
    step_mask = wl.step_keys if wl.step_keys is not None else np.ones(wl.n_keys, bool)
    pre = np.nonzero(~step_mask)[0]
    stp = np.nonzero(step_mask)[0]
    if pre.size:
        ix.store_keys(d["x"][pre].contiguous(), d["gamma"], d["key_idx"][pre].contiguous(),
                      d["page_table"], pool, dtype, eps=wl.eps,
                      key_seq=d["key_seq"][pre].contiguous(), rotate=args.rotate)
    sx = d["x"][stp].contiguous()
    sidx = d["key_idx"][stp].contiguous()
    sseq = d["key_seq"][stp].contiguous()
    ws = torch.empty(ix.workspace_size(wl.n_q, wl.n_seq, wl.max_pages, wl.k), dtype=torch.uint8,
                     device=dev)
    out_idx = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def ev_pairs():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]

    evs, call_evs, step_evs = ev_pairs(), ev_pairs(), ev_pairs()
    for a, b in evs:     # materialise the underlying hipEvent_t handles the library records
        a.record(stream)
        b.record(stream)
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    flush_sink = torch.empty((), dtype=torch.uint8, device=dev)

    q_rot = torch.empty_like(d["q"]) if args.rotate else None

    def step(i=None, inner_events=True):
        ix.store_keys(sx, d["gamma"], sidx, d["page_table"], pool, dtype, eps=wl.eps,
                      key_seq=sseq, rotate=args.rotate)
        events = None if i is None or not inner_events else evs[i]
        if args.fp8q:
            codes, scales = ix.quantize_q(d["q"])
            if i is not None:
                call_evs[i][0].record(stream)
            ix.logits_topk_fp8q(codes, scales, d["w"], pool, d["page_table"], d["seq_lens"],
                                d["cu_q"], wl.k, out_idx=out_idx, workspace=ws, events=events)
        else:
            q = ix.rotate_q(d["q"], out=q_rot) if args.rotate else d["q"]
            if i is not None:
                call_evs[i][0].record(stream)
            ix.logits_topk(q, d["w"], pool, dtype, d["page_table"], d["seq_lens"], d["cu_q"],
                           wl.k, out_idx=out_idx, workspace=ws, events=events)
        if i is not None:
            call_evs[i][1].record(stream)

    decode = cfg in (2, 4)

    spin = spin_cycles(torch, 150.0) if decode and flush is None else 0

    def timed_loop(inner_events: bool, ahead: bool = False):
        for i in range(args.steps):
            if flush is not None:
                # read, not write, the 512 MiB: written lines would be dirty in the MALL and
                # every read of the step would then also pay for writing them back
                flush_sink.copy_(flush.max())
            elif ahead:
                torch.cuda._sleep(spin)
            step_evs[i][0].record(stream)
            step(i, inner_events)
            step_evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The host clock times a plain pass.  Decode calls are shorter than the host's launch of
    # them, so their events come from two more passes in which a GPU spin before every step puts
    # the host ahead (the MALL flush does the same with --cold): one with events around the step
    # and the call only (events inside the call would add their own packets to it), and one with
    # events around the scoring kernel alone.
    t0 = time.perf_counter()
    timed_loop(inner_events=not decode)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if decode:
        timed_loop(inner_events=False, ahead=True)
        torch.cuda.synchronize()
    step_t = ev_stats(step_evs)
    call_t = ev_stats(call_evs)
    if decode:
        timed_loop(inner_events=True, ahead=True)
        torch.cuda.synchronize()

    # the host clock times the loop (with --cold it also covers the flushes, so the step events
    # time the steps); the events give the median and min of single steps and calls
    score_t = ev_stats(evs)
    ms = (t1 - t0) * 1e3 / args.steps if flush is None else step_t["mean"]
    pairs, nv = _pairs(wl)
    key_bytes = KEY_BYTES[dtype]
    if decode:
        # one pass over the visible keys of every sequence, plus q and w; the roofline covers the
        # whole idx_logits_topk call (scoring and selection), the score kernel alone beside it
        algo_bytes = float(nv.sum()) * key_bytes + wl.n_q * (64 * 128 * 2 + 64 * 4)
        achieved = algo_bytes / (call_t["median"] * 1e-3) / 1e9
        score_ach = algo_bytes / (score_t["median"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "region": "idx_logits_topk call (score + select), median of HIP events",
                "call_ms": call_t,
                "score_only": {"achieved": round(score_ach, 1),
                               "frac": round(score_ach / PEAK_HBM_GBS, 4), "kernel_ms": score_t}}
    else:
        flops = 2.0 * 64 * 128 * pairs
        score_ms = score_t["mean"]
        achieved = flops / (score_ms * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if args.fp8q else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "region": "scoring kernel, mean of HIP events around it on its stream",
                "kernel_ms": score_t, "call_ms": call_t}
    # prefill-shaped batches (>= 1024 queries, >= 4 per sequence) run a rows kernel (the bf16 one
    # stages pages straight into LDS), the others the split kernel
    prefill_shaped = wl.n_q >= 1024 and wl.n_q >= 4 * wl.n_seq
    kernel = ("score_rows_fp8q_kernel" if args.fp8q else
              "score_kernel" if not prefill_shaped else
              "score_rows_bf16_kernel" if dtype == 1 else "score_rows_kernel")
    # the bench's workload name (it names the cache dtype; the headline's equals wl.name)
    name = args.workload + ("-rotated" if args.rotate else "") + ("-fp8q" if args.fp8q else "")
    roof["traffic"] = committed_traffic(kernel, name)
    # decode rows of at least 16384 key columns are selected from bucketed keys, shorter ones from
    # the scores in segments
    sel = "topk_list_kernel" if wl.max_pages * 64 >= 16384 else "topk_hist_kernel"
    roof["kernel"] = kernel + (" + " + sel if decode and not args.fp8q else "")

    line = {
        "metric": "indexer keys scored/s (top-k queries/s alongside)",
        "value": pairs / (ms * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.fp8q else "bf16",
        "data": "synthetic" + (", MALL flushed before every step" if args.cold else ""),
        "config": {"workload": name, "queries": wl.n_q, "keys": int(wl.max_keys),
                   "visible_pairs": pairs, "k": wl.k, "kv_dtype": KV_NAMES[dtype],
                   "keys_stored_in_step": int(stp.size), "heads": 64, "head_dim": 128,
                   "workspace_bytes": int(ws.numel())},
        "topk_queries_per_s": wl.n_q / (ms * 1e-3),
        "step_ms": step_t,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, dtype, wl.step_keys, args.cpu_sample_rows,
                                            args.rotate, args.fp8q)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
