"""Benchmark: one mixed continuous-batching step of paged attention on one GPU.

A step is one pass of the whole hot path over one batch that is resident in
HBM: pa_append_kv writes the step's new K/V rows into their page slots, the
dispatch guard plans each route, pa_prefill_chunk runs the prefill chunks
(bf16 MFMA) and pa_decode runs the decode rows (split-K + log-sum-exp merge
when the guard picks it).  The workload is the mixed step with
Qwen3-4B attention heads: 4 prefill chunks of 512 tokens at prior offsets
0/512/1536/3072 plus 60 decode rows with contexts U[256, 4096]; 32 q heads,
8 KV heads, d = 128, bf16, page size 16, permuted pool of 1.25x the pages.
Inputs are synthetic N(0,1) (there are no weights or datasets here).

The timed steps launch the two routes through calls whose arguments are
marshalled once, so the host stays ahead of the GPU and the kernels run back
to back; events between the routes time each route on the launch stream.

Prints ONE JSON line.  `value` is the decode path's algorithmic KV GB/s; the
prefill path's algorithmic TFLOP/s is reported beside it, and `roofline`
describes whichever kernel takes the larger share of the step.  Two copies
of the KV pool are used alternately so consecutive steps cannot be served
from the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "paged decode attn KV GB/s (% HBM peak); chunked-prefill TFLOP/s (% MFMA peak)"
WORKLOAD = "mixed_step"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="wall-clock budget of the oracle's CPU baseline sample")
    ap.add_argument("--mode", choices=("step", "copy", "baselines", "configs", "ceiling"), default="step",
                    help="step: the benchmark; copy: calibration of the HBM counters and "
                         "the streaming ceiling (a plain 1 GiB device copy and a read-only "
                         "reduction of known size); baselines: the Qwen3-4B-shaped decode "
                         "through the production route, the same fused kernel unsplit over "
                         "pages and over a dense cache, and direct (non-flash) paged "
                         "attention; configs: one JSON line per named config and route "
                         "(cache-flushed per-call times, rate against peak, error against "
                         "the oracle on sampled requests); ceiling: the read rate of the "
                         "decode route's access pattern (pa_read_blocks over 2 GiB in 4 KiB "
                         "blocks, random order and in order, and 32 KiB blocks)")
    return ap.parse_args()


def copy_calibration(steps: int):
    """A plain copy of 1 GiB (1 GiB read + 1 GiB written per launch) and a
    read-only sum over 2 GiB, timed with events.  rocprofv3 counter runs of
    this mode give the bytes FETCH_SIZE / WRITE_SIZE report for known
    traffic, which scales the counters of the attention kernels."""
    import torch
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    big = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    res = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: y.copy_(x), 2 * n * 4),
                             ("sum_2GiB", lambda: big.sum(), (1 << 29) * 4)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        res[name] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1), "bytes": nbytes}
    print(json.dumps({"calibration": res}), flush=True)


def read_reference(steps: int = 20, warmup: int = 3) -> dict:
    """The read rate the decode route's access pattern reaches on this
    device: pa_read_blocks over 2 GiB (far past the 256 MB last-level cache)
    in 4 KiB blocks -- one (page, KV head) K or V block at d = 128 in bf16 --
    in a random order and in order, and in 32 KiB blocks (a page's K for 8 KV
    heads) in a random order; each with HIP events on the launch stream."""
    import torch
    import paged_kv_cache_02_amd as pa
    nbytes = 2 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(0)
    res = {}
    for name, bb, shuffle in (("4KiB_random", 4096, True), ("4KiB_in_order", 4096, False),
                              ("32KiB_random", 32768, True)):
        order = np.arange(nbytes // bb, dtype=np.int32)
        if shuffle:
            rng.shuffle(order)
        call = pa.bind_read_blocks(buf, torch.from_numpy(order).cuda(), bb, sink)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        res[name] = {"us": round(us, 1), "GB/s": round(nbytes / us / 1e3, 1)}
    del buf
    torch.cuda.empty_cache()
    return res


def baselines(steps: int, warmup: int):
    """What paging and the online softmax cost: the Qwen3-4B-shaped decode
    config (64 requests, 32/8 heads, d = 128, contexts in [1024, 8192]) timed
    through (1) pa_decode (the guard's balanced route), (2) the fused
    per-(request, KV head) kernel unsplit over the pages (pa_split_merge with
    one split: its merge pass is timed with it), (3) the same fused kernel
    over a dense cache (pa_decode_dense) and (4) direct paged attention with
    stored scores (pa_decode_direct).  One JSON line: microseconds per call
    and algorithmic GB/s (the K/V bytes and metadata every variant must
    read)."""
    import torch
    import paged_kv_cache_02_amd as pa
    import workloads as W
    b = W.make_config("qwen3_4b_decode", poison=False)
    dev = torch.device("cuda:0")

    def to_dev(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    q, kp, vp = to_dev(b.q), to_dev(b.k_pool), to_dev(b.v_pool)
    pt, sl, qo = i32(b.page_table), i32(b.seq_lens), i32(b.q_offsets)
    B, MP, P = b.num_seqs, b.page_table.shape[1], b.page_size
    # the dense cache [B, Hkv, MP * P, d]: each request's pages laid end to end
    kd = np.zeros((B, b.num_kv_heads, MP * P, b.head_dim), np.uint16)
    vd = np.zeros_like(kd)
    for r in range(B):
        L = int(b.seq_lens[r])
        n = (L + P - 1) // P
        pages = b.page_table[r, :n]
        kd[r, :, :n * P] = b.k_pool[pages].transpose(1, 0, 2, 3).reshape(b.num_kv_heads, n * P, -1)
        vd[r, :, :n * P] = b.v_pool[pages].transpose(1, 0, 2, 3).reshape(b.num_kv_heads, n * P, -1)
        kd[r, :, L:] = 0
        vd[r, :, L:] = 0
    kdt, vdt = to_dev(kd), to_dev(vd)
    del kd, vd
    desc = pa.make_desc(q, kp, pt, sl, b.max_seq_len, 1)
    out = torch.empty_like(q)
    lse = torch.empty(B, b.num_q_heads, dtype=torch.float32, device=dev)
    ws_dec = torch.empty(max(pa.pa_plan(desc)["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    ws_split = torch.empty(max(pa.pa_workspace_bytes(desc, 1), 256), dtype=torch.uint8, device=dev)
    ws_direct = torch.empty(max(int(pa.lib().pa_direct_workspace_bytes(ctypes.byref(desc))), 256),
                            dtype=torch.uint8, device=dev)
    variants = {
        "paged_balanced": lambda: pa.pa_decode(q, kp, vp, pt, sl, qo, b.scale, out=out, lse=lse,
                                               workspace=ws_dec, desc=desc),
        "paged_unsplit": lambda: pa.pa_split_merge(q, kp, vp, pt, sl, qo, b.scale, 1, out=out, lse=lse,
                                                   workspace=ws_split, desc=desc),
        "dense_unsplit": lambda: pa.pa_decode_dense(q, kdt, vdt, sl, b.scale, desc=desc, out=out, lse=lse),
        "direct_paged": lambda: pa.pa_decode_direct(q, kp, vp, pt, sl, b.scale, desc=desc, out=out, lse=lse,
                                                    workspace=ws_direct),
    }
    nbytes = decode_alg_bytes(b)
    res = {}
    for name, fn in variants.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        res[name] = {"us": round(us, 1), "GB/s": round(nbytes / us / 1e3, 1)}
        print(f"{name}: {res[name]}", file=sys.stderr, flush=True)
    print(json.dumps({"baselines": res, "workload": "qwen3_4b_decode", "alg_bytes": nbytes}), flush=True)


def config_sweep(iters: int, warmup: int):
    """One JSON line per named config and route.  Every call is timed on its
    own with HIP events after a 512 MiB write that leaves neither the 256 MB
    last-level cache nor the L2s holding any input; median, p10 and p90 over
    `iters` calls.  The inputs are the parity inputs (page tails and unused
    pages NaN), and the line carries the largest error against the oracle on
    a sample of requests with the oracle's own time on that sample."""
    import torch
    import oracle as ORACLE
    import paged_kv_cache_02_amd as pa
    import workloads as W
    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def to_dev(arr, dtype):
        t = (torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
             if dtype == W.BF16 else torch.from_numpy(np.ascontiguousarray(arr)))
        return t.to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    rng = np.random.default_rng(11)
    for name in ("tiny_decode", "qwen3_0p6b_decode", "qwen3_4b_decode", "mixed_step",
                 "long_splitk_decode"):
        full = W.make_config(name)
        if name == "mixed_step":
            routes = [("prefill", full.subset(*full.notes["prefill_requests"], name="chunks")),
                      ("decode", full.subset(*full.notes["decode_requests"], name="decode rows"))]
        elif name == "long_splitk_decode":
            routes = [("decode", full), ("split_merge_S16", full)]
        else:
            routes = [("decode", full)]
        kp, vp = to_dev(full.k_pool, full.dtype), to_dev(full.v_pool, full.dtype)
        for route, b in routes:
            q = to_dev(b.q, b.dtype)
            pt, sl, qo, qs = i32(b.page_table), i32(b.seq_lens), i32(b.q_offsets), i32(b.q_row_starts)
            desc = pa.make_desc(q, kp, pt, sl, b.max_seq_len, b.max_q_len)
            out = torch.empty_like(q)
            lse = torch.empty(b.total_q, b.num_q_heads, dtype=torch.float32, device=dev)
            if route == "prefill":
                need = pa.pa_plan(desc)["workspace_bytes"]
                ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
                fn = pa.bind_prefill_chunk(q, kp, vp, pt, sl, qo, b.scale, q_starts=qs, out=out,
                                           lse=lse, workspace=ws, desc=desc)
            elif route == "decode":
                ws = torch.empty(max(pa.pa_plan(desc)["workspace_bytes"], 256), dtype=torch.uint8,
                                 device=dev)
                fn = pa.bind_decode(q, kp, vp, pt, sl, qo, b.scale, out=out, lse=lse, workspace=ws,
                                    desc=desc)
            else:
                ws = torch.empty(pa.pa_workspace_bytes(desc, 16), dtype=torch.uint8, device=dev)
                fn = lambda: pa.pa_split_merge(q, kp, vp, pt, sl, qo, b.scale, 16, out=out, lse=lse,
                                               workspace=ws, desc=desc)
            times = []
            for i in range(warmup + iters):
                flush.fill_(i & 255)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                if i >= warmup:
                    times.append((e0, e1))
            torch.cuda.synchronize()
            us = np.array([a.elapsed_time(z) * 1e3 for a, z in times])
            t50, t10, t90 = (float(np.percentile(us, p)) for p in (50, 10, 90))
            if route == "prefill":
                work, unit, peak = prefill_alg_flops(b), "TFLOP/s", MFMA_BF16_PEAK_TFLOPS
                rate = work / (t50 * 1e-6) / 1e12
            else:
                work, unit, peak = decode_alg_bytes(b), "GB/s", HBM_PEAK_GBS
                rate = work / (t50 * 1e-6) / 1e9
            # parity on a sample of requests (their rows), with the oracle timed
            nsamp = min(b.num_seqs, 2 if route == "prefill" else 6)
            pick = (np.arange(nsamp) if route == "prefill"
                    else np.sort(rng.choice(b.num_seqs, nsamp, replace=False)))
            t0 = time.perf_counter()
            ro, rl = ORACLE.paged_attention(b.q_f32(), b.k_pool_f32(), b.v_pool_f32(), b.page_table,
                                            b.seq_lens, b.q_offsets, b.scale, requests=pick)
            oracle_s = time.perf_counter() - t0
            rows = np.concatenate([np.arange(b.q_row_starts[r], b.q_row_starts[r] + b.q_lens[r])
                                   for r in pick])
            o = out.float().cpu().numpy().astype(np.float64)[rows]
            l = lse.cpu().numpy().astype(np.float64)[rows]
            line = {
                "config": name, "route": route, "seed": int(full.seed),
                "shapes": {"B": int(b.num_seqs), "Hq": int(b.num_q_heads), "Hkv": int(b.num_kv_heads),
                           "d": int(b.head_dim), "page": int(b.page_size), "dtype": b.dtype,
                           "rows": int(b.total_q), "pool_pages": int(full.num_pages)},
                "sum_L": int(b.seq_lens.astype(np.int64).sum()),
                "work": int(work), "work_unit": "FLOP" if route == "prefill" else "B",
                "t_median_us": round(t50, 2), "t_p10_us": round(t10, 2), "t_p90_us": round(t90, 2),
                "rate": round(rate, 2), "rate_unit": unit, "frac_of_peak": round(rate / peak, 4),
                "max_abs_out_err": float(np.max(np.abs(o - ro[rows]))),
                "max_abs_lse_err": float(np.max(np.abs(l - rl[rows]))),
                "sample": f"{len(pick)} of {b.num_seqs} requests ({len(rows)} rows)",
                "oracle_s": round(oracle_s, 3), "host_cores": int(cores),
            }
            print(json.dumps(line), flush=True)
            del q, out, lse, ws
        del kp, vp
        torch.cuda.empty_cache()


_TOKEN = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """C++ source with its comments removed and whitespace runs collapsed,
    so an edit to comments or layout alone leaves the hash unchanged."""
    def keep(m):
        t = m.group(0)
        return " " if t.startswith("/") else t
    return " ".join(_TOKEN.sub(keep, src).split())


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_02_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def decode_alg_bytes(b) -> int:
    """K and V of every visible key once per KV head, q, out, lse, the page
    table entries read and the two int32 metadata arrays."""
    es = 4 if b.dtype == "f32" else 2
    keys = int(b.seq_lens.astype(np.int64).sum())
    pages = int(((b.seq_lens.astype(np.int64) + b.page_size - 1) // b.page_size).sum())
    B, Hq, d = b.num_seqs, b.num_q_heads, b.head_dim
    return (keys * b.num_kv_heads * d * 2 * es + 2 * B * Hq * d * es + B * Hq * 4 + pages * 4
            + 2 * B * 4)


def append_alg_bytes(b) -> int:
    """The new K and V rows read once and written once into their slots, plus
    the page-table entry each (row, KV head) write looks up."""
    rows = int(b.total_q)
    return 2 * 2 * rows * b.num_kv_heads * b.head_dim * 2 + rows * b.num_kv_heads * 4


def prefill_alg_flops(b) -> int:
    """4 * d * Hq per visible (query, key) pair: QK^T and PV, causal pairs only."""
    n = (b.seq_lens - b.q_offsets).astype(np.int64)
    o = b.q_offsets.astype(np.int64)
    pairs = int((n * o + n * (n + 1) // 2).sum())
    return 4 * b.head_dim * b.num_q_heads * pairs


def load_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch measured with rocprofv3 counters for this kernel
    source, or None if none were taken for the current source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(full, budget_s: float):
    """The oracle, untuned, on a bounded sample of the same workload."""
    import oracle as ORACLE
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    # the oracle's matrix products run on the BLAS pool, bounded by the CPUs
    # this process may use
    threads = max(1, min(blas, affinity))
    q, kp, vp = full.q_f32(), full.k_pool_f32(), full.v_pool_f32()
    dec0, dec1 = full.notes["decode_requests"]
    pf0, pf1 = full.notes["prefill_requests"]
    # decode rows: as many as fit half the budget
    t0 = time.perf_counter()
    done, nbytes = 0, 0
    for r in range(dec0, dec1):
        ORACLE.paged_attention(q, kp, vp, full.page_table, full.seq_lens, full.q_offsets,
                               full.scale, requests=[r])
        done += 1
        nbytes += int(full.seq_lens[r]) * full.num_kv_heads * full.head_dim * 2 * 2
        if time.perf_counter() - t0 > budget_s / 2:
            break
    t_dec = time.perf_counter() - t0
    # prefill: the first rows of the longest chunk
    r = pf1 - 1
    starts = full.q_row_starts
    K, V = ORACLE.gather(kp, vp, full.page_table[r], int(full.seq_lens[r]))
    pos = ORACLE.query_positions(int(full.seq_lens[r]), int(full.q_offsets[r]))
    t1 = time.perf_counter()
    rows, flops = 0, 0
    step = 16
    while time.perf_counter() - t1 < budget_s / 2 and rows < len(pos):
        sl = slice(int(starts[r]) + rows, int(starts[r]) + rows + step)
        ORACLE.attend(q[sl], K, V, pos[rows:rows + step], full.scale)
        flops += int(sum(4 * full.head_dim * full.num_q_heads * (p + 1) for p in pos[rows:rows + step]))
        rows += step
    t_pf = time.perf_counter() - t1
    return {
        "value": round(nbytes / t_dec / 1e9, 3), "unit": "GB/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of 60 decode rows ({nbytes / 1e6:.1f} MB of KV) in {t_dec:.1f} s; "
                  f"prefill: {rows} rows of the 512-token chunk at offset 3072 in {t_pf:.1f} s",
        "prefill_value": round(flops / t_pf / 1e12, 6), "prefill_unit": "TFLOP/s",
        "host_cpus": os.cpu_count(), "affinity_cpus": affinity, "blas_threads": blas,
        "cpu_model": host_cpu_model(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_02_amd as pa
    import workloads as W

    if args.mode == "copy":
        copy_calibration(args.steps)
        return
    if args.mode == "ceiling":
        print(json.dumps({"read_reference": read_reference(max(args.steps, 5), args.warmup)}), flush=True)
        return
    if args.mode == "baselines":
        baselines(args.steps, args.warmup)
        return
    if args.mode == "configs":
        config_sweep(args.steps, args.warmup)
        return
    torch.cuda.init()
    dev = torch.device("cuda:0")
    full = W.make_config(WORKLOAD, seed=args.seed, poison=False)
    pf = full.subset(*full.notes["prefill_requests"], name="prefill chunks")
    dc = full.subset(*full.notes["decode_requests"], name="decode rows")

    def to_dev(arr, dtype):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16) \
            if dtype == W.BF16 else torch.from_numpy(np.ascontiguousarray(arr))
        return t.to(dev)

    pools = [(to_dev(full.k_pool, full.dtype), to_dev(full.v_pool, full.dtype)) for _ in range(2)]
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    pf_t = {"q": to_dev(pf.q, pf.dtype), "pt": i32(pf.page_table), "sl": i32(pf.seq_lens),
            "qo": i32(pf.q_offsets), "qs": i32(pf.q_row_starts)}
    dc_t = {"q": to_dev(dc.q, dc.dtype), "pt": i32(dc.page_table), "sl": i32(dc.seq_lens),
            "qo": i32(dc.q_offsets)}
    pf_desc = pa.make_desc(pf_t["q"], pools[0][0], pf_t["pt"], pf_t["sl"], pf.max_seq_len,
                           pf.max_q_len)
    dc_desc = pa.make_desc(dc_t["q"], pools[0][0], dc_t["pt"], dc_t["sl"], dc.max_seq_len, 1)
    pf_plan = pa.pa_plan(pf_desc)
    dc_plan = pa.pa_plan(dc_desc)
    pf_out = torch.empty_like(pf_t["q"])
    pf_lse = torch.empty(pf.total_q, pf.num_q_heads, dtype=torch.float32, device=dev)
    dc_out = torch.empty_like(dc_t["q"])
    dc_lse = torch.empty(dc.total_q, dc.num_q_heads, dtype=torch.float32, device=dev)
    ws = torch.empty(max(dc_plan["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
    pf_ws = (torch.empty(pf_plan["workspace_bytes"], dtype=torch.uint8, device=dev)
             if pf_plan["workspace_bytes"] else None)

    # this step's new K/V rows (the prefill chunks' tokens and the decode
    # tokens), written into their page slots before attention reads them
    rng = np.random.default_rng(full.seed + 7)
    def new_rows(b):
        x = rng.standard_normal((b.total_q, b.num_kv_heads, b.head_dim)).astype(np.float32)
        return to_dev(W.f32_to_bf16_bits(x), W.BF16)
    # one append over the whole batch (chunk requests first, then decode
    # requests: the batch's own request order)
    ap_k, ap_v = new_rows(full), new_rows(full)
    full_t = {"pt": i32(full.page_table), "sl": i32(full.seq_lens), "qo": i32(full.q_offsets),
              "qs": i32(full.q_row_starts)}
    ap_desc = pa.make_desc(ap_k, pools[0][0], full_t["pt"], full_t["sl"], full.max_seq_len,
                           full.max_q_len)

    # the routes on each pool copy, with their arguments marshalled once so
    # that the host stays ahead of the GPU and the kernels run back to back
    calls = {}
    for i in (0, 1):
        kp, vp = pools[i]
        calls[("append", i)] = pa.bind_append_kv(
            ap_k, ap_v, kp, vp, full_t["pt"], full_t["sl"], full_t["qo"], q_starts=full_t["qs"],
            desc=ap_desc)
        calls[("prefill", i)] = pa.bind_prefill_chunk(
            pf_t["q"], kp, vp, pf_t["pt"], pf_t["sl"], pf_t["qo"], pf.scale, q_starts=pf_t["qs"],
            out=pf_out, lse=pf_lse, workspace=pf_ws, desc=pf_desc)
        calls[("decode", i)] = pa.bind_decode(
            dc_t["q"], kp, vp, dc_t["pt"], dc_t["sl"], dc_t["qo"], dc.scale, out=dc_out,
            lse=dc_lse, workspace=ws, desc=dc_desc)

    def step(i, ev=None):
        if ev is not None:
            ev[3].record()
        calls[("append", i & 1)]()
        if ev is not None:
            ev[0].record()
        calls[("prefill", i & 1)]()
        if ev is not None:
            ev[1].record()
        calls[("decode", i & 1)]()
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, events between the routes on the
    # stream the routes are launched on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    pf_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dc_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ap_ms = float(np.mean([e[3].elapsed_time(e[0]) for e in evs]))
    ap_bytes = append_alg_bytes(full)
    ap_gbs = ap_bytes / (ap_ms * 1e-3) / 1e9

    dec_bytes = decode_alg_bytes(dc)
    pf_flops = prefill_alg_flops(pf)
    dec_gbs = dec_bytes / (dc_ms * 1e-3) / 1e9
    pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12

    # the same step with attention as one mixed launch (pa_mixed_attention:
    # the chunks' row tiles and the decode (request, KV head) items in one
    # grid, no merge pass), timed the same way
    mx_q = to_dev(full.q, full.dtype)
    mx_out = torch.empty_like(mx_q)
    mx_lse = torch.empty(full.total_q, full.num_q_heads, dtype=torch.float32, device=dev)
    mx_desc = pa.make_desc(mx_q, pools[0][0], full_t["pt"], full_t["sl"], full.max_seq_len,
                           full.max_q_len)
    for i in (0, 1):
        kp, vp = pools[i]
        calls[("mixed", i)] = pa.bind_mixed_attention(
            mx_q, kp, vp, full_t["pt"], full_t["sl"], full_t["qo"], full.scale,
            q_starts=full_t["qs"], out=mx_out, lse=mx_lse, desc=mx_desc)

    def step_single(i, ev=None):
        if ev is not None:
            ev[0].record()
        calls[("append", i & 1)]()
        if ev is not None:
            ev[1].record()
        calls[("mixed", i & 1)]()
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        step_single(i)
    torch.cuda.synchronize()
    evm = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_single(i, evm[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mx_step_ms = (t1 - t0) * 1e3 / args.steps
    mx_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evm]))
    single = {
        "ms_per_step": round(mx_step_ms, 4), "attention_ms": round(mx_ms, 4),
        "kernel": "mixed_kernel<128,4>",
        "traffic": load_traffic("mixed", source_hash("mixed.hip", "prefill_core.h", "decode_core.h")),
        "attention_ms_separate_routes": round(pf_ms + dc_ms, 4),
        "speedup_vs_separate_routes": round((pf_ms + dc_ms) / mx_ms, 3),
        # the share of each roofline the one launch reaches over its own time
        "hbm_frac": round(dec_bytes / (mx_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(pf_flops / (mx_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
    }

    pf_hash = source_hash("prefill.hip", "prefill_core.h")
    dc_hash = source_hash("decode.hip", "decode_core.h", "merge.hip")
    kernels = {
        "prefill": {"bound": "mfma", "achieved": round(pf_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": load_traffic("prefill", pf_hash), "ms": round(pf_ms, 4),
                    "kernel": "prefill_kernel<128>", "work": pf_flops, "work_unit": "FLOP"},
        "decode": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "traffic": load_traffic("decode", dc_hash), "ms": round(dc_ms, 4),
                   "kernel": ("decode_mfma_kernel<128,4> + merge_kernel"
                              if dc_plan["path"] == "decode_balanced" else
                              f"decode_kernel<bf16,128,4> x{dc_plan['num_splits']} + merge_kernel"),
                   "work": dec_bytes, "work_unit": "B"},
    }
    kernels["append"] = {"bound": "hbm", "achieved": round(ap_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ap_gbs / HBM_PEAK_GBS, 4),
                         "traffic": load_traffic("append", source_hash("append.hip")),
                         "ms": round(ap_ms, 4), "kernel": "append_flat_kernel",
                         "work": ap_bytes, "work_unit": "B"}
    dominant = "prefill" if pf_ms >= dc_ms else "decode"
    roof = {k: kernels[dominant][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = kernels[dominant]["kernel"]

    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "mixed continuous-batching step, Qwen3-4B attention heads (32q/8kv, d=128)",
            "append": "new K/V rows of the step (2048 chunk tokens + 60 decode tokens) into their page slots",
            "prefill": "4 chunks x 512 tokens at offsets 0/512/1536/3072, causal",
            "decode": "60 rows, contexts U[256,4096], seed %d" % full.seed,
            "page_size": 16, "pool_pages": full.num_pages, "global_batch": 64,
            "decode_plan": dc_plan, "prefill_plan": pf_plan,
        },
        "prefill_tflops": round(pf_tflops, 2),
        "prefill_frac_of_mfma_peak": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "decode_frac_of_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4),
        "kernels": kernels,
        "single_launch": single,
        "roofline": roof,
        "cpu_baseline": None,
    }
    # after the timed region: the rate of the decode route's read pattern on
    # this device (random 4 KiB blocks), against which the route's GB/s is
    # also given
    try:
        ref = read_reference()
        result["hbm_read_reference"] = {
            "pattern": "pa_read_blocks: 2 GiB in 4 KiB blocks (one (page, KV head) K or V block), random order, "
                       "nontemporal 16-byte loads",
            "GB/s": ref["4KiB_random"]["GB/s"],
            "decode_frac": round(dec_gbs / ref["4KiB_random"]["GB/s"], 4),
            "all": ref,
        }
    except (RuntimeError, torch.cuda.OutOfMemoryError) as e:   # the reference is context, not the metric
        print(f"read reference skipped: {e}", file=sys.stderr)
        result["hbm_read_reference"] = None
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(full, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
