#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, resident in HBM:
  * forward, B=8 H=16 N=2048 d=128 bf16, non-causal        (fa_fwd)
  * forward, same inputs, causal                           (fa_fwd)
  * paged-KV decode, 64 sequences of 128..8192 tokens, H=32, d=128, pages of 16,
    shuffled pool, pairs sharing a 512-token prefix        (fa_paged_decode)

`value` is the forward throughput in TFLOP/s (algorithmic FLOPs of the two
forward calls over their kernel time, HIP events on the launch stream).  The
decode's HBM GB/s, per-call figures, the roofline of the dominant kernel and
the CPU oracle's rate on a bounded sample are reported in the same JSON line.
The backward pass (fa_bwd) of both forward calls, a paged prefill
(fa_paged_prefill: 16 sequences with 0..4096 cached tokens receiving 256..1792
new ones, H=32, d=128, causal) and a draft-tree verification (fa_tree_decode:
64 sequences of 128..8192 committed tokens, 64-node trees, H=32, d=128) and
the forward with RoPE (fa_fwd_rope, query rotation fused, against fa_rope on
q and k followed by fa_fwd) are timed after the steps, each in a loop of its
own, and reported under "bwd", "prefill", "tree" and "rope" (they are not part
of the step).  As context for the MFMA fractions, "mfma_ceiling" gives what a
plain 8192^3 bf16 GEMM through the vendor BLAS (torch.matmul) reaches on the
same GPU in the same run (under sustained matrix load the chip runs below the
clock its published peak assumes), "hbm_ceiling" what a plain 2 GiB device
copy reaches against the published HBM bandwidth, and "hbm_read_ceiling" what a
read-only probe (libfa_probe.so) reaches sequentially and over 4 KiB chunks in
random order, the grain of the paged kernels' reads.  "sweep" times the forward
on the other configurations, on their seeded inputs: the sequence sweep at 16k
tokens (N = 512 .. 16384, H=32, d=64, both masks) and the long-context one
(B=1 H=16 N=16384 d=128, causal).  The decode is also timed with 512 MiB
written between calls ("decode.flushed"), so that no call finds the previous
call's pages in the last-level cache.

"cpu_baseline" is the fp64 oracle timed on this host before the GPU is used:
every (b, h) head of the forward bench in both masks and every (sequence, head)
pair of the decode, over a process pool of one worker per core of the
process's affinity (BLAS pinned to one thread each); it reports the core
count, the BLAS library and both rates.  "parity" holds the max-abs errors of
O and LSE against that oracle for every configuration: the fp32 smoke one in
full, the forward bench at sampled rows of every head, the sweep and the
long-context one at sampled rows of two heads, the decode in full.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--min-warmup-s 1.0]
                    [--no-cpu-baseline] [--skip-bwd] [--skip-prefill] [--skip-tree] [--skip-rope]
                    [--skip-sweep] [--skip-gemm]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6       # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0           # HBM3E, 8 TB/s
METRIC = "attention fwd TFLOP/s & % bf16 MFMA peak; paged decode HBM GB/s (1 GPU)"


def fwd_flops(B, H, N, d, causal):
    """Algorithmic FLOPs: 4*N^2*d per head (2 for QK^T, 2 for PV); causal counts
    only the N(N+1)/2 visible pairs.  Masked work and exponentials not counted."""
    return 2.0 * B * H * d * N * (N + 1) if causal else 4.0 * B * H * N * N * d


def fwd_bytes(B, H, N, d):
    """Algorithmic HBM bytes of a bf16 forward: q, k, v read once, o written
    once (2 bytes each), and the fp32 log-sum-exp of every row."""
    return B * H * N * (4 * d * 2 + 4)


def fwd_roof_tflops(B, H, N, d, causal):
    """The forward's roofline: the bf16 matrix peak, or the HBM rate times the
    FLOPs per algorithmic byte when that is lower (short causal sequences)."""
    intensity = fwd_flops(B, H, N, d, causal) / fwd_bytes(B, H, N, d)
    return min(PEAK_BF16_TFLOPS, PEAK_HBM_GBS * 1e9 * intensity / 1e12)


def bwd_flops(B, H, N, d, causal):
    """Algorithmic backward FLOPs: the five N x N x d products of the gradient
    (S recomputed, dP, dV, dQ, dK), 2.5x the forward's.  The dK/dV and dQ
    kernels recompute S and dP once more each; that extra work is not counted."""
    return 2.5 * fwd_flops(B, H, N, d, causal)


def prefill_flops(wl, causal=True):
    """Algorithmic FLOPs of a paged prefill: 4*d per (new query, visible key)
    pair and head; causal query i of n new ones in a sequence of L tokens
    sees L - n + i + 1 keys."""
    L = wl.layout
    pairs = 0
    for s in range(L.S):
        n, total = int(wl.new_lens[s]), int(L.seq_lens[s])
        if causal:
            first = total - n + 1
            pairs += n * first + n * (n - 1) // 2
        else:
            pairs += n * total
    return 4.0 * L.d * L.H * pairs


def tree_work(wl, parents):
    """Algorithmic FLOPs and HBM bytes of a tree verification: 4*d flops per
    (node, visible key) pair and head; bytes = every distinct (page, head) row
    any node sees (K and V, shared pages once) plus q, o, lse, the used table
    entries, seq_lens, cu_seqlens_q and the parents."""
    from exact_attention_26_amd.workloads import page_valid_slots
    L = wl.layout
    pairs = 0
    for s in range(L.S):
        lo, hi = int(wl.cu_seqlens_q[s]), int(wl.cu_seqlens_q[s + 1])
        ctx = int(L.seq_lens[s]) - (hi - lo)
        depth = []                             # nodes on each node's path from the root
        for i in range(hi - lo):
            p = int(parents[lo + i])
            depth.append(1 + (depth[p] if 0 <= p < i else 0))
        pairs += sum(ctx + k for k in depth)
    flops = 4.0 * L.d * L.H * pairs
    kv = float(page_valid_slots(L).sum()) * L.H * L.d * 2 * 2
    pages_used = sum(L.used_pages(s).size for s in range(L.S))
    small = wl.total_q * L.H * (L.d * 2 * 2 + 4) + pages_used * 4 + L.S * 8 + wl.total_q * 4
    return flops, kv + small


def decode_bytes(layout):
    """Algorithmic HBM bytes of one decode call: every K/V row a query must see,
    each distinct physical (page, head) row once, plus q, o, lse, the used
    table entries and seq_lens."""
    from exact_attention_26_amd.workloads import page_valid_slots
    valid = page_valid_slots(layout)
    kv = float(valid.sum()) * layout.H * layout.d * 2 * 2
    logical = float(np.maximum(layout.seq_lens, 0).sum()) * layout.H * layout.d * 2 * 2
    pages_used = sum(layout.used_pages(s).size for s in range(layout.S))
    small = layout.S * layout.H * layout.d * 2 * 2 + layout.S * layout.H * 4 + pages_used * 4 \
        + layout.S * 4
    return kv + small, logical + small


def measured_traffic(kernel_key: str):
    """HBM bytes per launch (read + written) from the committed counter summary
    profiles/traffic.json, or None when any source the kernel is built from
    changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)["kernels"][kernel_key]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    if h.hexdigest()[:16] != rec["sha256_16"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


# ---------------------------------------------------------------------------
# the CPU baseline leg: the fp64 oracle timed on this host, and the GPU results
# checked against it.  Nothing outside these functions touches the oracle.
# ---------------------------------------------------------------------------
_ORC = {}                       # host inputs the forked oracle workers read


def _blas_info():
    """BLAS library numpy uses, and its thread count in this process."""
    try:
        from threadpoolctl import threadpool_info
        infos = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if infos:
            p = infos[0]
            return (f"{p.get('internal_api')} {p.get('version')} ({p.get('architecture')}, "
                    f"{p.get('threading_layer')})", max(x.get("num_threads", 1) for x in infos))
    except Exception:
        pass
    return f"numpy {np.__version__}, BLAS not identified", None


def _oracle_worker_init():
    """One BLAS thread per worker: the pool supplies the parallelism."""
    global _ORC_LIMIT
    from threadpoolctl import threadpool_limits
    _ORC_LIMIT = threadpool_limits(1)


def _oracle_fwd_head(task):
    """One (b, h) head of the forward bench workload: the full oracle, timed;
    returns the rows in _ORC['c1_rows'] for the parity check."""
    from oracle import attention_fp64
    causal, b, h = task
    q, k, v, scale = _ORC["c1"]
    t0 = time.perf_counter()
    o, lse = attention_fp64(q[b, h], k[b, h], v[b, h], causal=causal, scale=scale)
    dt = time.perf_counter() - t0
    rows = _ORC["c1_rows"]
    return dt, o[rows], lse[rows]


def _oracle_decode(task):
    """Some (sequence, head) pairs of the decode workload, timed."""
    from oracle import paged_decode_fp64
    q, kc, vc, table, lens, scale = _ORC["c4"]
    t0 = time.perf_counter()
    o, lse = paged_decode_fp64(q, kc, vc, table, lens, scale=scale, pairs=task)
    return time.perf_counter() - t0, o, lse


def cpu_baseline_run(cfg, c1, c4_layout, c4_pools, c4_q):
    """Time the oracle, as it stands, on the host cores: every (b, h) head of
    the forward bench workload in both masks, and every (sequence, head) pair of
    the paged decode, mapped over a process pool (one worker per core of this
    process's affinity, BLAS pinned to one thread each).  Must run before the
    GPU is touched (the pool is forked).  Returns the report and the oracle's
    results for the parity check."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    blas, blas_threads = _blas_info()
    q, k, v = c1
    _ORC["c1"] = (q, k, v, cfg.scale)
    _ORC["c1_rows"] = _parity_rows(cfg.N)
    L = c4_layout
    _ORC["c4"] = (c4_q, c4_pools[0], c4_pools[1], L.block_table, L.seq_lens, L.scale)
    tasks = [(causal, b, h) for causal in (False, True) for b in range(cfg.B) for h in range(cfg.H)]
    pairs = [(s, h) for s in range(L.S) for h in range(L.H)]
    chunks = [pairs[i:i + 16] for i in range(0, len(pairs), 16)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_oracle_worker_init) as pool:
        t0 = time.perf_counter()
        fwd = pool.map(_oracle_fwd_head, tasks, chunksize=1)
        t_fwd = time.perf_counter() - t0
        t0 = time.perf_counter()
        dec = pool.map(_oracle_decode, chunks, chunksize=1)
        t_dec = time.perf_counter() - t0
    n = len(tasks) // 2
    flops = fwd_flops(1, n, cfg.N, cfg.d, False) + fwd_flops(1, n, cfg.N, cfg.d, True)
    dec_bytes, _ = decode_bytes(L)
    report = {
        "value": flops / t_fwd / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": (f"all {n} (b,h) heads of the forward B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} "
                   f"in both masks ({2 * n} oracle calls), fp64 numpy oracle, {cores} worker "
                   f"processes, {t_fwd:.1f} s wall"),
        "workers": cores, "blas": blas, "blas_threads_in_parent": blas_threads,
        "blas_threads_per_worker": 1,
        "decode": {"value": dec_bytes / t_dec / 1e9, "unit": "GB/s",
                   "sample": (f"all {len(pairs)} (sequence, head) pairs of the paged decode "
                              f"S={L.S} H={L.H} d={L.d}, {t_dec:.1f} s wall"),
                   "seconds": round(t_dec, 3)},
        "seconds": round(t_fwd, 3)}
    oracle = {
        "c1": {(causal, b, h): (o, l) for (causal, b, h), (_, o, l) in zip(tasks, fwd)},
        "c4": (np.concatenate([o for _, o, _ in dec]).reshape(L.S, L.H, L.d),
               np.concatenate([l for _, _, l in dec]).reshape(L.S, L.H))}
    return report, oracle


def _parity_rows(N):
    """Query rows sampled for the parity check: wave and block edges, the
    middle, the end, and a seeded random dozen."""
    rng = np.random.default_rng(77)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 2, N - 1]
    rows = np.concatenate([np.array(fixed), rng.choice(N, size=min(12, N), replace=False)])
    return np.unique(np.clip(rows, 0, N - 1))


def _max_abs(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    fin = np.isfinite(want)
    if not np.array_equal(np.isfinite(got), fin) or not np.array_equal(got[~fin], want[~fin]):
        return float("inf")
    return float(np.max(np.abs(got[fin] - want[fin]))) if fin.any() else 0.0


def cpu_baseline_parity(samples, oracle, c4_layout):
    """Max-abs error of the GPU results on O and LSE against the oracle, per
    configuration: the smoke one in full, the forward bench at the sampled rows
    of every head (both masks), the sweep and the long-context one at the
    sampled rows of two heads per mode, the decode in full."""
    from oracle import attention_fp64
    out = {}
    smoke = samples.get("smoke")
    if smoke is not None:
        (q, k, v, scale), (o, lse) = smoke
        ro, rl = attention_fp64(q, k, v, causal=False, scale=scale)
        out["smoke B=1 H=2 N=256 d=64 fp32"] = {"o_max_abs": _max_abs(o, ro),
                                                "lse_max_abs": _max_abs(lse, rl), "rows": "all"}
    c1 = samples.get("c1")
    if c1 is not None and oracle is not None:
        for causal in (False, True):
            eo = el = 0.0
            for (cz, b, h), (ro, rl) in oracle["c1"].items():
                if cz != causal:
                    continue
                go, gl = c1[causal]
                eo = max(eo, _max_abs(go[b, h], ro))
                el = max(el, _max_abs(gl[b, h], rl))
            out[f"fwd B=8 H=16 N=2048 d=128 {'causal' if causal else 'non-causal'}"] = {
                "o_max_abs": eo, "lse_max_abs": el,
                "rows": f"{len(_parity_rows(2048))} sampled rows of all 128 heads"}
    for name, (cfgc, heads, rows, modes) in samples.get("sweep", {}).items():
        for causal, (q, k, v, go, gl) in modes.items():
            eo = el = 0.0
            for i, (b, h) in enumerate(heads):
                ro, rl = attention_fp64(q[i], k[i], v[i], causal=causal, scale=cfgc.scale,
                                        rows=rows)
                eo = max(eo, _max_abs(go[i], ro))
                el = max(el, _max_abs(gl[i], rl))
            out[f"{name} {'causal' if causal else 'non-causal'}"] = {
                "o_max_abs": eo, "lse_max_abs": el,
                "rows": f"{len(rows)} sampled rows of heads {heads}"}
    dec = samples.get("c4")
    if dec is not None and oracle is not None:
        ro, rl = oracle["c4"]
        out["paged decode S=64 H=32 d=128"] = {"o_max_abs": _max_abs(dec[0], ro),
                                               "lse_max_abs": _max_abs(dec[1], rl),
                                               "rows": "all (sequence, head) pairs"}
    for v in out.values():
        v["o_max_abs"] = float(f"{v['o_max_abs']:.3e}")
        v["lse_max_abs"] = float(f"{v['lse_max_abs']:.3e}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-s", type=float, default=1.0,
                    help="after the W warmup steps, keep warming each timed section until this "
                         "much wall time has passed (the GPU's clocks ramp up under sustained "
                         "load; a few milliseconds of warmup measure a partly idle GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true",
                    help="forward only (for profiling the forward kernel alone)")
    ap.add_argument("--skip-bwd", action="store_true", help="do not time the backward pass")
    ap.add_argument("--skip-prefill", action="store_true", help="do not time the paged prefill")
    ap.add_argument("--skip-tree", action="store_true", help="do not time the tree verification")
    ap.add_argument("--skip-rope", action="store_true", help="do not time the RoPE forward")
    ap.add_argument("--skip-sweep", action="store_true",
                    help="do not time the forward over the sequence sweep (d=64) and the "
                         "long-context configuration")
    ap.add_argument("--skip-gemm", action="store_true",
                    help="do not time the plain bf16 GEMM (the MFMA throughput the vendor BLAS "
                         "reaches on this GPU, reported next to the attention figures)")
    ap.add_argument("--only", choices=["fwd-noncausal", "fwd-causal", "decode", "bwd-noncausal",
                                       "bwd-causal", "prefill", "tree", "rope", "gemm", "sweep"],
                    help="run one call per step (for per-kernel counter runs)")
    ap.add_argument("--probe-copy", type=int, metavar="MIB",
                    help="instead of the hot path, copy a buffer of MIB MiB a few times "
                         "(a plain copy kernel of known size, to calibrate byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-GPU and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_26_amd as fa
    from exact_attention_26_amd import workloads as w
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)  # noqa: E731

    # ---- host inputs: the forward bench workload and the paged decode, drawn
    #      before the GPU is touched (the CPU baseline's worker pool is forked
    #      from this process and reads them)
    cfg = w.FWD_CONFIGS["fwd_b8_h16_n2048_d128"]
    decode = not args.skip_decode and args.only in (None, "decode") and not args.probe_copy
    with_cpu = (not args.no_cpu_baseline and args.only is None and decode
                and not args.probe_copy)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    c1_host = w.fwd_config_inputs(cfg) if not args.probe_copy else None
    if decode:
        L = w.decode_layout(**w.DECODE_C4)
        qdec_host = w.decode_q(L)
        pools_host = [w.decode_pool(L, which, poison=False, threads=threads)
                      for which in ("k", "v")]
    log("host inputs ready")
    cpu_report = oracle_res = None
    if with_cpu:
        log("timing the CPU oracle (forward bench and paged decode, all heads)")
        cpu_report, oracle_res = cpu_baseline_run(cfg, c1_host, L, pools_host, qdec_host)
        log(f"CPU oracle timed: {cpu_report['value']:.4f} TFLOP/s, "
            f"{cpu_report['decode']['value']:.2f} GB/s on {cpu_report['cores']} cores")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.probe_copy:
        n = args.probe_copy * 2 ** 20 // 4
        src = torch.arange(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"probe_copy_bytes_each_way": n * 4, "copies": max(1, args.steps)}))
        return

    def time_calls(fn):
        """Mean milliseconds of fn() over --steps calls, from HIP events recorded
        on the launch stream around each call.  All calls are enqueued before
        the one synchronisation at the end, so the GPU runs them back to back
        and no interval contains host time spent enqueueing the next call."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / args.steps

    def warm_up(fn):
        """W untimed calls, then more until --min-warmup-s of wall time has passed."""
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + args.min_warmup_s
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()

    samples = {}                 # GPU results the oracle leg checks (host copies)

    # ---- forward inputs on the device ----
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in c1_host)
    del c1_host
    o_nc = torch.empty_like(qd)
    o_c = torch.empty_like(qd)
    lse_nc = torch.empty(qd.shape[:-1], dtype=torch.float32, device=dev)
    lse_c = torch.empty_like(lse_nc)
    log("forward inputs ready")

    # ---- decode inputs on the device ----
    if decode:
        qdec = torch.from_numpy(qdec_host).to(dev).to(torch.bfloat16)
        pools = []
        for host in pools_host:
            pool = torch.empty((L.num_blocks, L.H, L.page_size, L.d), dtype=torch.bfloat16,
                               device=dev)
            for lo in range(0, L.num_blocks, w.POOL_CHUNK_PAGES):
                hi = min(L.num_blocks, lo + w.POOL_CHUNK_PAGES)
                pool[lo:hi].copy_(torch.from_numpy(host[lo:hi]).to(dev))
            pools.append(pool)
        del pools_host, host
        kc, vc = pools
        bt = torch.from_numpy(L.block_table).to(dev)
        sl = torch.from_numpy(L.seq_lens).to(dev)
        ws = torch.empty(fa.fa_paged_decode_workspace_size(L.S, L.H, L.d, L.page_size,
                                                            L.max_blocks),
                         dtype=torch.uint8, device=dev)
        o_dec = torch.empty_like(qdec)
        lse_dec = torch.empty((L.S, L.H), dtype=torch.float32, device=dev)
        dec_bytes, dec_logical = decode_bytes(L)
        log(f"decode inputs ready: {L.num_blocks} pages, sum L = {int(L.seq_lens.sum())}")

    stream = torch.cuda.current_stream(dev)

    run_nc = args.only in (None, "fwd-noncausal", "bwd-noncausal")
    run_c = args.only in (None, "fwd-causal", "bwd-causal")
    run_dec = decode and args.only in (None, "decode")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if run_nc:
            fa.fa_fwd(qd, kd, vd, o_nc, lse_nc, False, cfg.scale)
        if ev is not None:
            ev[1].record(stream)
        if run_c:
            fa.fa_fwd(qd, kd, vd, o_c, lse_c, True, cfg.scale)
        if ev is not None:
            ev[2].record(stream)
        if run_dec:
            fa.fa_paged_decode(qdec, kc, vc, bt, sl, o_dec, lse_dec, L.scale, ws)
        if ev is not None:
            ev[3].record(stream)

    warm_up(step)
    log("warmup done")

    # whole-step wall time (no per-call syncs inside)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-call kernel times from HIP events on the launch stream: every step's
    # events are enqueued with it and read after one final synchronisation
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    per_call = [[ev[i].elapsed_time(ev[i + 1]) for ev in evs] for i in range(3)]
    t_nc, t_c, t_dec = (sum(x) / args.steps for x in per_call)
    med_min = [(round(float(np.median(x)), 4), round(min(x), 4)) for x in per_call]
    log("timed steps done")

    f_nc = fwd_flops(cfg.B, cfg.H, cfg.N, cfg.d, False)
    f_c = fwd_flops(cfg.B, cfg.H, cfg.N, cfg.d, True)
    # (in --only modes without a forward the intervals are empty)
    tflops_nc = f_nc / (t_nc * 1e-3) / 1e12 if t_nc > 0 else 0.0
    tflops_c = f_c / (t_c * 1e-3) / 1e12 if t_c > 0 else 0.0
    value = (f_nc + f_c) / ((t_nc + t_c) * 1e-3) / 1e12 if t_nc + t_c > 0 else 0.0

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention forward B=8 H=16 N=2048 d=128 bf16 (non-causal + causal)"
                               + (" + paged-KV decode S=64 H=32 d=128 page=16 L=128..8192"
                                  if decode else ""),
                   "global_batch": cfg.B, "seq_len": cfg.N, "heads": cfg.H, "head_dim": cfg.d,
                   "parallelism": "single GPU"},
        "fwd": {"noncausal_ms": round(t_nc, 4), "noncausal_tflops": round(tflops_nc, 2),
                "noncausal_frac_peak": round(tflops_nc / PEAK_BF16_TFLOPS, 4),
                "noncausal_ms_median_min": med_min[0] if run_nc else None,
                "causal_ms": round(t_c, 4), "causal_tflops": round(tflops_c, 2),
                "causal_frac_peak": round(tflops_c / PEAK_BF16_TFLOPS, 4),
                "causal_ms_median_min": med_min[1] if run_c else None,
                "causal_traffic": measured_traffic(
                    "fwd_bf16_persist_kernel<128,true> B=8 H=16 N=2048"),
                "kernels": "fwd_bf16_persist_kernel<128,false>, <128,true>"},
        "roofline": {"bound": "mfma", "achieved": round(tflops_nc, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops_nc / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(
                         "fwd_bf16_persist_kernel<128,false> B=8 H=16 N=2048"),
                     "kernel": "fwd_bf16_persist_kernel<128,false>",
                     "flops_per_launch": f_nc},
    }
    # the step's last results, at the rows the oracle leg checks
    if with_cpu:
        rows = torch.from_numpy(_parity_rows(cfg.N)).to(dev)
        samples["c1"] = {c: (o_.index_select(2, rows).float().cpu().numpy(),
                             l_.index_select(2, rows).cpu().numpy())
                         for c, (o_, l_) in ((False, (o_nc, lse_nc)), (True, (o_c, lse_c)))}
        if run_dec:
            samples["c4"] = (o_dec.float().cpu().numpy(), lse_dec.cpu().numpy())
    if decode:
        gbs = dec_bytes / (t_dec * 1e-3) / 1e9
        # the same decode with 512 MiB written between calls (more than the
        # 256 MB last-level cache), so no call finds the previous one's pages
        # there; only the decode sits between the events
        flush = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        dcall = lambda: fa.fa_paged_decode(qdec, kc, vc, bt, sl, o_dec, lse_dec, L.scale, ws)  # noqa: E731
        warm_up(dcall)
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (a, b) in enumerate(fev):
            flush.fill_(i & 255)
            a.record(stream)
            dcall()
            b.record(stream)
        torch.cuda.synchronize()
        t_flushed = sum(a.elapsed_time(b) for a, b in fev) / args.steps
        del flush
        gbs_flushed = dec_bytes / (t_flushed * 1e-3) / 1e9
        out["decode"] = {"ms": round(t_dec, 4), "ms_median_min": med_min[2],
                         "hbm_gbs": round(gbs, 1),
                         "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": dec_bytes, "logical_bytes": dec_logical,
                         "logical_gbs": round(dec_logical / (t_dec * 1e-3) / 1e9, 1),
                         "flushed": {"ms": round(t_flushed, 4), "hbm_gbs": round(gbs_flushed, 1),
                                     "frac_peak": round(gbs_flushed / PEAK_HBM_GBS, 4),
                                     "between_calls": "512 MiB device write (cache flush)"}}
        out["roofline_decode"] = {"bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(gbs / PEAK_HBM_GBS, 4),
                                  "traffic": measured_traffic("decode_partial_kernel<128> C4")}
    # ---- backward of both forward calls, its own timed loop ----
    bwd_modes = [] if args.skip_bwd else [m for m in (False, True)
                                          if args.only in (None, f"bwd-{'causal' if m else 'noncausal'}")]
    t_bwd = {}
    if bwd_modes:
        do = torch.from_numpy(w.bwd_dout(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)).to(dev)
        do = do.to(torch.bfloat16)
        wsb = torch.empty(fa.fa_bwd_workspace_size(cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.uint8,
                          device=dev)
        dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
        fwd_out = {False: (o_nc, lse_nc), True: (o_c, lse_c)}
        for causal in bwd_modes:
            o_, lse_ = fwd_out[causal]
            warm_up(lambda: fa.fa_bwd(qd, kd, vd, o_, lse_, do, dq, dk, dv, causal, cfg.scale,
                                      wsb))
            t_bwd[causal] = time_calls(
                lambda: fa.fa_bwd(qd, kd, vd, o_, lse_, do, dq, dk, dv, causal, cfg.scale, wsb))
        log("backward timed")
        out["bwd"] = {}
        for causal in bwd_modes:
            tag = "causal" if causal else "noncausal"
            tf = bwd_flops(cfg.B, cfg.H, cfg.N, cfg.d, causal) / (t_bwd[causal] * 1e-3) / 1e12
            out["bwd"].update({f"{tag}_ms": round(t_bwd[causal], 4), f"{tag}_tflops": round(tf, 2),
                               f"{tag}_frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        out["bwd"]["flops"] = "2.5x forward (10 N^2 d per head non-causal)"
        out["bwd"]["traffic"] = {k: measured_traffic(f"{k} B=8 H=16 N=2048") for k in (
            "bwd_dkdv_kernel<128,false>", "bwd_dq_kernel<128,false>")}

    # ---- paged prefill, its own timed loop ----
    t_pre = None
    if not args.skip_prefill and args.only in (None, "prefill"):
        wl = w.prefill_workload(**w.PREFILL_P1)
        Lp = wl.layout
        qp = torch.from_numpy(w.prefill_q(wl)).to(dev).to(torch.bfloat16)
        ppools = []
        for which in ("k", "v"):
            pool = torch.empty((Lp.num_blocks, Lp.H, Lp.page_size, Lp.d), dtype=torch.bfloat16,
                               device=dev)

            def putp(lo, hi, x, pool=pool):
                pool[lo:hi].copy_(torch.from_numpy(x).to(dev))
            w.decode_pool(Lp, which, poison=False, chunk_callback=putp)
            ppools.append(pool)
        btp = torch.from_numpy(Lp.block_table).to(dev)
        slp = torch.from_numpy(Lp.seq_lens).to(dev)
        cup = torch.from_numpy(wl.cu_seqlens_q).to(dev)
        op_ = torch.empty_like(qp)
        lsep = torch.empty((wl.total_q, Lp.H), dtype=torch.float32, device=dev)

        def pcall():
            fa.fa_paged_prefill(qp, ppools[0], ppools[1], btp, slp, cup, op_, lsep, wl.max_q_len,
                                True, Lp.scale)
        warm_up(pcall)
        t_pre = time_calls(pcall)
        fl = prefill_flops(wl, True)
        tf = fl / (t_pre * 1e-3) / 1e12
        out["prefill"] = {"ms": round(t_pre, 4), "tflops": round(tf, 2),
                          "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "causal": True,
                          "new_tokens": wl.total_q, "cached_tokens": int(Lp.seq_lens.sum()),
                          "flops": fl,
                          "traffic": measured_traffic("prefill_bf16_kernel<128,true> P1")}
        log("prefill timed")

    # ---- draft-tree verification, its own timed loop ----
    t_tree = None
    tree_gbs = None
    if not args.skip_tree and args.only in (None, "tree"):
        wlt, part = w.tree_workload(**w.TREE_T1)
        Lt = wlt.layout
        qt_ = torch.from_numpy(w.prefill_q(wlt)).to(dev).to(torch.bfloat16)
        tpools = []
        for which in ("k", "v"):
            pool = torch.empty((Lt.num_blocks, Lt.H, Lt.page_size, Lt.d), dtype=torch.bfloat16,
                               device=dev)

            def putt(lo, hi, x, pool=pool):
                pool[lo:hi].copy_(torch.from_numpy(x).to(dev))
            w.decode_pool(Lt, which, poison=False, chunk_callback=putt)
            tpools.append(pool)
        btt = torch.from_numpy(Lt.block_table).to(dev)
        slt = torch.from_numpy(Lt.seq_lens).to(dev)
        cut = torch.from_numpy(wlt.cu_seqlens_q).to(dev)
        prt = torch.from_numpy(part).to(dev)
        ot = torch.empty_like(qt_)
        lset = torch.empty((wlt.total_q, Lt.H), dtype=torch.float32, device=dev)

        def tcall():
            fa.fa_tree_decode(qt_, tpools[0], tpools[1], btt, slt, cut, prt, ot, lset,
                              wlt.max_q_len, Lt.scale)
        warm_up(tcall)
        t_tree = time_calls(tcall)
        fl, by = tree_work(wlt, part)
        tree_gbs = by / (t_tree * 1e-3) / 1e9
        out["tree"] = {"ms": round(t_tree, 4),
                       "tflops": round(fl / (t_tree * 1e-3) / 1e12, 2),
                       "hbm_gbs": round(tree_gbs, 1),
                       "hbm_frac_peak": round(tree_gbs / PEAK_HBM_GBS, 4),
                       "nodes": wlt.total_q, "committed_tokens": int(Lt.seq_lens.sum()) - wlt.total_q,
                       "flops": fl, "algorithmic_bytes": by,
                       "traffic": measured_traffic("tree_bf16_kernel<128> T1")}
        log("tree timed")

    # ---- forward with RoPE: fused query rotation vs rotate-then-attend ----
    t_rope = None
    if not args.skip_rope and args.only in (None, "rope"):
        rc, rs = (torch.from_numpy(t).to(dev) for t in w.rope_tables(cfg.N, cfg.d))
        wsr = torch.empty(fa.fa_fwd_rope_workspace_size(cfg.B, cfg.H, cfg.N, cfg.d),
                          dtype=torch.uint8, device=dev)
        # the unfused path rotates k into the same workspace the fused call
        # uses, so both read their keys from the same memory (the forward's
        # speed depends on where its operands sit, by up to ~15%)
        qrot = torch.empty_like(qd)
        krot = wsr.view(torch.bfloat16).view(qd.shape)
        orr = torch.empty_like(qd)
        lsr = torch.empty_like(lse_nc)
        def timed(fn):
            warm_up(fn)
            return time_calls(fn)

        out["rope"] = {}
        for causal in (False, True):
            tag = "causal" if causal else "noncausal"

            def fused():
                fa.fa_fwd_rope(qd, kd, vd, orr, lsr, rc, rs, causal, cfg.scale, wsr)

            def unfused():
                fa.fa_rope(qd, qrot, rc, rs)
                fa.fa_rope(kd, krot, rc, rs)
                fa.fa_fwd(qrot, krot, vd, orr, lsr, causal, cfg.scale)
            tf_, tu_ = timed(fused), timed(unfused)
            fl = fwd_flops(cfg.B, cfg.H, cfg.N, cfg.d, causal)
            out["rope"].update({f"{tag}_fused_ms": round(tf_, 4), f"{tag}_unfused_ms": round(tu_, 4),
                                f"{tag}_fused_tflops": round(fl / (tf_ * 1e-3) / 1e12, 2)})
            if not causal:
                t_rope = tf_
        log("rope timed")

    # ---- the other forward configurations: the sequence sweep at 16k tokens
    #      (H=32, d=64) and the long-context one (B=1 H=16 N=16384 d=128,
    #      causal, q and k with standard deviation 3), on their seeded inputs
    if not args.skip_sweep and args.only in (None, "sweep"):
        out["sweep"] = {}
        samples["sweep"] = {}
        for name, c in w.FWD_CONFIGS.items():
            if not (name.startswith("sweep_") or name.startswith("long_")):
                continue
            host = w.fwd_config_inputs(c)
            qs, ks, vs = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in host)
            os_ = torch.empty_like(qs)
            ls = torch.empty(qs.shape[:-1], dtype=torch.float32, device=dev)
            heads = [(0, 0), (c.B - 1, c.H - 1)]
            prow = _parity_rows(c.N)
            prow_d = torch.from_numpy(prow).to(dev)
            modes = {}
            row = {}
            for causal in c.causal:
                fn = lambda: fa.fa_fwd(qs, ks, vs, os_, ls, causal, c.scale)  # noqa: E731
                warm_up(fn)
                t = time_calls(fn)
                tag = "causal" if causal else "noncausal"
                tf = fwd_flops(c.B, c.H, c.N, c.d, causal) / (t * 1e-3) / 1e12
                roof = fwd_roof_tflops(c.B, c.H, c.N, c.d, causal)
                row[f"{tag}_ms"] = round(t, 4)
                row[f"{tag}_tflops"] = round(tf, 2)
                row[f"{tag}_roof_tflops"] = round(roof, 1)
                row[f"{tag}_frac_roof"] = round(tf / roof, 4)
                if with_cpu:
                    modes[causal] = tuple(np.stack([x[b, h] for b, h in heads]) for x in host) + (
                        np.stack([os_[b, h].index_select(0, prow_d).float().cpu().numpy()
                                  for b, h in heads]),
                        np.stack([ls[b, h].index_select(0, prow_d).cpu().numpy()
                                  for b, h in heads]))
            out["sweep"][f"B={c.B} H={c.H} N={c.N} d={c.d}"] = row
            if with_cpu:
                samples["sweep"][f"B={c.B} H={c.H} N={c.N} d={c.d}"] = (c, heads, prow, modes)
            del qs, ks, vs, os_, ls, host
        log("sweep timed")

    # ---- the fp32 smoke configuration (B=1 H=2 N=256 d=64), checked in full
    if with_cpu:
        c0 = w.FWD_CONFIGS["smoke"]
        h0 = w.fwd_config_inputs(c0)
        o0, l0 = fa.attention(*(torch.from_numpy(x).to(dev) for x in h0), causal=False,
                              scale=c0.scale)
        torch.cuda.synchronize()
        samples["smoke"] = ((h0[0][0], h0[1][0], h0[2][0], c0.scale),
                            (o0[0].cpu().numpy(), l0[0].cpu().numpy()))

    # ---- context: the MFMA throughput a plain bf16 GEMM reaches through the
    #      vendor BLAS (torch.matmul -> hipBLASLt) on the same GPU, same clocks
    t_gemm = None
    if not args.skip_gemm and args.only in (None, "gemm"):
        n = 8192
        ga = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
        gb = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
        gc = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
        gemm = lambda: torch.matmul(ga, gb, out=gc)  # noqa: E731
        warm_up(gemm)
        t_g = t_gemm = time_calls(gemm)
        tg = 2.0 * n ** 3 / (t_g * 1e-3) / 1e12
        out["mfma_ceiling"] = {
            "kind": "bf16 GEMM 8192x8192x8192 (torch.matmul, vendor BLAS), N(0,1) operands",
            "ms": round(t_g, 4), "tflops": round(tg, 2),
            "frac_peak": round(tg / PEAK_BF16_TFLOPS, 4),
            "fwd_noncausal_over_gemm": round(tflops_nc / tg, 4) if run_nc else None,
            "fwd_causal_over_gemm": round(tflops_c / tg, 4) if run_c else None}
        del ga, gb, gc
        log("gemm timed")
    if not args.skip_gemm and args.only is None:
        # and the HBM bandwidth of plain device copies (read + write) through
        # torch, for the decode's GB/s
        nb = 2 ** 31
        src = torch.empty(nb // 2, dtype=torch.bfloat16, device=dev).normal_()
        dst = torch.empty_like(src)
        cp = lambda: dst.copy_(src)  # noqa: E731
        warm_up(cp)
        t_cp = time_calls(cp)
        gbs_cp = 2.0 * nb / (t_cp * 1e-3) / 1e9
        out["hbm_ceiling"] = {
            "kind": "device copy of 2 GiB (torch copy_), read + write bytes",
            "ms": round(t_cp, 4), "gbs": round(gbs_cp, 1),
            "frac_peak": round(gbs_cp / PEAK_HBM_GBS, 4)}
        del src, dst
        log("copy timed")
        # and the read-only rate of the probe library (16-byte non-temporal
        # loads): a sequential sweep and 4 KiB chunks in random order, the
        # grain of the paged kernels' reads
        import ctypes
        probe = ctypes.CDLL(os.path.join(ROOT, "exact_attention_26_amd", "libfa_probe.so"))
        probe.fa_probe_read.restype = ctypes.c_int
        probe.fa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        nb = 2 ** 32
        buf = torch.ones(nb, dtype=torch.uint8, device=dev)
        order = torch.from_numpy(np.random.default_rng(12).permutation(nb // 4096)
                                 .astype(np.int32)).to(dev)
        sink = torch.zeros(256, dtype=torch.int32, device=dev)

        def rd(order_ptr):
            rc = probe.fa_probe_read(buf.data_ptr(), nb, order_ptr, sink.data_ptr(),
                                     stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"fa_probe_read returned {rc}")
        rates = {}
        for name, ptr in (("sequential", None), ("random_4k", order.data_ptr())):
            warm_up(lambda: rd(ptr))
            rates[name] = nb / (time_calls(lambda: rd(ptr)) * 1e-3) / 1e9
        out["hbm_read_ceiling"] = {
            "kind": "read-only probe over 4 GiB (libfa_probe.so, 16-byte non-temporal loads)",
            "sequential_gbs": round(rates["sequential"], 1),
            "random_4k_gbs": round(rates["random_4k"], 1),
            "frac_peak": round(rates["sequential"] / PEAK_HBM_GBS, 4),
            "decode_over_random_4k": (round(gbs / rates["random_4k"], 4) if run_dec else None),
            "tree_over_random_4k": (round(tree_gbs / rates["random_4k"], 4)
                                    if tree_gbs is not None else None)}
        del buf, order, sink
        log("read probe timed")

    if args.only == "sweep":
        print(json.dumps({"only": "sweep", "sweep": out["sweep"]}), flush=True)
        return
    if args.only is not None:
        ms = {"fwd-noncausal": t_nc, "fwd-causal": t_c, "decode": t_dec,
              "bwd-noncausal": t_bwd.get(False), "bwd-causal": t_bwd.get(True),
              "prefill": t_pre, "tree": t_tree, "rope": t_rope, "gemm": t_gemm}[args.only]
        print(json.dumps({"only": args.only, "ms": ms}), flush=True)
        return
    if with_cpu:
        log("checking the GPU results against the oracle")
        out["cpu_baseline"] = cpu_report
        out["parity"] = cpu_baseline_parity(samples, oracle_res, L)
        cpu_report["gpu_speedup"] = {
            "fwd": round(value / cpu_report["value"], 1),
            "decode": round(gbs / cpu_report["decode"]["value"], 1)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
