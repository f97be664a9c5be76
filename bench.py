#!/usr/bin/env python3
"""Throughput of the fused attention forward + backward on one MI355X.

A step is one pass of the whole path over one batch: fa_fwd, then
fa_bwd_preprocess and fa_bwd (the dQ kernel and the dK/dV kernel). Inputs are drawn on the host, copied to HBM
before timing, and every output buffer is allocated once; the timed loop only
enqueues the three C-ABI calls. Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the largest single-GPU one in the metric's range: causal
attention over 65536 tokens (batch 1, 8 heads, head dim 128, bf16). The other
workloads of that range (causal N=8192 d=128, butterfly block-sparse N=16384
d=64) are timed in the same run and reported under "other_workloads". Other
workload names come from attn_inputs.WORKLOADS, and attn_inputs.PACKED_WORKLOADS
(packed variable-length batches with grouped key/value heads: forward +
backward through fa_fwd_varlen / fa_bwd_varlen, or decode through
fa_fwd_splitkv). The oracle CPU baseline runs first, on a bounded sample of the
same workload, in a pool of worker processes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s and % of MFMA bf16 peak, N=1k..64k, d=64/128"
DEFAULT_WORKLOAD = "causal_b1_h8_n65536_d128_bf16"
# the other workloads in the metric's N >= 4096 range, reported beside the default one
EXTRA_WORKLOADS = ["causal_b2_h32_n8192_d128_bf16", "butterfly_b4_h16_n16384_d64_f16"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["fa_device.h", "fa_fwd.hip", "fa_bwd.hip", "fa_launch.h"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_io_aware_04_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on kernel sources that have changed since."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get(kernel)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def cpu_pool_size() -> int:
    """Worker processes for the oracle baseline: the cores this process may run
    on, at most 16 (one GPU's share of a host)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


_CPU_JOB = None      # (workload, drawn inputs, mask, budget, units, pdrop): set before the pool forks


def _cpu_worker_init() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _cpu_worker(args):
    """Run the oracle on this worker's share of the units until the budget is used."""
    import numpy as np
    import oracle
    import oracle.dropout as od
    from exact_io_aware_04_amd import metrics
    widx, nworkers = args
    w, dr, mask, budget, units, pdrop = _CPU_JOB
    t0 = time.perf_counter()
    pairs, done, cached = 0, 0, None
    for b, h, r0, r1 in units[widx::nworkers]:
        if time.perf_counter() - t0 >= budget:
            break
        if cached is None or cached[0] != (b, h):
            cached = ((b, h), tuple(dr.f64(n, b, h) for n in (("q", "k", "v", "do") if w.backward else "qkv")))
        t = cached[1]
        rows = np.arange(r0, r1)
        if pdrop > 0:                          # whole heads (the dropout oracle has no row subsets)
            od.forward_head(*t[:3], w.scale, w.causal, pdrop, 0x5EED, 0, b * w.H + h, mask, 128)
            if w.backward:
                od.backward_head(*t, w.scale, w.causal, pdrop, 0x5EED, 0, b * w.H + h, mask, 128)
        else:
            oracle.forward_head(*t[:3], w.scale, w.causal, mask, 128, rows=rows, row_block=128)
            if w.backward:
                oracle.backward_head(*t, w.scale, w.causal, mask, 128, row_block=128, rows=rows)
        pairs += metrics.kept_pairs_rows(rows, w.N, w.causal, mask)
        done += 1
    return pairs, done, time.perf_counter() - t0


def cpu_baseline(w, dr, budget_s: float, pdrop: float = 0.0, workers: int = 0):
    """The float64 oracle on a bounded sample of the same workload, timed on the
    host's cores: units of (head, block of 128 query rows) in a seeded random
    order are dealt to a pool of single-threaded worker processes, each
    computing the forward (and backward) of its rows until the budget is used.
    TFLOP/s under the same FLOP convention as the GPU figure (kept pairs of the
    rows done x 4d, + 10d with the backward), over the pool's wall time. Must
    run before this process touches the GPU: the pool forks."""
    global _CPU_JOB
    import multiprocessing as mp
    import numpy as np
    mask = w.block_mask()
    rb = w.N if pdrop > 0 else min(w.N, 128)
    units = [(b, h, r0, min(w.N, r0 + rb)) for b in range(w.B) for h in range(w.H) for r0 in range(0, w.N, rb)]
    order = np.random.Generator(np.random.PCG64(w.seed)).permutation(len(units))
    units = [units[i] for i in order]
    nw = workers or cpu_pool_size()
    _CPU_JOB = (w, dr, mask, budget_s, units, pdrop)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(nw, initializer=_cpu_worker_init) as pool:
        out = pool.map(_cpu_worker, [(i, nw) for i in range(nw)])
    wall = time.perf_counter() - t0
    _CPU_JOB = None
    pairs = sum(o[0] for o in out)
    done = sum(o[1] for o in out)
    per_pair = 4 * w.d + (10 * w.d if w.backward else 0)
    unit = "whole heads" if pdrop > 0 else "(head, 128-query-row block) units"
    return {
        "value": round(pairs * per_pair / wall / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(nw),
        "kind": "oracle",
        "sample": (f"{done} of {len(units)} {unit} of {w.name} in seeded random order, "
                   f"{'forward+backward' if w.backward else 'forward'}, float64 numpy oracle materialising "
                   f"S and P rows, {nw} worker processes with one BLAS thread each, {wall:.1f} s wall"),
    }


def cpu_baseline_packed(w, pk, budget_s: float):
    """The float64 oracle on whole sequences of the packed workload (all heads),
    in order, until the budget is used; TFLOP/s under the same convention."""
    import numpy as np
    import oracle.varlen as ov
    from exact_io_aware_04_amd import metrics
    try:
        from threadpoolctl import threadpool_info
    except ImportError:
        threadpool_info = None
    lq, lk = w.lengths()
    q, k, v, do = (pk.f64(n) for n in ("q", "k", "v", "do")) if w.backward else (
        pk.f64("q"), pk.f64("k"), pk.f64("v"), None)
    done_pairs, t0, n_seq, elapsed = 0, time.perf_counter(), 0, 0.0
    for b in range(w.batch):
        sq, eq, sk, ek = (int(pk.cu_q[b]), int(pk.cu_q[b + 1]), int(pk.cu_k[b]), int(pk.cu_k[b + 1]))
        cq, ck = np.array([0, eq - sq]), np.array([0, ek - sk])
        ov.forward(q[sq:eq], k[sk:ek], v[sk:ek], cq, ck, 1.0 / math.sqrt(w.d), w.causal)
        if w.backward:
            ov.backward(q[sq:eq], k[sk:ek], v[sk:ek], do[sq:eq], cq, ck, 1.0 / math.sqrt(w.d), w.causal)
        done_pairs += metrics.kept_pairs_varlen([eq - sq], [ek - sk], w.causal) * w.hq
        n_seq += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s:
            break
    per_pair = 4 * w.d + (10 * w.d if w.backward else 0)
    cores = None
    if threadpool_info is not None:
        cores = max((p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"), default=None)
    return {"value": round(done_pairs * per_pair / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores or 1),
            "kind": "oracle",
            "sample": (f"{n_seq} of {w.batch} sequences (all {w.hq} query heads), "
                       f"{'forward+backward' if w.backward else 'forward'}, float64 oracle, {elapsed:.1f} s")}


def bench_packed(args, w) -> int:
    """Packed workloads: varlen forward + backward, or split-KV decode forward."""
    import numpy as np
    import torch
    import attn_inputs as ai
    from exact_io_aware_04_amd import fa, metrics
    lq, lk = w.lengths()
    log(f"[bench] drawing {w.name} ({int(lq.sum())} query / {int(lk.sum())} key rows)")
    pk = ai.draw_packed(lq, lk, w.hq, w.hk, w.d, w.dtype, w.seed)
    dev = torch.device("cuda:0")
    tdt = torch.float16 if w.dtype == ai.F16 else torch.bfloat16
    dt = fa.FA_F16 if w.dtype == ai.F16 else fa.FA_BF16

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q, k, v = up(pk.q), up(pk.k), up(pk.v)
    do = up(pk.do) if w.backward else None
    cu_q = torch.from_numpy(pk.cu_q).to(dev)
    cu_k = torch.from_numpy(pk.cu_k).to(dev)
    tq, tk = int(lq.sum()), int(lk.sum())
    mq, mk = int(lq.max()), int(lk.max())
    o = torch.empty_like(q)
    lse = torch.empty((tq, w.hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    scale = 1.0 / math.sqrt(w.d)
    causal = int(w.causal)
    args_common = (cu_q.data_ptr(), cu_k.data_ptr(), w.batch, tq, tk, mq, mk, w.hq, w.hk, w.d, dt, scale, causal)
    if w.decode:
        opart, lpart = fa.splitkv_workspace(tq, w.hq, w.d, w.n_splits, dev)

        def fwd():
            return fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     *args_common, w.n_splits, opart.data_ptr(), lpart.data_ptr(), s)
    else:
        def fwd():
            return fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    *args_common, s)
    if w.backward:
        Dv = torch.empty((tq, w.hq), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def bwd_pre():
            return fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), Dv.data_ptr(), 1, w.hq, tq, w.d, dt, s)

        def bwd():
            return fa.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                    Dv.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *args_common, s)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        assert fwd() == 0
        if w.backward:
            assert bwd_pre() == 0 and bwd() == 0
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    log(f"[bench] timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        if w.backward:
            bwd_pre()
            e[2].record(stream)
            bwd()
        e[3].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    pre_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K if w.backward else 0.0
    bwd_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K if w.backward else 0.0

    pairs = metrics.kept_pairs_varlen(lq, lk, w.causal) * w.hq
    f_fwd, f_bwd = 4 * w.d * pairs, 10 * w.d * pairs
    total = f_fwd + (f_bwd if w.backward else 0)
    value = total / (ms_step * 1e-3) / 1e12
    b_fwd, b_bwd = metrics.packed_bytes(tq, tk, w.hq, w.hk, w.d)
    if w.decode:
        achieved = b_fwd / (fwd_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "fa_fwd_splitkv", "achieved": round(achieved, 1),
                    "peak": metrics.MI355X_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / metrics.MI355X_HBM_GBPS, 4),
                    "traffic": measured_traffic(w.name, "fa_fwd_splitkv"), "launch_ms": round(fwd_ms, 4),
                    "bytes_per_launch": b_fwd}
        metric = "decode forward (split-KV) HBM GB/s and TFLOP/s, packed GQA batch"
    else:
        achieved = f_bwd / (bwd_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "fa_bwd_varlen", "achieved": round(achieved, 2),
                    "peak": metrics.MI355X_PEAK_DENSE_F16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / metrics.MI355X_PEAK_DENSE_F16_TFLOPS, 4),
                    "traffic": measured_traffic(w.name, "fa_bwd_varlen"),
                    "launch_ms": round(bwd_ms, 4), "flops_per_launch": f_bwd}
        metric = "packed varlen GQA attention fwd+bwd TFLOP/s"
    result = {
        "metric": metric, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "Hq": w.hq, "Hk": w.hk, "d": w.d, "causal": w.causal,
                   "total_q": tq, "total_k": tk, "max_q": mq, "max_k": mk, "n_splits": w.n_splits if w.decode else None,
                   "backward": w.backward, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / metrics.MI355X_PEAK_DENSE_F16_TFLOPS, 2),
        "phases_ms": {"fwd": round(fwd_ms, 4), "bwd_preprocess": round(pre_ms, 4), "bwd": round(bwd_ms, 4)},
        "bytes_model": {"algorithmic_fwd": b_fwd, "algorithmic_bwd": b_bwd},
        "roofline": roofline,
    }
    if args.cpu_seconds > 0:
        log(f"[bench] oracle CPU baseline ({args.cpu_seconds:.0f} s budget)")
        result["cpu_baseline"] = cpu_baseline_packed(w, pk, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def run_dense(w, dr, steps: int, warmup: int, pdrop: float = 0.0):
    """Time `steps` forward + backward steps of a dense workload on cuda:0.
    Returns the per-workload figures (throughput, phases, roofline, memory)."""
    import numpy as np
    import torch
    import attn_inputs as ai
    from exact_io_aware_04_amd import fa, metrics

    B, H, N, d = w.B, w.H, w.N, w.d
    dt = fa.FA_F16 if w.dtype == ai.F16 else fa.FA_BF16
    tdt = torch.float16 if w.dtype == ai.F16 else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q, k, v = up(dr.q), up(dr.k), up(dr.v)
    do = up(dr.do) if w.backward else None
    mask = w.block_mask()
    bm = torch.from_numpy(mask).to(dev) if mask is not None else None
    o = torch.empty_like(q)
    io = [q, k, v, o] + ([do] if w.backward else []) + ([bm] if bm is not None else [])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if w.backward:
        Dv = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        io += [dq, dk, dv]
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    bmp = bm.data_ptr() if bm is not None else None
    causal = int(w.causal)
    scale = float(w.scale)
    dseed = 0x5EED

    def fwd():
        if pdrop > 0:
            return fa.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
                                     d, dt, scale, causal, bmp, 128, pdrop, dseed, 0, s)
        return fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, dt,
                         scale, causal, bmp, 128, s)

    def bwd_pre():
        return fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), Dv.data_ptr(), B, H, N, d, dt, s)

    def bwd():
        if pdrop > 0:
            return fa.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                     Dv.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, dt, scale,
                                     causal, bmp, 128, pdrop, dseed, 0, s)
        return fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), Dv.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, dt, scale,
                         causal, bmp, 128, s)

    log(f"[bench] {w.name}: warmup {warmup}")
    for _ in range(warmup):
        assert fwd() == 0
        if w.backward:
            assert bwd_pre() == 0
            assert bwd() == 0
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info(dev)[0]

    K = steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    log(f"[bench] {w.name}: timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        if w.backward:
            bwd_pre()
            e[2].record(stream)
            bwd()
        e[3].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    free_after = torch.cuda.mem_get_info(dev)[0]
    ms_step = (t1 - t0) * 1e3 / K
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    if w.backward:
        pre_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
        bwd_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    else:
        pre_ms = bwd_ms = 0.0
    # per-step GPU time on the launch stream (first to last event of each step)
    per_step = sorted(e[0].elapsed_time(e[3]) for e in ev)
    step_ms = {"median": round(float(np.median(per_step)), 4), "min": round(per_step[0], 4),
               "max": round(per_step[-1], 4)}

    pairs = metrics.kept_pairs_per_head(N, w.causal, mask)
    f_fwd, f_bwd = metrics.flops(B, H, pairs, d)
    total = f_fwd + (f_bwd if w.backward else 0)
    value = total / (ms_step * 1e-3) / 1e12
    peak = metrics.MI355X_PEAK_DENSE_F16_TFLOPS
    fwd_tf = f_fwd / (fwd_ms * 1e-3) / 1e12
    bwd_tf = f_bwd / ((pre_ms + bwd_ms) * 1e-3) / 1e12 if w.backward else None
    if w.backward:
        kern, kflops, kms = "fa_bwd", f_bwd, bwd_ms
    else:
        kern, kflops, kms = "fa_fwd", f_fwd, fwd_ms
    achieved = kflops / (kms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": kern,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(w.name, kern) if pdrop == 0 else None,
        "launch_ms": round(kms, 4),
        "flops_per_launch": kflops,
    }
    a_fwd, a_bwd = metrics.algorithmic_bytes(B, H, N, d)
    s_fwd, s_all = metrics.standard_attention_bytes(B, H, N)
    io_bytes = sum(t.numel() * t.element_size() for t in io)
    peak_alloc = torch.cuda.max_memory_allocated(dev) - base_alloc
    memory = {
        # device memory beyond the inputs and outputs, at the allocator's peak: LSE and D
        "extra_bytes": int(peak_alloc - io_bytes),
        "lse_and_D_bytes": int(4 * B * H * N * (2 if w.backward else 1)),
        "inputs_outputs_bytes": int(io_bytes),
        # free device memory before minus after the timed steps: the library itself
        # allocates nothing (the warmup calls load the kernels' code first)
        "alloc_during_timed_steps_bytes": int(free_before - free_after),
        # S and P of every head in 16-bit, as standard attention would hold them
        "standard_S_P_bytes": int(B * H * metrics.score_and_prob_bytes_per_head(N)),
    }
    out = {
        "value": round(value, 2),
        "ms_per_step": round(ms_step, 4),
        "step_ms": step_ms,
        "pct_of_peak": round(100 * value / peak, 2),
        "phases_ms": {"fwd": round(fwd_ms, 4), "bwd_preprocess": round(pre_ms, 4), "bwd": round(bwd_ms, 4)},
        "phase_tflops": {"fwd": round(fwd_tf, 2), "bwd": round(bwd_tf, 2) if bwd_tf else None},
        "bytes_model": {"algorithmic_fwd": a_fwd, "algorithmic_bwd": a_bwd,
                        "standard_fwd": s_fwd, "standard_fwd_bwd": s_all},
        "memory": memory,
        "roofline": roofline,
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "block_mask": w.mask, "backward": w.backward, "dropout": pdrop, "parallelism": "single GPU"},
    }
    del q, k, v, o, lse, io
    if w.backward:
        del do, Dv, dq, dk, dv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768, 65536)


def sweep(steps: int, warmup: int) -> dict:
    """The metric's sweep: N = 1k..64k x d in {64, 128} x {non-causal, causal} x
    bf16 (and fp16 at d = 64), H = 2048 / d heads, B = max(1, 16384 / N), so
    every row holds 16384 tokens per head group. Inputs are N(0, 1) values drawn
    on the device from a seeded generator (2000 + row index) and rounded to the
    dtype; only timing is taken here (the parity tests cover the numbers).
    TFLOP/s under the same convention as the headline (4d + 10d per kept pair)."""
    import torch
    from exact_io_aware_04_amd import fa, metrics
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    rows, idx = [], 0
    for d in (64, 128):
        for dname in (("bf16", "f16") if d == 64 else ("bf16",)):
            tdt = torch.float16 if dname == "f16" else torch.bfloat16
            dt = fa.FA_F16 if dname == "f16" else fa.FA_BF16
            for causal in (False, True):
                for N in SWEEP_N:
                    H, B = 2048 // d, max(1, 16384 // N)
                    g = torch.Generator(device=dev).manual_seed(2000 + idx)
                    idx += 1
                    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device=dev).to(tdt) for _ in range(4))
                    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
                    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
                    Dv = torch.empty_like(lse)
                    scale = 1.0 / math.sqrt(d)
                    P = (q.data_ptr(), k.data_ptr(), v.data_ptr())

                    def fwd():
                        return fa.fa_fwd(*P, o.data_ptr(), lse.data_ptr(), B, H, N, d, dt, scale, int(causal), None, 128, st)

                    def pre():
                        return fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), Dv.data_ptr(), B, H, N, d, dt, st)

                    def bwd():
                        return fa.fa_bwd(*P, do.data_ptr(), lse.data_ptr(), Dv.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                         dv.data_ptr(), B, H, N, d, dt, scale, int(causal), None, 128, st)

                    for _ in range(warmup):
                        assert fwd() == 0 and pre() == 0 and bwd() == 0
                    torch.cuda.synchronize()
                    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
                    for e in ev:
                        e[0].record(stream)
                        fwd()
                        e[1].record(stream)
                        pre()
                        e[2].record(stream)
                        bwd()
                        e[3].record(stream)
                    torch.cuda.synchronize()
                    f_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
                    b_ms = sum(e[1].elapsed_time(e[3]) for e in ev) / steps
                    pairs = metrics.kept_pairs_per_head(N, causal, None) * B * H
                    ff, fb = 4 * d * pairs, 10 * d * pairs
                    tot = (ff + fb) / ((f_ms + b_ms) * 1e-3) / 1e12
                    rows.append({"N": N, "d": d, "dtype": dname, "causal": causal, "B": B, "H": H,
                                 "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                                 "fwd_tflops": round(ff / (f_ms * 1e-3) / 1e12, 1),
                                 "bwd_tflops": round(fb / (b_ms * 1e-3) / 1e12, 1),
                                 "tflops": round(tot, 1),
                                 "pct_of_peak": round(100 * tot / metrics.MI355X_PEAK_DENSE_F16_TFLOPS, 2)})
                    log(f"[sweep] N={N} d={d} {dname} causal={causal}: {tot:.1f} TFLOP/s "
                        f"({rows[-1]['pct_of_peak']}%)")
                    del q, k, v, do, o, dq, dk, dv, lse, Dv
                    torch.cuda.empty_cache()
    target = [r for r in rows if r["N"] >= 4096]
    return {"metric": METRIC, "mode": "sweep", "data": "synthetic", "steps": steps, "warmup": warmup,
            "rows": rows,
            "n_ge_4096": {"rows": len(target),
                          "min_pct_of_peak": min(r["pct_of_peak"] for r in target),
                          "max_pct_of_peak": max(r["pct_of_peak"] for r in target)}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability on P for dense workloads (fa_fwd_dropout / fa_bwd_dropout); 0 = off")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle CPU baseline (0 disables it)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other N >= 4096 workloads reported beside the default one")
    ap.add_argument("--sweep", action="store_true",
                    help="time the metric's sweep (N = 1k..64k, d = 64/128, causal and not) and print it "
                         "as one JSON object instead of the headline line")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        return 2

    import attn_inputs as ai

    if args.sweep:
        print(json.dumps(sweep(args.steps, args.warmup)), flush=True)
        return 0
    if args.workload in ai.PACKED_WORKLOADS:
        return bench_packed(args, ai.PACKED_WORKLOADS[args.workload])
    if args.workload not in ai.WORKLOADS:
        log(f"unknown workload {args.workload}; choose from {list(ai.WORKLOADS) + list(ai.PACKED_WORKLOADS)}")
        return 2
    w = ai.WORKLOADS[args.workload]
    pdrop = float(args.dropout)

    log(f"[bench] drawing {w.name}")
    dr = ai.draw_workload(w)
    cpu = None
    if args.cpu_seconds > 0:
        # before any GPU use: the baseline's worker pool forks this process
        log(f"[bench] oracle CPU baseline ({args.cpu_seconds:.0f} s budget, {cpu_pool_size()} workers)")
        cpu = cpu_baseline(w, dr, args.cpu_seconds, pdrop)

    head = run_dense(w, dr, args.steps, args.warmup, pdrop)
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": head["config"],
    }
    result.update({k: head[k] for k in ("step_ms", "pct_of_peak", "phases_ms", "phase_tflops", "bytes_model",
                                        "memory", "roofline")})
    result["cpu_baseline"] = cpu
    if args.workload == DEFAULT_WORKLOAD and pdrop == 0 and not args.no_extra:
        others = {}
        for name in EXTRA_WORKLOADS:
            wx = ai.WORKLOADS[name]
            log(f"[bench] drawing {name}")
            rx = run_dense(wx, ai.draw_workload(wx), args.steps, args.warmup)
            others[name] = {k: rx[k] for k in ("value", "ms_per_step", "pct_of_peak", "phases_ms", "phase_tflops",
                                               "roofline")}
        result["other_workloads"] = others
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
