#!/usr/bin/env python3
"""Throughput of the fused attention forward + backward on one MI355X.

A step is one pass of the whole path over one batch: fa_fwd, then
fa_bwd_preprocess and fa_bwd (the dQ kernel and the dK/dV kernel). Inputs are drawn on the host, copied to HBM
before timing, and every output buffer is allocated once; the timed loop only
enqueues the three C-ABI calls. Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the GPT-2-medium attention shape (batch 64, 16 heads,
length 1024, head dim 64, fp16, dense). Other workload names come from
attn_inputs.WORKLOADS, and attn_inputs.PACKED_WORKLOADS (packed variable-length
batches with grouped key/value heads: forward + backward through
fa_fwd_varlen / fa_bwd_varlen, or decode through fa_fwd_splitkv).
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
DEFAULT_WORKLOAD = "gpt2_medium_b64_h16_n1024_d64_f16"
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


def cpu_baseline(w, dr, budget_s: float, pdrop: float = 0.0):
    """Time the float64 oracle on whole heads of the same workload until the
    budget is used (at least one head); scale to TFLOP/s with the same FLOP
    convention as the GPU figure."""
    import numpy as np
    import oracle
    from exact_io_aware_04_amd import metrics
    try:
        from threadpoolctl import threadpool_info
    except ImportError:
        threadpool_info = None
    mask = w.block_mask()
    pairs = metrics.kept_pairs_per_head(w.N, w.causal, mask)
    f_fwd, f_bwd = metrics.flops(1, 1, pairs, w.d)
    per_head = f_fwd + (f_bwd if w.backward else 0)
    heads, elapsed = 0, 0.0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = (dr.f64(n, b, h) for n in "qkv")
            if pdrop > 0:
                import oracle.dropout as od
                od.forward_head(q, k, v, w.scale, w.causal, pdrop, 0x5EED, 0, b * w.H + h, mask, 128)
                if w.backward:
                    od.backward_head(q, k, v, dr.f64("do", b, h), w.scale, w.causal, pdrop, 0x5EED, 0, b * w.H + h,
                                     mask, 128)
            else:
                oracle.forward_head(q, k, v, w.scale, w.causal, mask, 128)
                if w.backward:
                    oracle.backward_head(q, k, v, dr.f64("do", b, h), w.scale, w.causal, mask, 128)
            heads += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    cores = None
    if threadpool_info is not None:
        cores = max((p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"), default=None)
    if not cores:
        cores = 1
    return {
        "value": round(heads * per_head / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{heads} of {w.B * w.H} heads (b,h in row-major order from (0,0)), "
                   f"{'forward+backward' if w.backward else 'forward'}, float64 numpy oracle "
                   f"materialising S and P, {elapsed:.1f} s"),
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
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import attn_inputs as ai
    from exact_io_aware_04_amd import fa, metrics

    if args.workload in ai.PACKED_WORKLOADS:
        return bench_packed(args, ai.PACKED_WORKLOADS[args.workload])
    if args.workload not in ai.WORKLOADS:
        log(f"unknown workload {args.workload}; choose from {list(ai.WORKLOADS) + list(ai.PACKED_WORKLOADS)}")
        return 2
    w = ai.WORKLOADS[args.workload]
    B, H, N, d = w.B, w.H, w.N, w.d
    dt = fa.FA_F16 if w.dtype == ai.F16 else fa.FA_BF16
    tdt = torch.float16 if w.dtype == ai.F16 else torch.bfloat16
    dev = torch.device("cuda:0")

    log(f"[bench] drawing {w.name}")
    dr = ai.draw_workload(w)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q, k, v = up(dr.q), up(dr.k), up(dr.v)
    do = up(dr.do) if w.backward else None
    mask = w.block_mask()
    bm = torch.from_numpy(mask).to(dev) if mask is not None else None
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if w.backward:
        Dv = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    bmp = bm.data_ptr() if bm is not None else None
    causal = int(w.causal)
    scale = float(w.scale)

    pdrop, dseed = float(args.dropout), 0x5EED

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

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        assert fwd() == 0
        if w.backward:
            assert bwd_pre() == 0
            assert bwd() == 0
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    log(f"[bench] timing {K} steps")
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
    ms_step = (t1 - t0) * 1e3 / K
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    if w.backward:
        pre_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
        bwd_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    else:
        pre_ms = bwd_ms = 0.0

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

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "block_mask": w.mask, "backward": w.backward, "dropout": pdrop, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / peak, 2),
        "phases_ms": {"fwd": round(fwd_ms, 4), "bwd_preprocess": round(pre_ms, 4), "bwd": round(bwd_ms, 4)},
        "phase_tflops": {"fwd": round(fwd_tf, 2), "bwd": round(bwd_tf, 2) if bwd_tf else None},
        "bytes_model": {"algorithmic_fwd": a_fwd, "algorithmic_bwd": a_bwd,
                        "standard_fwd": s_fwd, "standard_fwd_bwd": s_all},
        "roofline": roofline,
    }
    if args.cpu_seconds > 0:
        log(f"[bench] oracle CPU baseline ({args.cpu_seconds:.0f} s budget)")
        result["cpu_baseline"] = cpu_baseline(w, dr, args.cpu_seconds, pdrop)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
