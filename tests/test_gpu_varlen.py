"""Packed variable-length batches with grouped key/value heads: HIP path
(fa_fwd_varlen / fa_bwd_varlen through the binding) vs oracle/varlen.py.

Length mixes span several tiles, ragged tails, more queries than keys (causal
rows that see nothing), fewer queries than keys (decode-like rows), and empty
sequences. Tolerances are those of the dense tests (tests/harness.py),
applied per (sequence, head): gradients of each sequence's query heads and of
each key/value head it owns are checked on their own, element by element.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle.dropout as od
import oracle.varlen as ov
from error_model import Scales, gradient_scales_head
from harness import GRAD_REL_TOL, O_TOL, LSE_TOL, check_grads, from_dev, rel_fro, report, say, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    # name: (lengths_q, lengths_k, Hq, Hk)
    "mixed_gqa": ([1, 17, 128, 129, 300], [1, 40, 128, 200, 300], 4, 2),
    "more_q_than_k": ([200, 64], [50, 64], 2, 1),
    "decode_like": ([1, 3, 16], [700, 257, 1024], 8, 2),
    "empty_seqs": ([0, 90, 130, 5], [70, 0, 130, 300], 2, 2),
    "mqa_long": ([513], [513], 8, 1),
}


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


def run_varlen(pk: ai.PackedDrawn, hq, hk, scale, causal, p_drop=0.0, seed=0, offset=0):
    import torch
    from exact_io_aware_04_amd import fa
    q, k, v, do = (to_dev(getattr(pk, n), pk.dtype) for n in ("q", "k", "v", "do"))
    cu_q, cu_k = _dev_i32(pk.cu_q), _dev_i32(pk.cu_k)
    mq = int(max(1, np.diff(pk.cu_q).max()))
    mk = int(max(1, np.diff(pk.cu_k).max()))
    # outputs start as NaN: an element a kernel fails to write fails the comparison
    nan = lambda t: torch.full_like(t, float("nan"))
    lse0 = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device)
    drop = dict(p_drop=p_drop, seed=seed, offset=offset)
    o, lse = fa.forward_varlen(q, k, v, cu_q, cu_k, mq, mk, scale, causal, out=nan(q), lse=lse0, **drop)
    dq, dk, dv, D = fa.backward_varlen(q, k, v, o, lse, do, cu_q, cu_k, mq, mk, scale, causal,
                                       out=(nan(q), nan(k), nan(v)), **drop)
    torch.cuda.synchronize()
    return {"o": from_dev(o, pk.dtype), "lse": lse.double().cpu().numpy(), "dq": from_dev(dq, pk.dtype),
            "dk": from_dev(dk, pk.dtype), "dv": from_dev(dv, pk.dtype), "D": D.double().cpu().numpy(),
            "dev": (o, lse, dq, dk, dv)}


def check_sequence_group(res, grads, q, k, v, do, cu_q, cu_k, b, g, grp, scale, causal, dtype, what, zf=None):
    """Gradients of sequence b, key/value head g and its query heads against the
    oracle's, element by element (grads = oracle dQ, dK, dV of the packed batch).
    zf(h, rows, cols), under dropout, gives query head h's multiplier M / (1 - p)
    at positions inside the sequence."""
    sq, eq, sk, ek = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
    heads = list(range(g * grp, (g + 1) * grp))
    parts = []
    for h in heads:
        if eq > sq and ek > sk:
            z = None if zf is None else (lambda rows, cols, h=h: zf(h, rows, cols))
            parts.append(gradient_scales_head(q[sq:eq, h], k[sk:ek, g], v[sk:ek, g], do[sq:eq, h], scale, causal,
                                              diag_offset=(ek - sk) - (eq - sq), z=z))
    zq, zk = np.zeros((eq - sq, len(heads), q.shape[2])), np.zeros((ek - sk, q.shape[2]))
    sc = {
        "dq": Scales(*(np.stack([getattr(pp["dq"], f) for pp in parts], axis=1) if parts else zq
                       for f in ("r", "g", "f"))),
        "dk": Scales.combine([pp["dk"] for pp in parts]) if parts else Scales(zk, zk, zk),
        "dv": Scales.combine([pp["dv"] for pp in parts]) if parts else Scales(zk, zk, zk),
    }
    got = {"dq": res["dq"][sq:eq][:, heads], "dk": res["dk"][sk:ek, g], "dv": res["dv"][sk:ek, g]}
    ref = {"dq": grads[0][sq:eq][:, heads], "dk": grads[1][sk:ek, g], "dv": grads[2][sk:ek, g]}
    return check_grads(got, ref, f"{what} seq {b} kv-head {g}", sc, dtype)


def _check(res, ref, dtype, what):
    o, lse = res["o"], res["lse"]
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    err = float(np.abs(o - ref[0]).max())
    assert err <= O_TOL[dtype], f"{what}: O error {err:.3e}"
    live = np.isfinite(ref[1])
    assert (np.isneginf(lse) == ~live).all(), f"{what}: LSE -inf pattern"
    if live.any():
        lerr = float(np.abs(lse[live] - ref[1][live]).max())
        assert lerr <= LSE_TOL[dtype], f"{what}: LSE error {lerr:.3e}"
    q, k, v, do, cu_q, cu_k, scale, causal = ref[2]
    g = ov.backward(*ref[2])
    for n in ("dq", "dk", "dv"):
        assert np.isfinite(res[n]).all(), f"{what}: non-finite {n}"
    hq, hk = q.shape[1], k.shape[1]
    for b in range(len(cu_q) - 1):
        for kvh in range(hk):
            check_sequence_group(res, g, q, k, v, do, cu_q, cu_k, b, kvh, hq // hk, scale, causal, dtype, what)
    dref = (res["_do"] * o).sum(axis=2)
    derr = float((np.abs(res["D"] - dref) / (1 + np.abs(dref))).max())
    assert derr <= 1e-3, f"{what}: D error {derr:.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", list(CASES))
def test_varlen_parity(case, d, dtype, causal):
    lq, lk, hq, hk = CASES[case]
    seed = 30_000 + 13 * list(CASES).index(case) + d + (1 if dtype == ai.BF16 else 0) + (2 if causal else 0)
    say(f"[varlen] {case} d={d} {dtype} causal={causal} seed={seed}")
    pk = ai.draw_packed(lq, lk, hq, hk, d, dtype, seed)
    scale = 1.0 / np.sqrt(d)
    res = run_varlen(pk, hq, hk, scale, causal)
    q, k, v, do = (pk.f64(n) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = ov.forward(q, k, v, pk.cu_q, pk.cu_k, scale, causal)
    res["_do"] = do
    _check(res, (o_ref, lse_ref, (q, k, v, do, pk.cu_q, pk.cu_k, scale, causal)), dtype,
           f"{case} d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_equal_lengths_match_dense_bitwise(d, causal):
    """Equal lengths and Hk == Hq: the packed path must give the dense path's bits
    (same kernels, same arithmetic order, other strides)."""
    import torch
    from exact_io_aware_04_amd import fa
    B, H, N = 3, 2, 200
    say(f"[varlen-vs-dense] d={d} causal={causal}")
    dr = ai.draw(B, H, N, d, ai.BF16, 777 + d + causal)
    q, k, v, do = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, None, causal)
    dq, dk, dv, D = fa.backward(q, k, v, o, lse, do, None, causal)
    pk = lambda x: x.transpose(1, 2).contiguous().view(B * N, H, d)
    cu = _dev_i32(np.arange(B + 1) * N)
    o2, lse2 = fa.forward_varlen(pk(q), pk(k), pk(v), cu, cu, N, N, None, causal)
    dq2, dk2, dv2, D2 = fa.backward_varlen(pk(q), pk(k), pk(v), o2, lse2, pk(do), cu, cu, N, N, None, causal)
    torch.cuda.synchronize()
    assert torch.equal(o2, pk(o))
    assert torch.equal(lse2, lse.transpose(1, 2).contiguous().view(B * N, H))
    for a, b_ in ((dq2, dq), (dk2, dk), (dv2, dv)):
        assert torch.equal(a, pk(b_))


def test_varlen_backward_deterministic():
    import torch
    lq, lk, hq, hk = CASES["mixed_gqa"]
    pk = ai.draw_packed(lq, lk, hq, hk, 128, ai.BF16, 4242)
    say("[varlen-determinism] mixed_gqa d=128 bf16 causal")
    a = run_varlen(pk, hq, hk, 1 / np.sqrt(128), True)["dev"]
    b = run_varlen(pk, hq, hk, 1 / np.sqrt(128), True)["dev"]
    for x, y in zip(a, b):
        assert torch.equal(x, y)


SPLIT_CASES = {
    # name: (lengths_q, lengths_k, Hq, Hk)
    "decode_gqa": ([1, 1, 1, 1], [700, 1500, 33, 4096], 8, 2),
    "decode_q4_mha": ([4, 4, 2], [2048, 900, 64], 4, 4),
    "prefill_mqa": ([300, 129], [300, 500], 4, 1),
}


@pytest.mark.parametrize("n_splits", [1, 3, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", [(64, ai.F16), (128, ai.BF16)])
@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_splitkv_parity(case, d, dtype, causal, n_splits):
    import torch
    from exact_io_aware_04_amd import fa
    lq, lk, hq, hk = SPLIT_CASES[case]
    seed = 40_000 + 31 * list(SPLIT_CASES).index(case) + d + (2 if causal else 0) + n_splits
    say(f"[splitkv] {case} d={d} {dtype} causal={causal} splits={n_splits} seed={seed}")
    pk = ai.draw_packed(lq, lk, hq, hk, d, dtype, seed)
    scale = 1.0 / np.sqrt(d)
    q, k, v = (to_dev(getattr(pk, n), pk.dtype) for n in ("q", "k", "v"))
    cu_q, cu_k = _dev_i32(pk.cu_q), _dev_i32(pk.cu_k)
    mq, mk = int(max(lq)), int(max(lk))
    ws = fa.splitkv_workspace(q.shape[0], hq, d, n_splits, q.device)
    ws[0].fill_(float("nan"))                 # every partial a split owns must be written
    ws[1].fill_(float("nan"))
    o, lse = fa.forward_splitkv(q, k, v, cu_q, cu_k, mq, mk, n_splits, scale, causal, workspace=ws)
    o_v, lse_v = fa.forward_varlen(q, k, v, cu_q, cu_k, mq, mk, scale, causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = ov.forward(pk.f64("q"), pk.f64("k"), pk.f64("v"), pk.cu_q, pk.cu_k, scale, causal)
    what = f"{case} d={d} {dtype} causal={causal} splits={n_splits}"
    for oo, ll, tag in ((o, lse, "splitkv"), (o_v, lse_v, "varlen")):
        og, lg = from_dev(oo, dtype), ll.double().cpu().numpy()
        assert np.isfinite(og).all(), f"{what} {tag}: non-finite O"
        err = float(np.abs(og - o_ref).max())
        assert err <= O_TOL[dtype], f"{what} {tag}: O error {err:.3e}"
        live = np.isfinite(lse_ref)
        assert (np.isneginf(lg) == ~live).all(), f"{what} {tag}: LSE pattern"
        lerr = float(np.abs(lg[live] - lse_ref[live]).max()) if live.any() else 0.0
        assert lerr <= LSE_TOL[dtype], f"{what} {tag}: LSE error {lerr:.3e}"
    assert not torch.isnan(ws[1]).any(), f"{what}: unwritten partial LSE"


def test_packed_bench_workload_sampled():
    """The varlen GQA workload bench.py times, at full size: whole (sequence,
    key/value group) blocks checked against the oracle (the two shortest
    sequences and the longest one, one group each)."""
    w = ai.PACKED_WORKLOADS["varlen_gqa_b16_hq32_hk8_max4096_d128_bf16"]
    lq, lk = w.lengths()
    say(f"[packed-full] {w.name} total_q={int(lq.sum())}")
    pk = ai.draw_packed(lq, lk, w.hq, w.hk, w.d, w.dtype, w.seed)
    scale = 1.0 / np.sqrt(w.d)
    res = run_varlen(pk, w.hq, w.hk, scale, w.causal)
    grp = w.hq // w.hk
    order = np.argsort(lq)
    qf, kf, vf, dof = pk.f64("q"), pk.f64("k"), pk.f64("v"), pk.f64("do")
    for b, g in ((int(order[0]), 3), (int(order[1]), 0), (int(order[-1]), 7)):
        sq, eq, sk, ek = (int(pk.cu_q[b]), int(pk.cu_q[b + 1]), int(pk.cu_k[b]), int(pk.cu_k[b + 1]))
        say(f"[packed-full] seq {b} len {eq - sq} group {g}")
        heads = list(range(g * grp, (g + 1) * grp))
        q, do = qf[sq:eq][:, heads], dof[sq:eq][:, heads]
        k, v = kf[sk:ek][:, [g]], vf[sk:ek][:, [g]]
        cu_q, cu_k = np.array([0, eq - sq]), np.array([0, ek - sk])
        o_ref, lse_ref = ov.forward(q, k, v, cu_q, cu_k, scale, w.causal)
        dq, dk, dv, _ = ov.backward(q, k, v, do, cu_q, cu_k, scale, w.causal)
        what = f"seq {b} (len {eq - sq}) group {g}"
        err = float(np.abs(res["o"][sq:eq][:, heads] - o_ref).max())
        assert err <= O_TOL[w.dtype], f"{what}: O error {err:.3e}"
        assert float(np.abs(res["lse"][sq:eq][:, heads] - lse_ref).max()) <= LSE_TOL[w.dtype], what
        parts = [gradient_scales_head(q[:, i], k[:, 0], v[:, 0], do[:, i], scale, w.causal) for i in range(grp)]
        sc = {"dq": Scales(*(np.stack([getattr(pp["dq"], f) for pp in parts], axis=1) for f in ("r", "g", "f"))),
              "dk": Scales.combine([pp["dk"] for pp in parts]), "dv": Scales.combine([pp["dv"] for pp in parts])}
        report(what, check_grads({"dq": res["dq"][sq:eq][:, heads], "dk": res["dk"][sk:ek, g],
                                  "dv": res["dv"][sk:ek, g]},
                                 {"dq": dq, "dk": dk[:, 0], "dv": dv[:, 0]}, what, sc, w.dtype))


def test_decode_bench_workload_sampled():
    """The split-KV decode workload bench.py times, at full size, in its launch
    configuration (8 splits): sampled sequences, all query heads."""
    import torch
    from exact_io_aware_04_amd import fa
    w = ai.PACKED_WORKLOADS["decode_splitkv_b32_hq32_hk8_k16384_d128_bf16"]
    lq, lk = w.lengths()
    say(f"[decode-full] {w.name} total_k={int(lk.sum())}")
    pk = ai.draw_packed(lq, lk, w.hq, w.hk, w.d, w.dtype, w.seed)
    scale = 1.0 / np.sqrt(w.d)
    q, k, v = (to_dev(getattr(pk, n), pk.dtype) for n in ("q", "k", "v"))
    cu_q, cu_k = _dev_i32(pk.cu_q), _dev_i32(pk.cu_k)
    o, lse = fa.forward_splitkv(q, k, v, cu_q, cu_k, int(lq.max()), int(lk.max()), w.n_splits, scale, w.causal)
    torch.cuda.synchronize()
    og, lg = from_dev(o, w.dtype), lse.double().cpu().numpy()
    qf, kf, vf = pk.f64("q"), pk.f64("k"), pk.f64("v")
    for b in (0, 5, 31):
        sq, eq, sk, ek = (int(pk.cu_q[b]), int(pk.cu_q[b + 1]), int(pk.cu_k[b]), int(pk.cu_k[b + 1]))
        o_ref, lse_ref = ov.forward(qf[sq:eq], kf[sk:ek], vf[sk:ek], np.array([0, eq - sq]), np.array([0, ek - sk]),
                                    scale, w.causal)
        err = float(np.abs(og[sq:eq] - o_ref).max())
        assert err <= O_TOL[w.dtype], f"seq {b}: O error {err:.3e}"
        assert float(np.abs(lg[sq:eq] - lse_ref).max()) <= LSE_TOL[w.dtype], f"seq {b}: LSE"


@pytest.mark.parametrize("d,dtype,causal", [(64, ai.F16, True), (128, ai.BF16, False)])
def test_packed_outputs_stay_inside_their_buffers(d, dtype, causal):
    """Canaries around every packed output buffer (raw C entry points, sliced
    pointers); lengths leave ragged row tiles at every sequence end."""
    import torch
    from exact_io_aware_04_amd import fa
    lq, lk, hq, hk = [5, 40, 130], [9, 40, 100], 4, 2
    say(f"[canary-packed] d={d} {dtype} causal={causal}")
    pk = ai.draw_packed(lq, lk, hq, hk, d, dtype, 4242 + d)
    q, k, v, do = (to_dev(getattr(pk, n), pk.dtype) for n in ("q", "k", "v", "do"))
    cu_q, cu_k = _dev_i32(pk.cu_q), _dev_i32(pk.cu_k)
    tq, tk = q.shape[0], k.shape[0]
    PAD = 64
    def guarded(like_numel, dt):
        buf = torch.full((like_numel + 2 * PAD,), 7.0, dtype=dt, device="cuda")
        return buf, buf[PAD:PAD + like_numel]
    ob, o = guarded(q.numel(), q.dtype)
    lb, lse = guarded(tq * hq, torch.float32)
    Db, D = guarded(tq * hq, torch.float32)
    qb_, dq = guarded(q.numel(), q.dtype)
    kb_, dk = guarded(k.numel(), k.dtype)
    vb_, dv = guarded(v.numel(), v.dtype)
    s = torch.cuda.current_stream().cuda_stream
    code = fa.FA_BF16 if dtype == ai.BF16 else fa.FA_F16
    sc = 1.0 / np.sqrt(d)
    mq, mk = max(lq), max(lk)
    assert fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            cu_q.data_ptr(), cu_k.data_ptr(), len(lq), tq, tk, mq, mk, hq, hk, d, code, sc,
                            int(causal), s) == 0
    assert fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), D.data_ptr(), 1, hq, tq, d, code, s) == 0
    assert fa.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), D.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(),
                            len(lq), tq, tk, mq, mk, hq, hk, d, code, sc, int(causal), s) == 0
    torch.cuda.synchronize()
    for buf in (ob, lb, Db, qb_, kb_, vb_):
        assert (buf[:PAD] == 7.0).all() and (buf[-PAD:] == 7.0).all()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()


# ---- dropout on packed batches (fa_fwd_varlen_dropout / fa_bwd_varlen_dropout)

DROP_SEED = 0x0DDB_A11_5EED


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,dtype", [(64, ai.F16), (128, ai.BF16)])
@pytest.mark.parametrize("case", ["mixed_gqa", "more_q_than_k", "empty_seqs"])
def test_varlen_dropout_parity(case, d, dtype, causal):
    """Packed dropout against oracle/varlen.py with dropout: O and LSE per
    element, gradients per (sequence, key/value head) under the rounding bound
    with the keep mask of query head b Hq + h folded into the terms."""
    lq, lk, hq, hk = CASES[case]
    p, offset = 0.2, 5
    seed = 40_000 + 13 * list(CASES).index(case) + d + (2 if causal else 0)
    say(f"[varlen dropout] {case} d={d} {dtype} causal={causal} p={p} seed={seed}")
    pk = ai.draw_packed(lq, lk, hq, hk, d, dtype, seed)
    scale = 1.0 / np.sqrt(d)
    res = run_varlen(pk, hq, hk, scale, causal, p, DROP_SEED + seed, offset)
    q, k, v, do = (pk.f64(n) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = ov.forward(q, k, v, pk.cu_q, pk.cu_k, scale, causal, p, DROP_SEED + seed, offset)
    grads = ov.backward(q, k, v, do, pk.cu_q, pk.cu_k, scale, causal, p, DROP_SEED + seed, offset)
    what = f"{case} d={d} {dtype} causal={causal} p={p}"
    assert np.isfinite(res["o"]).all(), what
    err = float(np.abs(res["o"] - o_ref).max())
    assert err <= O_TOL[dtype] / (1 - p), f"{what}: O error {err:.3e}"
    live = np.isfinite(lse_ref)
    assert (np.isneginf(res["lse"]) == ~live).all(), f"{what}: LSE -inf pattern"
    if live.any():
        assert float(np.abs(res["lse"][live] - lse_ref[live]).max()) <= LSE_TOL[dtype], what
    for b in range(len(lq)):
        zf = lambda h, rows, cols, b=b: od.keep_mask(b * hq + h, rows, cols, p, DROP_SEED + seed, offset) / (1 - p)
        for g in range(hk):
            errs = check_sequence_group(res, grads, q, k, v, do, pk.cu_q, pk.cu_k, b, g, hq // hk, scale, causal,
                                        dtype, what, zf)
            if b == 0 and g == 0:
                report(what, errs)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_dropout_matches_dense_dropout_bitwise(d, causal):
    """Equal lengths and Hk == Hq: the packed dropout path gives the dense dropout
    path's bits (mask head b H + h, positions inside the sequence), and p = 0
    gives the packed path without dropout bit for bit."""
    import torch
    from exact_io_aware_04_amd import fa
    B, H, N = 3, 2, 200
    p, seed, off = 0.3, 4242 + d, 9
    say(f"[varlen dropout vs dense] d={d} causal={causal}")
    dr = ai.draw(B, H, N, d, ai.BF16, 919 + d + causal)
    q, k, v, do = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward_dropout(q, k, v, p, seed, off, None, causal)
    dq, dk, dv, D = fa.backward_dropout(q, k, v, o, lse, do, p, seed, off, None, causal)
    pk = lambda x: x.transpose(1, 2).contiguous().view(B * N, H, d)
    cu = _dev_i32(np.arange(B + 1) * N)
    o2, lse2 = fa.forward_varlen(pk(q), pk(k), pk(v), cu, cu, N, N, None, causal, p_drop=p, seed=seed, offset=off)
    dq2, dk2, dv2, _ = fa.backward_varlen(pk(q), pk(k), pk(v), o2, lse2, pk(do), cu, cu, N, N, None, causal,
                                          p_drop=p, seed=seed, offset=off)
    o0, lse0 = fa.forward_varlen(pk(q), pk(k), pk(v), cu, cu, N, N, None, causal)
    g0 = fa.backward_varlen(pk(q), pk(k), pk(v), o0, lse0, pk(do), cu, cu, N, N, None, causal)
    dev_pk = (pk(q), pk(k), pk(v))
    from exact_io_aware_04_amd.fa import FA_BF16, fa_bwd_preprocess, fa_bwd_varlen_dropout, fa_fwd_varlen_dropout
    o3, lse3 = torch.empty_like(o0), torch.empty_like(lse0)
    st = fa_fwd_varlen_dropout(*(t.data_ptr() for t in dev_pk), o3.data_ptr(), lse3.data_ptr(), cu.data_ptr(),
                               cu.data_ptr(), B, B * N, B * N, N, N, H, H, d, FA_BF16, 1.0 / np.sqrt(d), int(causal),
                               0.0, seed, off, None)
    assert st == 0
    D3 = torch.empty_like(lse0)
    assert fa_bwd_preprocess(o3.data_ptr(), pk(do).data_ptr(), D3.data_ptr(), 1, H, B * N, d, FA_BF16, None) == 0
    g3 = tuple(torch.empty_like(t) for t in dev_pk)
    st = fa_bwd_varlen_dropout(*(t.data_ptr() for t in dev_pk), pk(do).data_ptr(), lse3.data_ptr(), D3.data_ptr(),
                               *(t.data_ptr() for t in g3), cu.data_ptr(), cu.data_ptr(), B, B * N, B * N, N, N, H,
                               H, d, FA_BF16, 1.0 / np.sqrt(d), int(causal), 0.0, seed, off, None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o2, pk(o))
    assert torch.equal(lse2, lse.transpose(1, 2).contiguous().view(B * N, H))
    for a, b_ in ((dq2, dq), (dk2, dk), (dv2, dv)):
        assert torch.equal(a, pk(b_))
    assert torch.equal(o3, o0) and torch.equal(lse3, lse0)
    for a, b_ in zip(g3, g0[:3]):
        assert torch.equal(a, b_)
