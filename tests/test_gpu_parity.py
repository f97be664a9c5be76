"""HIP path vs the float64 oracle, through the C ABI (Python binding).

Small shapes span several tiles and ragged tails and are compared element by
element; the five full-size workloads run in the launch configuration the
benchmark times and are compared on whole sampled heads, sampled rows /
columns, and invariants that hold at any size. Every GPU step prints its case
first so that a failure names it.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from harness import (GRAD_REL_TOL, LSE_TOL, O_TOL, check_D, check_forward, check_grads, from_dev, rel_fro,
                     report, run_gpu, say, to_dev)
from error_model import UNIT_ROUNDOFF, gradient_scales_head

pytestmark = pytest.mark.gpu

SMALL_N = [1, 17, 64, 127, 128, 129, 255, 256, 1000]
MODES = ["dense", "causal", "mask", "causal_mask"]


def _mask_for(mode, n, seed):
    if "mask" not in mode:
        return None
    return ai.random_block_mask(-(-n // 128), 0.5, seed)


def _oracle_head(dr, b, h, scale, causal, mask, backward=True):
    """Oracle O, LSE (and dQ, dK, dV, D) of head (b, h), plus the gradients'
    element-wise error scales under "scales"."""
    q, k, v = (dr.f64(n, b, h) for n in "qkv")
    o, lse = oracle.forward_head(q, k, v, scale, causal, mask, 128)
    out = {"o": o, "lse": lse}
    if backward:
        do = dr.f64("do", b, h)
        out["dq"], out["dk"], out["dv"], out["D"] = oracle.backward_head(q, k, v, do, scale, causal, mask, 128)
        out["scales"] = gradient_scales_head(q, k, v, do, scale, causal, mask, 128)
    return out


def _grads(res, b, h):
    return {k: res[k][b, h] for k in ("dq", "dk", "dv")}


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", SMALL_N)
def test_small_shapes(n, d, dtype, mode):
    causal = "causal" in mode
    seed = 10_000 + 97 * n + d + (1 if dtype == ai.BF16 else 0) + 7 * MODES.index(mode)
    mask = _mask_for(mode, n, seed)
    say(f"[small] N={n} d={d} {dtype} {mode} seed={seed}")
    dr = ai.draw(1, 2, n, d, dtype, seed)
    scale = 1.0 / np.sqrt(d)
    res = run_gpu(dr, scale, causal, mask, backward=True)
    o_dev = res["o"]
    for h in range(2):
        ref = _oracle_head(dr, 0, h, scale, causal, mask)
        what = f"N={n} d={d} {dtype} {mode} h={h}"
        check_forward(res["o"][0, h], res["lse"][0, h], ref["o"], ref["lse"], dtype, what)
        report(what, check_grads(_grads(res, 0, h), ref, what, ref["scales"], dtype))
        check_D(res["D"][0, h], dr.f64("do", 0, h), o_dev[0, h], what)


def _rescales_per_row(s_scaled, causal, tile=64, threshold=8.0):
    """How often the forward's conditional rescale fires per row on these scores:
    the running reference moves (after the first tile) when a tile's maximum, in
    log2 units, exceeds it by more than `threshold`. Test-side coverage count only."""
    n = s_scaled.shape[0]
    x = s_scaled * np.log2(np.e)
    if causal:
        x = np.where(np.tril(np.ones((n, n), dtype=bool)), x, -np.inf)
    counts = np.zeros(n, dtype=np.int64)
    ref = np.full(n, -np.inf)
    for j0 in range(0, n, tile):
        m = x[:, j0:j0 + tile].max(axis=1)
        grow = m > ref + threshold
        counts += grow & np.isfinite(ref)
        ref = np.where(grow, m, ref)
    return counts


def check_forward_rounding(o, dr, b, h, scale, causal, ref, dtype, what):
    """O against the oracle under its rounding bound, and under the stated max-abs
    tolerance (2e-3 fp16, 1e-2 bf16) wherever that bound is within it. The PV
    product consumes the probabilities rounded to the operand type (RNE, unit
    roundoff u), which moves O_ic by at most u sum_j P_ij |V_jc - O_ic| <=
    u ((P |V|)_ic + |O_ic|) (the weights stay normalised), and O itself is
    rounded (u |O_ic|); a wrong rescale factor or a wrong tile errs by O(1). A
    bf16 output with |O| >= 2.56 can round by more than 1e-2 on its own."""
    u = UNIT_ROUNDOFF[dtype]
    q, k, v = (dr.f64(x, b, h) for x in "qkv")
    n = q.shape[0]
    sc = scale * (q @ k.T)
    if causal:
        sc = np.where(np.tril(np.ones((n, n), dtype=bool)), sc, -np.inf)
    p = np.exp(sc - ref["lse"][:, None])
    bound = u * (p @ np.abs(v) + 2.0 * np.abs(ref["o"])) + 1e-4
    assert np.isfinite(o).all(), what
    err = np.abs(o - ref["o"])
    inside = bound <= O_TOL[dtype]
    say(f"    {what}: O max-abs error {err.max():.3e} (rounding bound up to {bound.max():.3e}); "
        f"{inside.mean() * 100:.1f}% of elements have a bound within {O_TOL[dtype]:g}, "
        f"max error there {err[inside].max() if inside.any() else 0.0:.3e}")
    assert (err <= bound).all(), f"{what}: O error {err.max():.3e} beyond the rounding bound"
    assert (err[inside] <= O_TOL[dtype]).all(), f"{what}: O error beyond the stated tolerance"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_running_max_keeps_rising(d, dtype, causal):
    """Key norms ramp up along the sequence, so every row's maximum climbs tile
    after tile and the forward rescales its running state several times per
    row (counted below from the oracle's scores); results must still match."""
    n = 1000
    seed = 777 + d + (1 if dtype == ai.BF16 else 0) + (2 if causal else 0)
    say(f"[rescale] N={n} d={d} {dtype} causal={causal} seed={seed}")
    dr = ai.draw_ramped_keys(1, 2, n, d, dtype, seed, lo=0.2, hi=12.0, q_mult=2.0)
    scale = 1.0 / np.sqrt(d)
    q0, k0 = dr.f64("q", 0, 0), dr.f64("k", 0, 0)
    fired = _rescales_per_row(scale * (q0 @ k0.T), causal)
    assert fired[n // 2:].mean() >= 2.0, f"inputs exercise too few rescales ({fired.mean():.2f} per row)"
    res = run_gpu(dr, scale, causal, None, backward=True)
    for h in range(2):
        ref = _oracle_head(dr, 0, h, scale, causal, None)
        what = f"rescale N={n} d={d} {dtype} causal={causal} h={h}"
        check_forward_rounding(res["o"][0, h], dr, 0, h, scale, causal, ref, dtype, what)
        assert np.abs(res["lse"][0, h] - ref["lse"]).max() <= LSE_TOL[dtype], f"{what}: LSE"
        report(what, check_grads(_grads(res, 0, h), ref, what, ref["scales"], dtype))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
def test_fully_masked_rows(causal, dtype):
    """Rows whose tiles are all masked: O = 0, LSE = -inf, no gradient (reading R8b)."""
    n, d = 300, 64
    mask = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], dtype=np.uint8)
    say(f"[masked rows] causal={causal} {dtype}")
    dr = ai.draw(1, 1, n, d, dtype, 4242)
    scale = 0.125
    res = run_gpu(dr, scale, causal, mask)
    ref = _oracle_head(dr, 0, 0, scale, causal, mask)
    check_forward(res["o"][0, 0], res["lse"][0, 0], ref["o"], ref["lse"], dtype, "masked rows")
    assert (res["o"][0, 0, 128:256] == 0).all()
    report("masked rows", check_grads(_grads(res, 0, 0), ref, "masked rows", ref["scales"], dtype))
    assert (res["dq"][0, 0, 128:256] == 0).all()


@pytest.mark.parametrize("d", [64, 128])
def test_mask_rows_longer_than_2048_tiles(d):
    """A block mask with 2049 tiles per row: the kernels find kept tiles below
    2048 from a per-workgroup bitmask and read the flags of tiles past it from
    memory. Pairs of tiles form independent 256-key groups, so each group is a
    dense attention problem the oracle computes on its own."""
    n_tiles = 2049
    n = 128 * n_tiles
    t = np.arange(n_tiles)
    mask = (t[:, None] // 2 == t[None, :] // 2).astype(np.uint8)
    say(f"[mask 2049 tiles] N={n} d={d} f16")
    dr = ai.draw(1, 1, n, d, ai.F16, 90_210 + d)
    scale = 1.0 / np.sqrt(d)
    res = run_gpu(dr, scale, False, mask)
    assert np.isfinite(res["o"]).all(), "unwritten output rows"
    q, k, v, do = (dr.f64(name, 0, 0) for name in ("q", "k", "v", "do"))
    for grp in (0, 511, 1023, 1024):
        a, b = 256 * grp, min(256 * grp + 256, n)
        o, lse = oracle.forward_head(q[a:b], k[a:b], v[a:b], scale, False)
        dq, dk, dv, _ = oracle.backward_head(q[a:b], k[a:b], v[a:b], do[a:b], scale, False)
        scales = gradient_scales_head(q[a:b], k[a:b], v[a:b], do[a:b], scale, False)
        what = f"group {grp} (rows {a}..{b - 1})"
        check_forward(res["o"][0, 0, a:b], res["lse"][0, 0, a:b], o, lse, ai.F16, what)
        report(what, check_grads({"dq": res["dq"][0, 0, a:b], "dk": res["dk"][0, 0, a:b], "dv": res["dv"][0, 0, a:b]},
                                 {"dq": dq, "dk": dk, "dv": dv}, what, scales, ai.F16))


@pytest.mark.parametrize("d,dtype,causal", [(64, ai.F16, False), (128, ai.BF16, True)])
def test_random_mask_across_mask_words(d, dtype, causal):
    """Random block mask over 130 tiles per row, so the kept-tile search crosses
    the 64-tile words of the per-workgroup bitmask; rows in the tiles at the
    word boundaries, and key columns there, against the oracle."""
    n_tiles = 130
    n = 128 * n_tiles
    mask = ai.random_block_mask(n_tiles, 0.12, 7_130 + d)
    say(f"[mask 130 tiles] N={n} d={d} {dtype} causal={causal}")
    dr = ai.draw(1, 1, n, d, dtype, 7_131 + d)
    scale = 1.0 / np.sqrt(d)
    res = run_gpu(dr, scale, causal, mask)
    tiles = [0, 1, 62, 63, 64, 65, 127, 128, 129]
    rows = np.array(sorted({128 * t + r for t in tiles for r in (0, 61, 127)}))
    q, k, v, do = (dr.f64(name, 0, 0) for name in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_head(q, k, v, scale, causal, mask, 128, rows=rows)
    check_forward(res["o"][0, 0, rows], res["lse"][0, 0, rows], o_ref, lse_ref, dtype, "sampled rows")
    say(f"[mask 130 tiles] oracle gradients at {rows.size} rows / columns")
    dq, dk, dv, _ = oracle.backward_head_sampled(q, k, v, do, scale, causal, mask, 128, rows, rows)
    scales = gradient_scales_head(q, k, v, do, scale, causal, mask, 128, q_rows=rows, k_cols=rows)
    report("sampled rows / columns",
           check_grads({"dq": res["dq"][0, 0, rows], "dk": res["dk"][0, 0, rows], "dv": res["dv"][0, 0, rows]},
                       {"dq": dq, "dk": dk, "dv": dv}, "sampled rows / columns", scales, dtype))
    for name in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[name]).all(), f"non-finite {name}"


@pytest.mark.parametrize("causal", [False, True])
def test_grid_with_partial_round_of_heads(causal):
    """11 heads x 3 blocks per head: the first 8 heads are dealt to the XCDs
    round-robin by head, the last 3 heads' blocks keep their order; every
    head is compared whole against the oracle."""
    B, H, n, d = 1, 11, 300, 64
    say(f"[block order] B={B} H={H} N={n} d={d} causal={causal}")
    dr = ai.draw(B, H, n, d, ai.F16, 4_711 + int(causal))
    scale = 1.0 / np.sqrt(d)
    res = run_gpu(dr, scale, causal, None)
    for h in range(H):
        ref = _oracle_head(dr, 0, h, scale, causal, None)
        what = f"head {h}"
        check_forward(res["o"][0, h], res["lse"][0, h], ref["o"], ref["lse"], ai.F16, what)
        report(what, check_grads(_grads(res, 0, h), ref, what, ref["scales"], ai.F16))


@pytest.mark.parametrize("B,H,n,d,dtype", [(2, 8, 1000, 128, ai.BF16), (3, 8, 300, 64, ai.F16)])
def test_causal_ranked_block_order(B, H, n, d, dtype):
    """Causal heads short enough for the ranked block order (N d <= 2^19, 16 and
    24 heads: two and three heads per XCD, run rank by rank across them) in all
    three kernels, every head compared whole against the oracle."""
    say(f"[ranked order] B={B} H={H} N={n} d={d} {dtype}")
    dr = ai.draw(B, H, n, d, dtype, 8_800 + n + d)
    scale = 1.0 / np.sqrt(d)
    res = run_gpu(dr, scale, True, None)
    for b in range(B):
        for h in range(H):
            ref = _oracle_head(dr, b, h, scale, True, None)
            what = f"head ({b},{h})"
            check_forward(res["o"][b, h], res["lse"][b, h], ref["o"], ref["lse"], dtype, what)
            errs = check_grads(_grads(res, b, h), ref, what, ref["scales"], dtype)
            if h == 0:
                report(what, errs)


@pytest.mark.parametrize("dtype,causal", [(ai.BF16, True), (ai.F16, False)])
def test_wide_blocks_short_heads(dtype, causal):
    """64 heads of N = 1024 at d = 128: 256 blocks of 256 query rows, the
    smallest grid that runs the 8-wave forward and dQ workgroups (with the
    ranked block order when causal); every head compared whole against the
    oracle."""
    B, H, n, d = 4, 16, 1024, 128
    say(f"[8-wave blocks] B={B} H={H} N={n} d={d} {dtype} causal={causal}")
    dr = ai.draw(B, H, n, d, dtype, 9_100 + int(causal))
    scale = 1.0 / np.sqrt(d)
    res = run_gpu(dr, scale, causal, None)
    for b in range(B):
        for h in range(H):
            ref = _oracle_head(dr, b, h, scale, causal, None)
            what = f"head ({b},{h})"
            check_forward_rounding(res["o"][b, h], dr, b, h, scale, causal, ref, dtype, what)
            lerr = np.abs(res["lse"][b, h] - ref["lse"]).max()
            assert lerr <= LSE_TOL[dtype], f"{what}: LSE max-abs error {lerr:.3e}"
            errs = check_grads(_grads(res, b, h), ref, what, ref["scales"], dtype)
            if b == 0 and h == 0:
                report(what, errs)


def test_forward_is_bitwise_deterministic():
    import torch
    from exact_io_aware_04_amd import fa
    say("[determinism] N=1000 d=128 bf16 causal x3")
    dr = ai.draw(2, 4, 1000, 128, ai.BF16, 77, with_do=False)
    q, k, v = (to_dev(getattr(dr, n), dr.dtype) for n in "qkv")
    outs = [fa.forward(q, k, v, 0.09, True) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


@pytest.mark.parametrize("causal,d,dtype", [(True, 128, ai.BF16), (False, 64, ai.F16)])
def test_backward_is_bitwise_deterministic(causal, d, dtype):
    """The backward has no atomics: repeated runs give identical dq, dk, dv bits."""
    import torch
    from exact_io_aware_04_amd import fa
    say(f"[determinism] backward N=1000 d={d} {dtype} causal={causal} x3")
    dr = ai.draw(2, 4, 1000, d, dtype, 78)
    q, k, v, do = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, None, causal)
    runs = [fa.backward(q, k, v, o, lse, do, None, causal) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(r[:3], runs[0][:3]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("n,d,dtype,causal", [(200, 64, ai.F16, True), (300, 128, ai.BF16, False),
                                              (33, 64, ai.BF16, False), (161, 128, ai.F16, True)])
def test_outputs_stay_inside_their_buffers(n, d, dtype, causal):
    """Canaries around every output buffer; raw C entry points with sliced pointers."""
    import torch
    from exact_io_aware_04_amd import fa
    B, H = 1, 2
    say(f"[canary] N={n} d={d} {dtype} causal={causal}")
    dr = ai.draw(B, H, n, d, dtype, 91 + n + d)
    q, k, v, do = (to_dev(getattr(dr, x), dr.dtype) for x in ("q", "k", "v", "do"))
    tdt = q.dtype
    numel = B * H * n * d
    PAD = 64
    def guarded(count, dt):
        buf = torch.full((count + 2 * PAD,), 7.0, dtype=dt, device="cuda")
        return buf, buf[PAD:PAD + count]
    ob, o = guarded(numel, tdt)
    lb, lse = guarded(B * H * n, torch.float32)
    Db, D = guarded(B * H * n, torch.float32)
    qb_, dq = guarded(numel, tdt)
    kb_, dk = guarded(numel, tdt)
    vb_, dv = guarded(numel, tdt)
    s = torch.cuda.current_stream().cuda_stream
    code = fa.FA_BF16 if dtype == ai.BF16 else fa.FA_F16
    sc = 1.0 / np.sqrt(d)
    assert fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, n, d,
                     code, sc, int(causal), None, 128, s) == 0
    assert fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), D.data_ptr(), B, H, n, d, code, s) == 0
    assert fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), D.data_ptr(),
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, n, d, code,
                     sc, int(causal), None, 128, s) == 0
    torch.cuda.synchronize()
    for buf in (ob, lb, Db, qb_, kb_, vb_):
        assert (buf[:PAD] == 7.0).all() and (buf[-PAD:] == 7.0).all()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()


# ---------------------------------------------------------------------------
# Full-size workloads (the benchmark's launch configuration)
# ---------------------------------------------------------------------------
def _full_run(name):
    w = ai.WORKLOADS[name]
    say(f"[full] {name}: drawing inputs")
    dr = ai.draw_workload(w)
    mask = w.block_mask()
    say(f"[full] {name}: GPU fwd{'+bwd' if w.backward else ''}")
    res = run_gpu(dr, w.scale, w.causal, mask, backward=w.backward)
    return w, dr, mask, res


def test_full_single_head_forward():
    w, dr, mask, res = _full_run("single_head_fwd_n256_d64_f16")
    ref = _oracle_head(dr, 0, 0, w.scale, w.causal, mask, backward=False)
    check_forward(res["o"][0, 0], res["lse"][0, 0], ref["o"], ref["lse"], w.dtype, w.name)


def test_full_gpt2_medium_shape():
    w, dr, mask, res = _full_run("gpt2_medium_b64_h16_n1024_d64_f16")
    rng = np.random.Generator(np.random.PCG64(5))
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [tuple(x) for x in rng.integers(0, [w.B, w.H], size=(6, 2))]
    for b, h in heads:
        say(f"[full] {w.name}: oracle head ({b},{h})")
        ref = _oracle_head(dr, b, h, w.scale, w.causal, mask)
        what = f"{w.name} head ({b},{h})"
        check_forward(res["o"][b, h], res["lse"][b, h], ref["o"], ref["lse"], w.dtype, what)
        report(what, check_grads(_grads(res, b, h), ref, what, ref["scales"], w.dtype))
    assert np.isfinite(res["o"]).all() and np.isfinite(res["dq"]).all()


def test_full_causal_8k():
    w, dr, mask, res = _full_run("causal_b2_h32_n8192_d128_bf16")
    for b, h in [(0, 0), (1, 31)]:
        say(f"[full] {w.name}: oracle head ({b},{h})")
        ref = _oracle_head(dr, b, h, w.scale, w.causal, mask)
        what = f"{w.name} head ({b},{h})"
        check_forward(res["o"][b, h], res["lse"][b, h], ref["o"], ref["lse"], w.dtype, what)
        report(what, check_grads(_grads(res, b, h), ref, what, ref["scales"], w.dtype))
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all()


def test_full_butterfly_16k():
    w, dr, mask, res = _full_run("butterfly_b4_h16_n16384_d64_f16")
    for b, h in [(3, 5), (0, 11)]:
        say(f"[full] {w.name}: oracle head ({b},{h})")
        ref = _oracle_head(dr, b, h, w.scale, w.causal, mask)
        what = f"{w.name} head ({b},{h})"
        check_forward(res["o"][b, h], res["lse"][b, h], ref["o"], ref["lse"], w.dtype, what)
        report(what, check_grads(_grads(res, b, h), ref, what, ref["scales"], w.dtype))
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all()


def test_full_causal_64k_sampled():
    """N = 65536: whole heads are out of the oracle's reach; compare sampled
    rows of O/LSE/dQ, sampled late key columns of dK/dV, and two invariants
    over every key of the head (sum_j dV_j = sum_i dO_i, sum_j dK_j = 0)."""
    w, dr, mask, res = _full_run("causal_b1_h8_n65536_d128_bf16")
    N = w.N
    rng = np.random.Generator(np.random.PCG64(11))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, N // 2, N - 129, N - 1],
                                     rng.integers(0, N, 56)]))
    cols = np.unique(np.concatenate([[N - 1, N - 128, N - 129, N - 2048],
                                     rng.integers(N - 2048, N, 28)]))
    for h in (0, 7):
        say(f"[full] {w.name}: oracle rows/cols head {h}")
        q, k, v, do = (dr.f64(n, 0, h) for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = oracle.forward_head(q, k, v, w.scale, True, None, 128, rows=rows)
        check_forward(res["o"][0, h, rows], res["lse"][0, h, rows], o_ref, lse_ref, w.dtype, f"{w.name} h{h}")
        dq, dk, dv, _ = oracle.backward_head_sampled(q, k, v, do, w.scale, True, None, 128, rows, cols,
                                                     first_row=N - 2048)
        scales = gradient_scales_head(q, k, v, do, w.scale, True, q_rows=rows, k_cols=cols, first_row=N - 2048)
        report(f"{w.name} h{h} sampled",
               check_grads({"dq": res["dq"][0, h, rows], "dk": res["dk"][0, h, cols], "dv": res["dv"][0, h, cols]},
                           {"dq": dq, "dk": dk, "dv": dv}, f"{w.name} h{h} sampled", scales, w.dtype))
        # invariants over the whole head (hold for any N)
        sum_dv, sum_do = res["dv"][0, h].sum(axis=0), do.sum(axis=0)
        assert rel_fro(sum_dv, sum_do) <= GRAD_REL_TOL
        sum_dk = res["dk"][0, h].sum(axis=0)
        assert np.linalg.norm(sum_dk) <= 1e-2 * np.abs(res["dk"][0, h]).sum(axis=0).max()
    for n in ("o", "dq", "dk", "dv"):
        assert np.isfinite(res[n]).all()


@pytest.mark.timeout(900)
def test_full_causal_64k_early_key_columns():
    """N = 65536, early key columns: key j is seen by every query i >= j, so
    dK_j and dV_j of j near 0 sum over up to 65536 rows, the longest loops of
    the dK/dV kernel (up to 1024 query tiles per key block). The oracle needs
    LSE_i and D_i of every row for them (a full forward of one head in
    float64), so this runs on one head."""
    w, dr, mask, res = _full_run("causal_b1_h8_n65536_d128_bf16")
    N, h = w.N, 3
    cols = np.array([0, 1, 63, 64, 127, 128, 4095, 32767])
    rows = np.array([0, 1, 64, 4095])
    say(f"[full] {w.name}: oracle (all {N} rows) for key columns {cols.tolist()} of head {h}")
    q, k, v, do = (dr.f64(n, 0, h) for n in ("q", "k", "v", "do"))
    dq, dk, dv, _ = oracle.backward_head_sampled(q, k, v, do, w.scale, True, None, 128, rows, cols, first_row=0)
    say(f"[full] {w.name}: error scales for head {h}")
    scales = gradient_scales_head(q, k, v, do, w.scale, True, q_rows=rows, k_cols=cols, first_row=0)
    report(f"{w.name} h{h} early columns",
           check_grads({"dq": res["dq"][0, h, rows], "dk": res["dk"][0, h, cols], "dv": res["dv"][0, h, cols]},
                       {"dq": dq, "dk": dk, "dv": dv}, f"{w.name} h{h} early columns", scales, w.dtype))


def test_largest_head_d128_causal():
    """The largest head the ABI accepts at d = 128 (N d 4 < 2^31: N = 4,194,303,
    ragged against every tile size): byte offsets inside the head reach ~1 GiB
    and the buffer ranges approach 2^31. Sampled rows of O/LSE/dQ and late key
    columns of dK/dV against the oracle, gradient invariants over the whole head."""
    import torch
    from exact_io_aware_04_amd import fa
    N, d = 4_194_303, 128
    say(f"[largest] N={N} d={d} bf16 causal: drawing inputs")
    dr = ai.draw(1, 1, N, d, ai.BF16, 4242)
    q, k, v, do = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(d)
    say("[largest] GPU forward + backward")
    o, lse = fa.forward(q, k, v, scale, True)
    dq, dk, dv, _ = fa.backward(q, k, v, o, lse, do, scale, True)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"largest head: non-finite {name}"
    # whole-head invariants (any N): sum_j dV_j = sum_i dO_i, sum_j dK_j = 0
    sum_dv = dv[0, 0].double().sum(dim=0).cpu().numpy()
    sum_do = do[0, 0].double().sum(dim=0).cpu().numpy()
    assert rel_fro(sum_dv, sum_do) <= GRAD_REL_TOL
    sum_dk = dk[0, 0].double().sum(dim=0).cpu().numpy()
    assert np.linalg.norm(sum_dk) <= 1e-2 * float(dk[0, 0].double().abs().sum(dim=0).max())
    rng = np.random.Generator(np.random.PCG64(17))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, N // 2, N - 129, N - 2, N - 1], rng.integers(0, N, 8)]))
    first = N - 256
    cols = np.unique(np.concatenate([[N - 1, N - 2, N - 128, N - 129, N - 256], rng.integers(first, N, 11)]))
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    got = {"o": o[0, 0, ri].float().cpu().numpy().astype(np.float64),
           "lse": lse[0, 0, ri].double().cpu().numpy(),
           "dq": dq[0, 0, ri].float().cpu().numpy().astype(np.float64),
           "dk": dk[0, 0, ci].float().cpu().numpy().astype(np.float64),
           "dv": dv[0, 0, ci].float().cpu().numpy().astype(np.float64)}
    del q, k, v, do, o, lse, dq, dk, dv
    say("[largest] oracle on sampled rows / columns")
    q64, k64, v64, do64 = (dr.f64(n, 0, 0) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_head(q64, k64, v64, scale, True, None, 128, rows=rows, row_block=16)
    check_forward(got["o"], got["lse"], o_ref, lse_ref, ai.BF16, "largest head")
    gq, gk, gv, _ = oracle.backward_head_sampled(q64, k64, v64, do64, scale, True, None, 128, rows, cols,
                                                 first_row=first, row_block=16)
    scales = gradient_scales_head(q64, k64, v64, do64, scale, True, q_rows=rows, k_cols=cols, first_row=first,
                                  row_block=16)
    report("largest head sampled",
           check_grads({"dq": got["dq"], "dk": got["dk"], "dv": got["dv"]}, {"dq": gq, "dk": gk, "dv": gv},
                       "largest head sampled", scales, ai.BF16))

