"""Dropout on P (fa_fwd_dropout / fa_bwd_dropout) vs oracle/dropout.py.

Besides tolerance parity on outputs and gradients, the keep mask itself is
compared bit for bit: with V the identity the forward's output row i is
P_i: o Z_i: (zero exactly where dropped), and with dO the identity the
backward's dV exposes the mask the dK/dV kernel regenerates.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle.dropout as od
from error_model import gradient_scales_head
from harness import LSE_TOL, O_TOL, check_grads, from_dev, report, say, to_dev

pytestmark = pytest.mark.gpu

SEED = 0x5EED_0000_1234_ABCD


def _run(dr, scale, causal, p, seed, offset, mask=None):
    import torch
    from exact_io_aware_04_amd import fa
    q, k, v, do = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v", "do"))
    bm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    o, lse = fa.forward_dropout(q, k, v, p, seed, offset, scale, causal, bm)
    dq, dk, dv, D = fa.backward_dropout(q, k, v, o, lse, do, p, seed, offset, scale, causal, bm)
    torch.cuda.synchronize()
    return {"o": from_dev(o, dr.dtype), "lse": lse.double().cpu().numpy(), "dq": from_dev(dq, dr.dtype),
            "dk": from_dev(dk, dr.dtype), "dv": from_dev(dv, dr.dtype), "dev": (o, lse, dq, dk, dv)}


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("mode", ["dense", "causal", "mask"])
@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [17, 128, 300])
def test_dropout_parity(n, d, dtype, mode, p):
    causal = mode == "causal"
    seed = 50_000 + 7 * n + d + (1 if dtype == ai.BF16 else 0) + (3 if causal else 0) + int(10 * p)
    mask = ai.random_block_mask(-(-n // 128), 0.6, seed) if mode == "mask" else None
    say(f"[dropout] N={n} d={d} {dtype} {mode} p={p} seed={seed}")
    dr = ai.draw(1, 2, n, d, dtype, seed)
    scale = 1.0 / np.sqrt(d)
    res = _run(dr, scale, causal, p, SEED + seed, 3, mask)
    for h in range(2):
        q, k, v, do = (dr.f64(x, 0, h) for x in ("q", "k", "v", "do"))
        o_ref, lse_ref = od.forward_head(q, k, v, scale, causal, p, SEED + seed, 3, h, mask, 128)
        dq, dk, dv, _ = od.backward_head(q, k, v, do, scale, causal, p, SEED + seed, 3, h, mask, 128)
        what = f"N={n} d={d} {dtype} {mode} p={p} h={h}"
        err = float(np.abs(res["o"][0, h] - o_ref).max())
        assert err <= O_TOL[dtype] / (1 - p), f"{what}: O error {err:.3e}"
        live = np.isfinite(lse_ref)
        assert (np.isneginf(res["lse"][0, h]) == ~live).all(), what
        if live.any():
            assert float(np.abs(res["lse"][0, h][live] - lse_ref[live]).max()) <= LSE_TOL[dtype], what
        z = lambda rows, cols, h=h: od.keep_mask(h, rows, cols, p, SEED + seed, 3) / (1.0 - p)
        scales = gradient_scales_head(q, k, v, do, scale, causal, mask, 128, z=z)
        report(what, check_grads({n_: res[n_][0, h] for n_ in ("dq", "dk", "dv")}, {"dq": dq, "dk": dk, "dv": dv},
                                 what, scales, dtype))


@pytest.mark.parametrize("d", [64, 128])
def test_mask_bits_exact(d):
    """V = I (forward) and dO = I (dK/dV kernel): zero patterns equal the oracle mask exactly."""
    import torch
    from exact_io_aware_04_amd import fa
    n, p = 64, 0.3
    say(f"[dropout-mask] d={d}")
    rng = np.random.default_rng(d)
    q = torch.from_numpy((0.3 * rng.standard_normal((1, 2, n, d))).astype(np.float32)).to(torch.bfloat16).cuda()
    k = torch.from_numpy((0.3 * rng.standard_normal((1, 2, n, d))).astype(np.float32)).to(torch.bfloat16).cuda()
    eye = torch.zeros((1, 2, n, d), dtype=torch.bfloat16)
    eye[0, :, torch.arange(n), torch.arange(n)] = 1.0
    eye = eye.cuda()
    o, lse = fa.forward_dropout(q, k, eye, p, SEED, 11)
    _, _, dv, _ = fa.backward_dropout(q, k, eye, o, lse, eye, p, SEED, 11)
    torch.cuda.synchronize()
    for h in range(2):
        keep = od.keep_mask(h, np.arange(n), np.arange(n), p, SEED, 11)
        fwd_keep = o[0, h, :, :n].float().cpu().numpy() != 0
        np.testing.assert_array_equal(fwd_keep, keep)
        bwd_keep = dv[0, h, :n, :n].float().cpu().numpy().T != 0     # dV[j, i] = P_ij Z_ij
        np.testing.assert_array_equal(bwd_keep, keep)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_p_zero_matches_plain_path_bitwise(d, causal):
    import torch
    from exact_io_aware_04_amd import fa
    say(f"[dropout-p0] d={d} causal={causal}")
    dr = ai.draw(2, 2, 200, d, ai.BF16, 900 + d)
    q, k, v, do = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v", "do"))
    a = fa.forward(q, k, v, None, causal)
    b = fa.forward_dropout(q, k, v, 0.0, 123, 0, None, causal)
    ga = fa.backward(q, k, v, a[0], a[1], do, None, causal)
    gb = fa.backward_dropout(q, k, v, b[0], b[1], do, 0.0, 123, 0, None, causal)
    torch.cuda.synchronize()
    for x, y in zip(list(a) + list(ga[:3]), list(b) + list(gb[:3])):
        assert torch.equal(x, y)


def test_offset_and_seed_change_the_mask():
    import torch
    from exact_io_aware_04_amd import fa
    say("[dropout-offset]")
    dr = ai.draw(1, 1, 128, 64, ai.F16, 5)
    q, k, v = (to_dev(getattr(dr, n), dr.dtype) for n in ("q", "k", "v"))
    o1, _ = fa.forward_dropout(q, k, v, 0.5, 1, 0)
    o2, _ = fa.forward_dropout(q, k, v, 0.5, 1, 1)
    o3, _ = fa.forward_dropout(q, k, v, 0.5, 2, 0)
    o4, _ = fa.forward_dropout(q, k, v, 0.5, 1, 0)
    torch.cuda.synchronize()
    assert not torch.equal(o1, o2) and not torch.equal(o1, o3)
    assert torch.equal(o1, o4)
