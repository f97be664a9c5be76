"""The gradient error model of tests/error_model.py, on the CPU.

* its scales against pure-Python loops over the terms they sum;
* sampled rows / columns against the whole-head computation;
* a numpy emulation of the kernels' 16-bit roundings (P rounded for the PV
  and P^T dO products, dS rounded, O rounded before D is formed, the forward
  row sum over rounded probabilities) stays inside the bound, while planted
  mistakes of the kinds a kernel could make (a missing key tile, a swapped
  row, a dropped -D, a dropped scale) fall outside it.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
import oracle.dropout as od
from error_model import UNIT_ROUNDOFF, elementwise_bound, gradient_scales_head
from harness import check_grads


def _inputs(n, d, dtype, seed, nk=None):
    dr = ai.draw(1, 1, max(n, nk or n), d, dtype, seed)
    q, k, v, do = (dr.f64(x, 0, 0) for x in ("q", "k", "v", "do"))
    nk = nk or n
    return q[:n], k[:nk], v[:nk], do[:n]


@pytest.mark.parametrize("causal,use_mask,use_z,off", [(False, False, False, 0), (True, False, False, 0),
                                                       (False, True, True, 0), (True, True, False, 2)])
def test_scales_match_loops(causal, use_mask, use_z, off):
    n, nk, d, s = 5, 5 + off, 3, 0.37
    q, k, v, do = _inputs(n, d, ai.F16, 7 + off, nk)
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8) if use_mask else None
    mb = 4
    zfun = (lambda r, c: od.keep_mask(0, r, c, 0.3, 99, 0) / 0.7) if use_z else None
    got = gradient_scales_head(q, k, v, do, s, causal, mask, mb, diag_offset=off, z=zfun, row_block=2)
    keep = oracle.kept_pairs(np.arange(n), np.arange(nk), causal, mask, mb, off)
    S = np.where(keep, s * q @ k.T, -np.inf)
    P = np.zeros((n, nk))
    for i in range(n):
        if keep[i].any():
            e = np.exp(S[i] - S[i][keep[i]].max())
            P[i] = np.where(keep[i], e, 0.0) / e[keep[i]].sum()
    Z = zfun(np.arange(n), np.arange(nk)) if use_z else np.ones((n, nk))
    O = (P * Z) @ v
    D = [sum(do[i, c] * O[i, c] for c in range(d)) for i in range(n)]
    dP = Z * (do @ v.T)
    dS = P * (dP - np.array(D)[:, None])
    E = [math.sqrt(sum(do[i, c] ** 2 * (O[i, c] ** 2 + sum((P[i, j] * Z[i, j] * v[j, c]) ** 2 for j in range(nk)))
                       for c in range(d))) for i in range(n)]
    for i in range(n):
        for c in range(d):
            rq = s * math.sqrt(sum((dS[i, j] * k[j, c]) ** 2 for j in range(nk)))
            fq = s * math.sqrt(sum(k[j, c] ** 2 for j in range(nk) if keep[i, j]))
            gq = s * E[i] * sum(P[i, j] * abs(k[j, c]) for j in range(nk))
            assert got["dq"].r[i, c] == pytest.approx(rq, rel=1e-12, abs=1e-300)
            assert got["dq"].f[i, c] == pytest.approx(fq, rel=1e-12, abs=1e-300)
            assert got["dq"].g[i, c] == pytest.approx(gq, rel=1e-12, abs=1e-300)
    for j in range(nk):
        for c in range(d):
            rv = math.sqrt(sum((P[i, j] * Z[i, j] * do[i, c]) ** 2 for i in range(n)))
            rk = s * math.sqrt(sum((dS[i, j] * q[i, c]) ** 2 for i in range(n)))
            gk = s * math.sqrt(sum((P[i, j] * E[i] * q[i, c]) ** 2 for i in range(n)))
            fk = s * math.sqrt(sum(q[i, c] ** 2 for i in range(n) if keep[i, j]))
            assert got["dv"].r[j, c] == pytest.approx(rv, rel=1e-12, abs=1e-300)
            assert got["dk"].r[j, c] == pytest.approx(rk, rel=1e-12, abs=1e-300)
            assert got["dk"].g[j, c] == pytest.approx(gk, rel=1e-12, abs=1e-300)
            assert got["dk"].f[j, c] == pytest.approx(fk, rel=1e-12, abs=1e-300)


def test_sampled_scales_equal_whole_head():
    n, d = 300, 16
    q, k, v, do = _inputs(n, d, ai.BF16, 3)
    full = gradient_scales_head(q, k, v, do, 0.25, True, row_block=64)
    rows = np.array([0, 5, 130, 299])
    cols = np.array([200, 250, 299])
    part = gradient_scales_head(q, k, v, do, 0.25, True, q_rows=rows, k_cols=cols, first_row=200, row_block=64)
    for f in ("r", "g", "f"):
        np.testing.assert_allclose(getattr(part["dq"], f), getattr(full["dq"], f)[rows], rtol=1e-12)
        for name in ("dk", "dv"):
            np.testing.assert_allclose(getattr(part[name], f), getattr(full[name], f)[cols], rtol=1e-12)


def _round(x, dtype):
    return ai.bits_to_f64(ai.round_bits(np.asarray(x, dtype=np.float32), dtype), dtype)


def _emulate(q, k, v, do, s, causal, dtype, p_first: bool, mistake=None):
    """The kernels' arithmetic with every 16-bit rounding they perform, in
    float64 otherwise (no fp32 accumulation error: the model's eps covers it)."""
    n = q.shape[0]
    keep = oracle.kept_pairs(np.arange(n), np.arange(n), causal, None, 128)
    S = np.where(keep, s * q @ k.T, -np.inf)
    m = S.max(axis=1)
    pf = _round(np.exp(S - m[:, None]), dtype)              # forward probabilities, rounded
    ell = pf.sum(axis=1)
    O = _round((pf @ v) / ell[:, None], dtype)
    lse = m + np.log(ell)
    D = (do * O).sum(axis=1)
    P = np.exp(S - lse[:, None])
    Pr = _round(P, dtype)
    dv = Pr.T @ do
    dP = do @ v.T
    dsv = (Pr if p_first else P) * (dP - (0.0 if mistake == "no_D" else D[:, None]))
    dS = _round(dsv, dtype)
    sc = 1.0 if mistake == "no_scale" else s
    dq, dk = sc * dS @ k, sc * dS.T @ q
    if mistake == "missing_tile":             # key tile 64..127 never reaches dQ
        dq = sc * dS[:, :64] @ k[:64] + sc * dS[:, 128:] @ k[128:]
    if mistake == "swapped_row":
        dk[[10, 11]] = dk[[11, 10]]
    return {n_: _round(x, dtype) for n_, x in (("dq", dq), ("dk", dk), ("dv", dv))}


@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_first", [False, True])
def test_emulated_roundings_pass_and_mistakes_fail(dtype, causal, p_first):
    n, d = 256, 64
    s = 1.0 / math.sqrt(d)
    q, k, v, do = _inputs(n, d, dtype, 11 + causal)
    ref = dict(zip(("dq", "dk", "dv"), oracle.backward_head(q, k, v, do, s, causal)[:3]))
    scales = gradient_scales_head(q, k, v, do, s, causal)
    errs = check_grads(_emulate(q, k, v, do, s, causal, dtype, p_first), ref, "emulated", scales, dtype)
    for name, e in errs.items():
        assert e["worst"] < 0.5, (name, e)          # well inside the bound
        assert e["max_ratio"] < 2.0 * UNIT_ROUNDOFF[dtype]
    for mistake in ("missing_tile", "swapped_row", "no_D", "no_scale"):
        bad = _emulate(q, k, v, do, s, causal, dtype, p_first, mistake)
        caught = False
        for name in ("dq", "dk", "dv"):
            b = elementwise_bound(ref[name], scales[name], dtype)
            caught |= bool((np.abs(bad[name] - ref[name]) > b).any())
        assert caught, mistake
