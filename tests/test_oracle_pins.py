"""Pins that tie the float64 oracle to what the pages and the mathematics fix.

Each test names the passage or closed form it checks. Several tests plant a
plausible mistake in a copy of the oracle's arithmetic (on the CPU) and
assert that some pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from attn_inputs import butterfly_block_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# P1: the page-3 worked example, printed digits and closed form
# ---------------------------------------------------------------------------
def test_worked_example_matches_printed_digits():
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_example.json")))
    s = np.array(g["scores"])
    v = np.array(g["values"])
    c = g["split"]
    pr, tol = g["printed"], g["printed_abs_tolerance"]

    st1 = oracle.softmax_block_state(s[None, :c], v[:c, None])
    st2 = oracle.softmax_block_state(s[None, c:], v[c:, None])
    assert st1[0][0] == pr["m_block1"] and st2[0][0] == pr["m_block2"]
    assert abs(st1[1][0] - pr["l_block1"]) < tol["l_block1"]
    assert abs(st2[1][0] - pr["l_block2"]) < tol["l_block2"]
    assert abs(st1[2][0, 0] - pr["otilde_block1"]) < tol["otilde_block1"]
    assert abs(st2[2][0, 0] - pr["otilde_block2"]) < tol["otilde_block2"]
    m, ell, ot = oracle.merge_softmax_blocks(st1, st2)
    assert m[0] == pr["m"]
    assert abs(ell[0] - pr["l"]) < tol["l"]
    assert abs(ot[0, 0] - pr["otilde"]) < tol["otilde"]
    assert abs(ot[0, 0] / ell[0] - pr["o"]) < tol["o"]

    # The same row as attention: d = 1, q = 1, keys = the scores, scale 1.
    q = np.ones((4, 1))
    k = s[:, None].copy()
    o, lse = oracle.forward_head(q, k, v[:, None].copy(), scale=1.0)
    assert np.all(np.abs(o[:, 0] - pr["o"]) < tol["o"])
    # Closed form: l = e^-3 + e^-2 + e^-1 + 1, LSE = 4 + ln l, O = sum e^{s-4} v / l.
    ell_cf = math.exp(-3) + math.exp(-2) + math.exp(-1) + 1.0
    o_cf = (10 * math.exp(-3) + 20 * math.exp(-2) + 30 * math.exp(-1) + 40) / ell_cf
    np.testing.assert_allclose(o[:, 0], o_cf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, 4.0 + math.log(ell_cf), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P2: merging two block states equals the full softmax (key design 2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split", [1, 7, 32, 63])
def test_two_block_merge_equals_full_softmax(split):
    n, d = 64, 8
    q, k, v = rand((5, d), 1), rand((n, d), 2), rand((n, d), 3)
    scale = 0.37
    s = scale * q @ k.T
    a = oracle.softmax_block_state(s[:, :split], v[:split])
    b = oracle.softmax_block_state(s[:, split:], v[split:])
    m, ell, ot = oracle.merge_softmax_blocks(a, b)
    o, lse = oracle.forward_head(q, k, v, scale)
    np.testing.assert_allclose(ot / ell[:, None], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m + np.log(ell), lse, rtol=1e-12, atol=1e-13)
    # Order of the blocks does not matter.
    m2, ell2, ot2 = oracle.merge_softmax_blocks(b, a)
    np.testing.assert_allclose(ot2 / ell2[:, None], o, rtol=1e-12, atol=1e-13)


def test_independently_normalised_blocks_do_not_merge_by_sum():
    """Page 1 warns that adding per-block softmax outputs is wrong: show the merge is needed."""
    n, d = 32, 4
    q, k, v = rand((3, d), 4), rand((n, d), 5), rand((n, d), 6)
    s = q @ k.T
    o, _ = oracle.forward_head(q, k, v, 1.0)
    a = oracle.softmax_block_state(s[:, :16], v[:16])
    b = oracle.softmax_block_state(s[:, 16:], v[16:])
    naive = a[2] / a[1][:, None] + b[2] / b[1][:, None]
    assert np.abs(naive - o).max() > 1e-3


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (pure-Python loops, no numpy linear algebra)
# ---------------------------------------------------------------------------
def _loop_attention(q, k, v, scale, causal, bm, bs):
    n, d = len(q), len(q[0])
    O, L = [], []
    for i in range(n):
        sc = []
        for j in range(n):
            ok = (not causal or j <= i) and (bm is None or bm[i // bs][j // bs])
            if ok:
                sc.append((j, scale * sum(q[i][t] * k[j][t] for t in range(d))))
        if not sc:
            O.append([0.0] * d)
            L.append(-math.inf)
            continue
        mx = max(x for _, x in sc)
        w = [(j, math.exp(x - mx)) for j, x in sc]
        tot = sum(x for _, x in w)
        O.append([sum(x * v[j][t] for j, x in w) / tot for t in range(d)])
        L.append(mx + math.log(tot))
    return np.array(O), np.array(L)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_forward_matches_loop_brute_force(causal, masked):
    n, d, bs = 6, 3, 2
    q, k, v = rand((n, d), 10), rand((n, d), 11), rand((n, d), 12)
    bm = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], dtype=np.uint8) if masked else None
    o, lse = oracle.forward_head(q, k, v, 0.7, causal, bm, bs)
    o2, lse2 = _loop_attention(q.tolist(), k.tolist(), v.tolist(), 0.7, causal,
                               None if bm is None else bm.tolist(), bs)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P3: rows of P sum to one; P4: identical keys; P5: causal first row
# ---------------------------------------------------------------------------
def test_rows_of_p_sum_to_one():
    n, d = 40, 6
    q, k = rand((n, d), 20, 3.0), rand((n, d), 21, 3.0)
    eye = np.eye(n)
    for causal in (False, True):
        # O with V = identity is P itself.
        p, _ = oracle.forward_head(q, k, eye, 0.5, causal)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    n, d = 24, 5
    q, v, g = rand((n, d), 30), rand((n, d), 31), rand((n, d), 32)
    k = np.tile(rand((1, d), 33), (n, 1))
    o, _ = oracle.forward_head(q, k, v, 0.8, causal)
    if causal:
        ref = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    else:
        ref = np.tile(v.mean(axis=0), (n, 1))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    dq, _, _, _ = oracle.backward_head(q, k, v, g, 0.8, causal)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_causal_first_row_and_last_row():
    n, d = 17, 4
    q, k, v = rand((n, d), 40), rand((n, d), 41), rand((n, d), 42)
    s = 0.6
    o, lse = oracle.forward_head(q, k, v, s, causal=True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], s * q[0] @ k[0], rtol=1e-14)
    o_full, lse_full = oracle.forward_head(q, k, v, s, causal=False)
    np.testing.assert_allclose(o[-1], o_full[-1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[-1], lse_full[-1], rtol=1e-13)


# ---------------------------------------------------------------------------
# P6: finite differences of L = sum(O * G)
# ---------------------------------------------------------------------------
def _fd_grads(q, k, v, g, scale, causal, bm, bs, h=1e-6):
    def loss(qq, kk, vv):
        o, _ = oracle.forward_head(qq, kk, vv, scale, causal, bm, bs)
        return float((o * g).sum())
    out = []
    for which in range(3):
        base = [q, k, v]
        grad = np.zeros_like(base[which])
        for idx in np.ndindex(grad.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            grad[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        out.append(grad)
    return out


FD_CASES = [
    dict(n=5, d=3, scale=1.0, causal=False, masked=False),
    dict(n=6, d=4, scale=0.37, causal=True, masked=False),
    dict(n=6, d=2, scale=0.37, causal=False, masked=True),
    dict(n=6, d=3, scale=1.0, causal=True, masked=True),
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: f"n{c['n']}d{c['d']}s{c['scale']}c{int(c['causal'])}m{int(c['masked'])}")
def test_backward_matches_finite_differences(case):
    n, d = case["n"], case["d"]
    q, k, v, g = (rand((n, d), 50 + i) for i in range(4))
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8) if case["masked"] else None
    dq, dk, dv, _ = oracle.backward_head(q, k, v, g, case["scale"], case["causal"], bm, 2)
    fq, fk, fv = _fd_grads(q, k, v, g, case["scale"], case["causal"], bm, 2)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)


def _mutant_backward(q, k, v, do, scale, mutation):
    """The oracle's backward arithmetic with one planted mistake (dense case)."""
    s = scale * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    D = (p * dp).sum(axis=1, keepdims=True)
    if mutation == "drop_D":             # the form printed in page 2's backward display
        ds = p * dp
    elif mutation == "sign_D":
        ds = p * (dp + D)
    else:
        ds = p * (dp - D)
    dq = scale * ds @ k
    dk = scale * ds.T @ q
    if mutation == "drop_scale":         # the pages' pseudocode omits the scale
        dq, dk = ds @ k, ds.T @ q
    if mutation == "transpose_dk":
        dk = scale * ds @ q
    if mutation == "dv_from_pT":
        dv = p @ do
    return dq, dk, dv


@pytest.mark.parametrize("mutation", ["drop_D", "sign_D", "drop_scale", "transpose_dk", "dv_from_pT"])
def test_finite_differences_catch_planted_mistakes(mutation):
    n, d, scale = 5, 5, 0.37
    q, k, v, g = (rand((n, d), 60 + i) for i in range(4))
    fq, fk, fv = _fd_grads(q, k, v, g, scale, False, None, 2)
    good = _mutant_backward(q, k, v, g, scale, None)
    for a, b in zip(good, (fq, fk, fv)):
        np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-8)
    bad = _mutant_backward(q, k, v, g, scale, mutation)
    worst = max(np.abs(a - b).max() for a, b in zip(bad, (fq, fk, fv)))
    assert worst > 1e-3, mutation


# ---------------------------------------------------------------------------
# P7: D identity; P8: special cases; P9: gradient invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_D_identity(causal):
    n, d = 33, 7
    q, k, v, g = (rand((n, d), 70 + i) for i in range(4))
    o, _ = oracle.forward_head(q, k, v, 0.4, causal)
    _, _, _, D = oracle.backward_head(q, k, v, g, 0.4, causal)
    np.testing.assert_allclose(D, (g * o).sum(axis=1), rtol=1e-12, atol=1e-12)


def test_single_token_and_zero_scale():
    d = 4
    q, k, v, g = (rand((1, d), 80 + i) for i in range(4))
    o, lse = oracle.forward_head(q, k, v, 0.9)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.9 * (q[0] @ k[0]), rtol=1e-13)
    dq, dk, dv, _ = oracle.backward_head(q, k, v, g, 0.9)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, g, rtol=1e-15)

    n = 12
    q, k, v, g = (rand((n, d), 90 + i) for i in range(4))
    o, lse = oracle.forward_head(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-14)
    dq, _, _, _ = oracle.backward_head(q, k, v, g, 0.0)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    n, d = 29, 6
    q, k, v, g = (rand((n, d), 100 + i) for i in range(4))
    dq, dk, dv, _ = oracle.backward_head(q, k, v, g, 0.5, causal)
    # sum_j dS_ij = 0 for every row, so sum_j dK_j = scale * sum_ij dS_ij q_i = 0.
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-10)
    # sum_j dV_j = sum_j sum_i P_ij dO_i = sum_i dO_i.
    np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------
# P10: mask reductions; R8b: fully masked rows
# ---------------------------------------------------------------------------
def test_all_ones_mask_equals_dense_and_diagonal_mask_is_blockwise():
    n, d, bs = 48, 4, 16
    q, k, v, g = (rand((n, d), 110 + i) for i in range(4))
    ones = np.ones((3, 3), dtype=np.uint8)
    for causal in (False, True):
        a = oracle.forward_head(q, k, v, 0.5, causal, ones, bs)
        b = oracle.forward_head(q, k, v, 0.5, causal)
        np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-14)
        ga = oracle.backward_head(q, k, v, g, 0.5, causal, ones, bs)
        gb = oracle.backward_head(q, k, v, g, 0.5, causal)
        for x, y in zip(ga, gb):
            np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)
    diag = np.eye(3, dtype=np.uint8)
    o, lse = oracle.forward_head(q, k, v, 0.5, False, diag, bs)
    grads = oracle.backward_head(q, k, v, g, 0.5, False, diag, bs)
    for t in range(3):
        sl = slice(t * bs, (t + 1) * bs)
        ob, lb = oracle.forward_head(q[sl], k[sl], v[sl], 0.5)
        np.testing.assert_allclose(o[sl], ob, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[sl], lb, rtol=1e-13)
        gq, gk, gv, _ = oracle.backward_head(q[sl], k[sl], v[sl], g[sl], 0.5)
        np.testing.assert_allclose(grads[0][sl], gq, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(grads[1][sl], gk, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(grads[2][sl], gv, rtol=1e-12, atol=1e-13)


def test_butterfly_mask_structure():
    m = butterfly_block_mask(128)
    assert m.sum() == 1024 and (m.sum(axis=1) == 8).all() and (m == m.T).all()
    assert all(m[i, i] for i in range(128))
    tiny = butterfly_block_mask(4)
    np.testing.assert_array_equal(tiny, [[1, 1, 1, 0], [1, 1, 0, 1], [1, 0, 1, 1], [0, 1, 1, 1]])


def test_fully_masked_row_gives_zero_output_and_no_gradient():
    n, d, bs = 8, 3, 4
    q, k, v, g = (rand((n, d), 120 + i) for i in range(4))
    bm = np.array([[1, 0], [0, 0]], dtype=np.uint8)     # rows 4..7 see no key
    o, lse = oracle.forward_head(q, k, v, 1.0, False, bm, bs)
    assert np.all(o[4:] == 0) and np.all(np.isneginf(lse[4:]))
    dq, dk, dv, D = oracle.backward_head(q, k, v, g, 1.0, False, bm, bs)
    assert np.all(dq[4:] == 0) and np.all(dk[4:] == 0) and np.all(dv[4:] == 0)
    ref = oracle.forward_head(q[:4], k[:4], v[:4], 1.0)
    np.testing.assert_allclose(o[:4], ref[0], rtol=1e-13)


# ---------------------------------------------------------------------------
# P11: permutation equivariance
# ---------------------------------------------------------------------------
def test_permutation_equivariance():
    n, d = 20, 5
    q, k, v, g = (rand((n, d), 130 + i) for i in range(4))
    perm = np.random.Generator(np.random.PCG64(7)).permutation(n)
    o, lse = oracle.forward_head(q, k, v, 0.3)
    o2, lse2 = oracle.forward_head(q, k[perm], v[perm], 0.3)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    o3, lse3 = oracle.forward_head(q[perm], k, v, 0.3)
    np.testing.assert_allclose(o3, o[perm], rtol=1e-13, atol=1e-14)
    dq, dk, dv, _ = oracle.backward_head(q, k, v, g, 0.3)
    dq2, dk2, dv2, _ = oracle.backward_head(q, k[perm], v[perm], g, 0.3)
    np.testing.assert_allclose(dq2, dq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk2, dk[perm], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv2, dv[perm], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# The sampled backward equals the whole-head backward at the sampled indices
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal,masked", [(False, False), (True, False), (False, True), (True, True)])
def test_sampled_backward_matches_whole_head(causal, masked):
    n, d, bs = 64, 8, 16
    q, k, v, g = (rand((n, d), 140 + i) for i in range(4))
    bm = butterfly_block_mask(4) if masked else None
    dq, dk, dv, D = oracle.backward_head(q, k, v, g, 0.35, causal, bm, bs)
    rows = np.array([0, 5, 17, 63])
    cols = np.array([1, 31, 32, 62])
    sq, sk, sv, sd = oracle.backward_head_sampled(q, k, v, g, 0.35, causal, bm, bs, rows, cols)
    np.testing.assert_allclose(sq, dq[rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sk, dk[cols], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sv, dv[cols], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sd, D[rows], rtol=1e-11, atol=1e-12)
    if causal:
        late = np.array([40, 47, 63])
        tq, tk, tv, _ = oracle.backward_head_sampled(q, k, v, g, 0.35, causal, bm, bs, rows, late,
                                                     first_row=40)
        np.testing.assert_allclose(tk, dk[late], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(tv, dv[late], rtol=1e-11, atol=1e-12)
        with pytest.raises(AssertionError):
            oracle.backward_head_sampled(q, k, v, g, 0.35, causal, bm, bs, rows, cols, first_row=40)


@pytest.mark.parametrize("causal", [False, True])
def test_row_subsets_partition_the_backward(causal):
    """Each query row adds its own terms to dK and dV: the backward restricted
    to disjoint row subsets sums to the whole-head backward, and dQ / D of a
    subset's rows are the whole head's."""
    n, d = 50, 6
    q, k, v, g = (rand((n, d), 160 + i) for i in range(4))
    whole = oracle.backward_head(q, k, v, g, 0.45, causal)
    rng = np.random.default_rng(3)
    perm = rng.permutation(n)
    parts = [np.sort(perm[:17]), np.sort(perm[17:30]), np.sort(perm[30:])]
    acc_k, acc_v = np.zeros_like(k), np.zeros_like(v)
    for rows in parts:
        dq, dk, dv, D = oracle.backward_head(q, k, v, g, 0.45, causal, row_block=4, rows=rows)
        np.testing.assert_allclose(dq[rows], whole[0][rows], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(D[rows], whole[3][rows], rtol=1e-12, atol=1e-14)
        others = np.setdiff1d(np.arange(n), rows)
        assert (dq[others] == 0).all() and (D[others] == 0).all()
        acc_k += dk
        acc_v += dv
    np.testing.assert_allclose(acc_k, whole[1], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(acc_v, whole[2], rtol=1e-11, atol=1e-12)


def test_batched_helpers_loop_over_heads():
    B, H, n, d = 2, 3, 10, 4
    q, k, v, g = (rand((B, H, n, d), 150 + i) for i in range(4))
    o, lse = oracle.forward(q, k, v, 0.5, causal=True)
    dq, dk, dv, D = oracle.backward(q, k, v, g, 0.5, causal=True)
    for b in range(B):
        for h in range(H):
            oh, lh = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)
            gh = oracle.backward_head(q[b, h], k[b, h], v[b, h], g[b, h], 0.5, True)
            np.testing.assert_array_equal(dq[b, h], gh[0])
