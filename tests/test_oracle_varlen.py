"""Pins for the packed variable-length / grouped-head oracle (oracle/varlen.py).

Each pin ties the oracle to something other than its own code: a pure-Python
brute force of the definition, the dense batched oracle on equal lengths,
explicit head repetition for grouped heads, closed-form special cases of the
causal alignment, finite differences and gradient invariants.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.dropout as od
import oracle.varlen as ov


def _case(seed, lq, lk, hq, hk, d=8):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((cu_q[-1], hq, d))
    k = rng.standard_normal((cu_k[-1], hk, d))
    v = rng.standard_normal((cu_k[-1], hk, d))
    do = rng.standard_normal((cu_q[-1], hq, d))
    return q, k, v, do, cu_q, cu_k


def _brute(q, k, v, cu_q, cu_k, scale, causal):
    """The definition with Python loops: per sequence, head and query row, the
    visible keys are j <= i + (n_k - n_q) when causal (all keys otherwise)."""
    tq, hq, d = q.shape
    grp = hq // k.shape[1]
    o = np.zeros_like(q)
    lse = np.full((tq, hq), -math.inf)
    for b in range(len(cu_q) - 1):
        sq, eq, sk, ek = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        nq, nk = eq - sq, ek - sk
        for h in range(hq):
            for i in range(nq):
                vis = [j for j in range(nk) if (not causal) or j <= i + (nk - nq)]
                if not vis:
                    continue
                sc = [scale * sum(q[sq + i, h, c] * k[sk + j, h // grp, c] for c in range(d)) for j in vis]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                tot = sum(w)
                lse[sq + i, h] = m + math.log(tot)
                for c in range(d):
                    o[sq + i, h, c] = sum(wj * v[sk + j, h // grp, c] for wj, j in zip(w, vis)) / tot
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk,hq,hk", [([3, 5], [4, 5], 4, 2), ([1, 2, 6], [7, 2, 3], 3, 1), ([4], [4], 2, 2)])
def test_brute_force(causal, lq, lk, hq, hk):
    q, k, v, _, cu_q, cu_k = _case(11, lq, lk, hq, hk)
    o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.37, causal)
    ob, lb = _brute(q, k, v, cu_q, cu_k, 0.37, causal)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], lb[np.isfinite(lb)], rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense_batched(causal):
    B, H, N, d = 3, 2, 9, 8
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    o, lse = oracle.forward(q, k, v, 0.5, causal)
    dq, dk, dv, dd = oracle.backward(q, k, v, do, 0.5, causal)
    pk = lambda x: x.transpose(0, 2, 1, 3).reshape(B * N, H, d)
    cu = np.arange(B + 1) * N
    o2, lse2 = ov.forward(pk(q), pk(k), pk(v), cu, cu, 0.5, causal)
    g2 = ov.backward(pk(q), pk(k), pk(v), pk(do), cu, cu, 0.5, causal)
    np.testing.assert_allclose(o2, pk(o), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse.transpose(0, 2, 1).reshape(B * N, H), rtol=1e-13)
    for a, b_ in zip(g2[:3], (dq, dk, dv)):
        np.testing.assert_allclose(a, pk(b_), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g2[3], dd.transpose(0, 2, 1).reshape(B * N, H), rtol=1e-12, atol=1e-12)


def test_grouped_heads_equal_repeated_heads():
    q, k, v, do, cu_q, cu_k = _case(7, [5, 3], [6, 8], 6, 2)
    grp = 3
    kr, vr = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    for causal in (False, True):
        o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.4, causal)
        o_r, lse_r = ov.forward(q, kr, vr, cu_q, cu_k, 0.4, causal)
        np.testing.assert_allclose(o, o_r, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, lse_r, rtol=1e-13)
        dq, dk, dv, _ = ov.backward(q, k, v, do, cu_q, cu_k, 0.4, causal)
        dq_r, dk_r, dv_r, _ = ov.backward(q, kr, vr, do, cu_q, cu_k, 0.4, causal)
        np.testing.assert_allclose(dq, dq_r, rtol=1e-12, atol=1e-12)
        # a shared key/value head collects the gradients of every query head reading it
        np.testing.assert_allclose(dk, dk_r.reshape(dk.shape[0], 2, grp, -1).sum(axis=2), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv, dv_r.reshape(dv.shape[0], 2, grp, -1).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_causal_alignment_special_cases():
    # one query against many keys (decode): causal sees every key
    q, k, v, _, cu_q, cu_k = _case(3, [1, 1], [6, 9], 2, 1)
    a = ov.forward(q, k, v, cu_q, cu_k, 0.3, True)
    b_ = ov.forward(q, k, v, cu_q, cu_k, 0.3, False)
    np.testing.assert_allclose(a[0], b_[0], rtol=1e-14)
    # the last query row of each sequence sees every key
    q, k, v, _, cu_q, cu_k = _case(4, [3, 4], [7, 4], 2, 2)
    a = ov.forward(q, k, v, cu_q, cu_k, 0.3, True)
    b_ = ov.forward(q, k, v, cu_q, cu_k, 0.3, False)
    last = cu_q[1:] - 1
    np.testing.assert_allclose(a[0][last], b_[0][last], rtol=1e-14)
    # more queries than keys: the first n_q - n_k queries see nothing
    q, k, v, _, cu_q, cu_k = _case(5, [6], [2], 1, 1)
    o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.3, True)
    assert np.all(o[:4] == 0) and np.all(np.isneginf(lse[:4])) and np.all(np.isfinite(lse[4:]))
    # query row 4 sees key 0 only: O = v_0
    np.testing.assert_allclose(o[4, 0], v[0, 0], rtol=1e-14)


def test_empty_sequences():
    q, k, v, do, cu_q, cu_k = _case(9, [0, 3, 2], [4, 0, 3], 2, 1)
    o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.3, False)
    assert np.all(o[0:3] == 0) and np.all(np.isneginf(lse[0:3]))      # sequence 1 has no keys
    dq, dk, dv, dd = ov.backward(q, k, v, do, cu_q, cu_k, 0.3, False)
    assert np.all(dk[0:4] == 0) and np.all(dv[0:4] == 0)                # sequence 0 has no queries
    assert np.all(dq[0:3] == 0)


def test_finite_differences_grouped_varlen_causal():
    q, k, v, do, cu_q, cu_k = _case(21, [2, 3], [4, 3], 4, 2, d=4)
    scale, h = 0.7, 1e-6
    dq, dk, dv, _ = ov.backward(q, k, v, do, cu_q, cu_k, scale, True)

    def loss(q_, k_, v_):
        return float((ov.forward(q_, k_, v_, cu_q, cu_k, scale, True)[0] * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_gradient_invariants_and_d_identity():
    q, k, v, do, cu_q, cu_k = _case(13, [5, 2], [3, 6], 4, 1)
    o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.5, True)
    dq, dk, dv, dd = ov.backward(q, k, v, do, cu_q, cu_k, 0.5, True)
    live = np.isfinite(lse)
    np.testing.assert_allclose(dd[live], (do * o).sum(axis=2)[live], rtol=1e-12, atol=1e-12)
    for b in range(2):
        sk, ek, sq, eq = cu_k[b], cu_k[b + 1], cu_q[b], cu_q[b + 1]
        np.testing.assert_allclose(dk[sk:ek].sum(axis=0), 0.0, atol=1e-12)
        dsum = (do[sq:eq] * live[sq:eq, :, None]).sum(axis=(0, 1))
        np.testing.assert_allclose(dv[sk:ek, 0].sum(axis=0), dsum, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [[0, 9], [0, 3, 9], [0, 1, 2, 5, 5, 9], [0, 8, 9]])
def test_merge_of_key_subsets_equals_full(causal, cuts):
    """Page 1, key design 2: results over disjoint key subsets merge into the
    full softmax. Subsets a causal row cannot see carry LSE = -inf."""
    rng = np.random.default_rng(17)
    nq, nk, d = 4, 9, 6
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    off = nk - nq
    o_full, lse_full = oracle.forward_head(q, k, v, 0.6, causal, diag_offset=off)
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        keys = np.arange(a, b)
        vis = np.ones((nq, keys.size), bool) if not causal else keys[None, :] <= np.arange(nq)[:, None] + off
        sc = np.where(vis, 0.6 * q @ k[a:b].T, -np.inf)
        m = sc.max(axis=1, initial=-np.inf)
        live = np.isfinite(m)
        e = np.where(vis, np.exp(sc - np.where(live, m, 0)[:, None]), 0.0)
        ell = e.sum(axis=1)
        parts_o.append(np.where(live[:, None], (e @ v[a:b]) / np.where(live, ell, 1)[:, None], 0.0))
        parts_l.append(np.where(live, np.where(live, m, 0) + np.log(np.where(live, ell, 1)), -np.inf))
    o, lse = oracle.merge_normalised(parts_o, parts_l)
    np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_full, rtol=1e-12)
    if len(parts_o) > 1:   # the plain average of the partial outputs is not the merge
        assert not np.allclose(np.mean(parts_o, axis=0), o_full)


def test_merge_forms_agree():
    """The (O, LSE) merge and the (m, l, O~) merge of page 3's block states agree."""
    rng = np.random.default_rng(23)
    s1, s2 = rng.standard_normal((3, 4)), rng.standard_normal((3, 5))
    v1, v2 = rng.standard_normal((4, 2)), rng.standard_normal((5, 2))
    m, ell, acc = oracle.merge_softmax_blocks(oracle.softmax_block_state(s1, v1), oracle.softmax_block_state(s2, v2))
    a1, a2 = oracle.softmax_block_state(s1, v1), oracle.softmax_block_state(s2, v2)
    o, lse = oracle.merge_normalised([a1[2] / a1[1][:, None], a2[2] / a2[1][:, None]],
                                     [a1[0] + np.log(a1[1]), a2[0] + np.log(a2[1])])
    np.testing.assert_allclose(o, acc / ell[:, None], rtol=1e-13)
    np.testing.assert_allclose(lse, m + np.log(ell), rtol=1e-13)


# ---- dropout on packed batches (oracle.dropout per sequence and head)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_equal_lengths_match_dense_dropout(causal):
    """Equal-length packed batch with dropout == the dense dropout oracle: the
    mask of query head h of sequence b is that of dense head b H + h."""
    B, H, N, d = 3, 2, 9, 8
    rng = np.random.default_rng(6)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    p, seed, off = 0.3, 0xABCDEF12345, 5
    o, lse = od.forward(q, k, v, 0.5, causal, p, seed, off)
    dq, dk, dv, dd = od.backward(q, k, v, do, 0.5, causal, p, seed, off)
    pk = lambda x: x.transpose(0, 2, 1, 3).reshape(B * N, H, d)
    cu = np.arange(B + 1) * N
    o2, lse2 = ov.forward(pk(q), pk(k), pk(v), cu, cu, 0.5, causal, p, seed, off)
    g2 = ov.backward(pk(q), pk(k), pk(v), pk(do), cu, cu, 0.5, causal, p, seed, off)
    np.testing.assert_allclose(o2, pk(o), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse.transpose(0, 2, 1).reshape(B * N, H), rtol=1e-13)
    for a, b_ in zip(g2[:3], (dq, dk, dv)):
        np.testing.assert_allclose(a, pk(b_), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g2[3], dd.transpose(0, 2, 1).reshape(B * N, H), rtol=1e-12, atol=1e-12)
    # and it differs from the run without dropout
    o0, _ = ov.forward(pk(q), pk(k), pk(v), cu, cu, 0.5, causal)
    assert np.abs(o0 - o2).max() > 1e-3


def test_dropout_grouped_heads_equal_repeated_heads():
    """With dropout, a shared key/value head still collects the gradients of
    every query head that reads it, each query head with its own mask."""
    q, k, v, do, cu_q, cu_k = _case(8, [5, 3, 0], [6, 8, 2], 6, 2)
    grp = 3
    kr, vr = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    p, seed = 0.25, 99
    for causal in (False, True):
        o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.4, causal, p, seed)
        o_r, lse_r = ov.forward(q, kr, vr, cu_q, cu_k, 0.4, causal, p, seed)
        np.testing.assert_allclose(o, o_r, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, lse_r, rtol=1e-13)
        dq, dk, dv, _ = ov.backward(q, k, v, do, cu_q, cu_k, 0.4, causal, p, seed)
        dq_r, dk_r, dv_r, _ = ov.backward(q, kr, vr, do, cu_q, cu_k, 0.4, causal, p, seed)
        np.testing.assert_allclose(dq, dq_r, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dk, dk_r.reshape(dk.shape[0], 2, grp, -1).sum(axis=2), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv, dv_r.reshape(dv.shape[0], 2, grp, -1).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_dropout_packed_causal_alignment_uses_positions_in_the_sequence():
    """Causal packed rows with fewer queries than keys: row i of sequence b
    matches the dense dropout head of b Hq + h at query position i, keys
    0..n_k-1, with the diagonal moved by n_k - n_q."""
    q, k, v, do, cu_q, cu_k = _case(9, [3, 4], [7, 4], 2, 2)
    p, seed, off = 0.4, 7, 3
    o, lse = ov.forward(q, k, v, cu_q, cu_k, 0.6, True, p, seed, off)
    sq, eq, sk, ek = int(cu_q[0]), int(cu_q[1]), int(cu_k[0]), int(cu_k[1])
    o_h, lse_h = od.forward_head(q[sq:eq, 1], k[sk:ek, 1], v[sk:ek, 1], 0.6, True, p, seed, off, 0 * 2 + 1,
                                 diag_offset=(ek - sk) - (eq - sq))
    np.testing.assert_allclose(o[sq:eq, 1], o_h, rtol=1e-13, atol=1e-13)
    sq, eq, sk, ek = int(cu_q[1]), int(cu_q[2]), int(cu_k[1]), int(cu_k[2])
    keep = od.keep_mask(1 * 2 + 0, np.arange(eq - sq), np.arange(ek - sk), p, seed, off)
    # the second sequence's head 0 uses the mask rows 0..3 of head 2, not the packed row numbers
    o_h, _ = od.forward_head(q[sq:eq, 0], k[sk:ek, 0], v[sk:ek, 0], 0.6, True, p, seed, off, 2, diag_offset=0)
    np.testing.assert_allclose(o[sq:eq, 0], o_h, rtol=1e-13, atol=1e-13)
    assert keep.shape == (4, 4) and not keep.all()
