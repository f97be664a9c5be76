"""Pins for the dropout oracle (oracle/dropout.py).

The attention math with a given mask is pinned by p = 0 reducing to the plain
oracle, finite differences with the mask held fixed, the D identity, the
unchanged LSE and unbiasedness (the mean output over many seeds approaches
the output without dropout). The generator's bit pattern is pinned to a
library routine: rocRAND's header implementation of Philox4x32-10, compiled
here for the host (tests/philox_rocrand_ref.cpp), at random counters and keys.
Its statistical properties are pinned too: keep rate, byte uniformity,
determinism and sensitivity to every counter and key field.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import oracle.dropout as od


def _qkv(seed, nq=7, nk=9, d=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d)),
            rng.standard_normal((nq, d)))


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_plain_attention(causal):
    q, k, v, do = _qkv(1, 8, 8)
    o, lse = od.forward_head(q, k, v, 0.4, causal, 0.0, 99, 0, 3)
    o2, lse2 = oracle.forward_head(q, k, v, 0.4, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    g = od.backward_head(q, k, v, do, 0.4, causal, 0.0, 99, 0, 3)
    g2 = oracle.backward_head(q, k, v, do, 0.4, causal)
    for a, b in zip(g, g2):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate(p):
    m = od.keep_mask(5, np.arange(256), np.arange(256), p, 0x1234_5678_9ABC_DEF0, 7)
    n = m.size
    sigma = np.sqrt(n * p * (1 - p))
    assert abs(m.sum() - n * (1 - p)) <= 5 * sigma


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(shutil.which(HIPCC) is None, reason="hipcc is needed to build the rocRAND host reference")
def test_philox_matches_rocrand(tmp_path):
    """The oracle's generator equals rocRAND's Philox4x32-10 (a separate
    implementation of the same published function) on 400 random counters and
    keys, including counters with all four words nonzero and keys above 2^32."""
    src = os.path.join(os.path.dirname(__file__), "philox_rocrand_ref.cpp")
    exe = str(tmp_path / "philox_ref")
    r = subprocess.run([HIPCC, "-O1", "-x", "hip", "--offload-arch=gfx950", src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    rng = np.random.default_rng(5)
    n = 400
    seeds = rng.integers(0, 2 ** 64, n, dtype=np.uint64)
    ctr = rng.integers(0, 2 ** 32, (n, 4), dtype=np.uint64)
    ctr[:, 1] &= np.uint64(2 ** 30 - 1)             # the reference takes (c0, c1) as 4 (c0 + 2^32 c1) in 64 bits
    ctr[:50] = 0                                   # small counters (the kernels' row / column blocks)
    ctr[:50, 0] = np.arange(50)
    seeds[:5] = [0, 1, 1234, 2 ** 32, 2 ** 64 - 1]
    lines = "".join(f"{int(s)} {int(a)} {int(b)} {int(c)} {int(d)}\n" for s, (a, b, c, d) in zip(seeds, ctr))
    out = subprocess.run([exe], input=lines, capture_output=True, text=True, timeout=60)
    assert out.returncode == 0
    ref = np.array([[int(x) for x in l.split()] for l in out.stdout.splitlines()], dtype=np.uint64)
    assert ref.shape == (n, 4)
    got = od.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], seeds & np.uint64(0xFFFFFFFF),
                           seeds >> np.uint64(32))
    np.testing.assert_array_equal(np.stack(got, axis=1).astype(np.uint64), ref)


def test_word_bytes_uniform():
    j, i = np.meshgrid(np.arange(128), np.arange(256))
    words = np.concatenate([w.ravel() for w in od.philox4x32_10(j, i, 11, 0, 2024, 7)])
    for shift in (0, 8, 16, 24):
        counts = np.bincount((words >> np.uint32(shift)) & np.uint32(255), minlength=256)
        expected = words.size / 256
        chi2 = float(((counts - expected) ** 2 / expected).sum())
        assert chi2 < 400.0        # 255 degrees of freedom: mean 255, sd ~22.6


def test_deterministic_and_sensitive_to_every_field():
    rows, cols = np.arange(64), np.arange(64)
    base = od.keep_mask(2, rows, cols, 0.5, 777, 3)
    np.testing.assert_array_equal(base, od.keep_mask(2, rows, cols, 0.5, 777, 3))
    others = [od.keep_mask(3, rows, cols, 0.5, 777, 3), od.keep_mask(2, rows, cols, 0.5, 778, 3),
              od.keep_mask(2, rows, cols, 0.5, 777 + (1 << 32), 3), od.keep_mask(2, rows, cols, 0.5, 777, 4),
              od.keep_mask(2, rows + 64, cols, 0.5, 777, 3), od.keep_mask(2, rows, cols + 64, 0.5, 777, 3)]
    for m in others:   # independent masks agree on about half the elements at p = 0.5
        agree = float((m == base).mean())
        assert 0.45 < agree < 0.55


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_with_fixed_mask(causal):
    q, k, v, g = _qkv(3, 6, 6, 4)
    p, seed, scale, h = 0.3, 4242, 0.8, 1e-6
    dq, dk, dv, _ = od.backward_head(q, k, v, g, scale, causal, p, seed, 1, 0)

    def loss(q_, k_, v_):
        return float((od.forward_head(q_, k_, v_, scale, causal, p, seed, 1, 0)[0] * g).sum())

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            b = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*a) - loss(*b)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_d_identity_and_lse_unchanged():
    q, k, v, do = _qkv(4)
    o, lse = od.forward_head(q, k, v, 0.5, True, 0.25, 5, 0, 9, diag_offset=2)
    _, lse0 = oracle.forward_head(q, k, v, 0.5, True, diag_offset=2)
    np.testing.assert_array_equal(lse, lse0)
    _, _, _, dd = od.backward_head(q, k, v, do, 0.5, True, 0.25, 5, 0, 9, diag_offset=2)
    np.testing.assert_allclose(dd, (do * o).sum(axis=1), rtol=1e-12, atol=1e-13)


def test_unbiased_over_seeds():
    q, k, v, _ = _qkv(6, 4, 6, 3)
    o0, _ = oracle.forward_head(q, k, v, 0.7, False)
    mean = np.mean([od.forward_head(q, k, v, 0.7, False, 0.4, s, 0, 0)[0] for s in range(3000)], axis=0)
    # the rescale 1 / (1 - p) makes the expectation the undropped output
    np.testing.assert_allclose(mean, o0, atol=0.06)
    wrong = np.mean([od.forward_head(q, k, v, 0.7, False, 0.4, s, 0, 0)[0] * 0.6 for s in range(3000)], axis=0)
    assert np.abs(wrong - o0).max() > 0.1    # dropping the rescale is caught


def test_queries_sharing_a_call_are_independent():
    """The two queries of a generator row pair use the two 16-bit halves of the
    same words; their keep decisions must still be independent."""
    m = od.keep_mask(4, np.arange(512), np.arange(256), 0.5, 31337, 2)
    even, odd = m[0::2], m[1::2]
    n = even.size
    agree = int((even == odd).sum())
    assert abs(agree - n / 2) <= 5 * np.sqrt(n / 4)
    # and the rate of the quantised threshold: floor(p 2^16) / 2^16 dropped
    p = 0.3
    t = od.drop_threshold(p)
    assert t == int(np.floor(p * 65536)) and 0 <= p * 65536 - t < 1
