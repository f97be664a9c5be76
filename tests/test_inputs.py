"""The seeded input module: 16-bit rounding, determinism, workload table."""
import numpy as np
import pytest
import torch

import attn_inputs as ai


def test_bf16_rounding_matches_torch_and_ties_to_even():
    rng = np.random.Generator(np.random.PCG64(3))
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        rng.standard_normal(1000).astype(np.float32) * 1e-39,        # subnormals
        np.array([3.4e38, -3.4e38, 0.0, -0.0, 1e-45], dtype=np.float32),
    ])
    ours = ai.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # Exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6).
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=np.float32)
    got = ai.bits_to_f64(ai.round_to_bf16_bits(ties), ai.BF16)
    np.testing.assert_array_equal(got, [1.0, 1 + 2 ** -6])
    # Overflow rounds to infinity.
    big = np.array([np.float32(3.4028235e38)], dtype=np.float32)
    assert np.isinf(ai.bits_to_f64(ai.round_to_bf16_bits(big), ai.BF16)[0])


def test_f16_rounding_matches_torch():
    x = np.random.Generator(np.random.PCG64(4)).standard_normal(100000).astype(np.float32) * 100
    ours = ai.round_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("dtype", [ai.F16, ai.BF16])
def test_upcast_is_exact(dtype):
    x = np.random.Generator(np.random.PCG64(5)).standard_normal(4096).astype(np.float32)
    bits = ai.round_bits(x, dtype)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.float16 if dtype == ai.F16 else torch.bfloat16)
    np.testing.assert_array_equal(ai.bits_to_f64(bits, dtype), t.double().numpy())


def test_draws_are_seeded_and_ordered():
    a = ai.draw(1, 2, 16, 8, ai.F16, 99)
    b = ai.draw(1, 2, 16, 8, ai.F16, 99)
    for n in "qkv":
        np.testing.assert_array_equal(getattr(a, n), getattr(b, n))
    # q, k, v, do are consecutive draws from one PCG64 stream.
    rng = np.random.Generator(np.random.PCG64(99))
    q = rng.standard_normal((1, 2, 16, 8), dtype=np.float32)
    k = rng.standard_normal((1, 2, 16, 8), dtype=np.float32)
    np.testing.assert_array_equal(a.k, ai.round_to_f16_bits(k))
    np.testing.assert_array_equal(a.q, ai.round_to_f16_bits(q))
    c = ai.draw(1, 1, 4, 4, ai.BF16, 7, mult=0.5)
    rng = np.random.Generator(np.random.PCG64(7))
    q = rng.standard_normal((1, 1, 4, 4), dtype=np.float32) * np.float32(0.5)
    np.testing.assert_array_equal(c.q, ai.round_to_bf16_bits(q))


def test_workload_table():
    w = ai.WORKLOADS
    assert len(w) == 5
    c3 = w["causal_b2_h32_n8192_d128_bf16"]
    assert (c3.B, c3.H, c3.N, c3.d, c3.dtype, c3.causal, c3.mult) == (2, 32, 8192, 128, ai.BF16, True, 0.5)
    c5 = w["butterfly_b4_h16_n16384_d64_f16"]
    assert c5.block_mask().shape == (128, 128) and c5.block_mask().sum() == 1024
    assert w["single_head_fwd_n256_d64_f16"].scale == 0.125


def test_ramped_keys_are_seeded_and_rise():
    a = ai.draw_ramped_keys(1, 2, 300, 64, ai.F16, 5, lo=0.2, hi=12.0, q_mult=2.0)
    b = ai.draw_ramped_keys(1, 2, 300, 64, ai.F16, 5, lo=0.2, hi=12.0, q_mult=2.0)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(getattr(a, n), getattr(b, n))
        assert getattr(a, n).shape == (1, 2, 300, 64) and getattr(a, n).dtype == np.uint16
    k = np.abs(a.f64("k", 0, 1))
    assert k[-10:].mean() > 20 * k[:10].mean()        # key rows scaled from 0.2 up to 12
    assert 1.5 < np.abs(a.f64("q")).std() / 0.8 < 3.0  # q scaled by 2 (|N(0,1)| has sd ~0.6)
