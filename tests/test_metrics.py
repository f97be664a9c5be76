"""Host-side work/traffic models: pinned to the pages' memory arithmetic and to
brute-force pair counts."""
import numpy as np
import pytest

import attn_inputs as ai
from exact_io_aware_04_amd import metrics


def test_score_and_probability_memory_matches_page_2():
    # Page 2, "注意力为什么是平方复杂度": N = 8192, fp16 S and P of one head ~ 268 MB,
    # 32 heads ~ 8.6 GB; N = 64K: ~17 GB per head, ~550 GB for 32 heads.
    one = metrics.score_and_prob_bytes_per_head(8192)
    assert one == 268_435_456 and round(one / 1e6) == 268
    assert round(32 * one / 1e9, 1) == 8.6
    big = metrics.score_and_prob_bytes_per_head(65536)
    assert round(big / 1e9) == 17 and round(32 * big / 1e9, -1) == 550


def _brute_pairs(n, causal, mask, bs):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    keep = np.ones((n, n), dtype=bool)
    if causal:
        keep &= j <= i
    if mask is not None:
        keep &= (np.asarray(mask) != 0)[i // bs, j // bs]
    return int(keep.sum())


@pytest.mark.parametrize("n", [1, 100, 128, 129, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_pair_count_matches_brute_force(n, causal, masked):
    mask = ai.random_block_mask(-(-n // 128), 0.5, n) if masked else None
    assert metrics.kept_pairs_per_head(n, causal, mask) == _brute_pairs(n, causal, mask, 128)


def test_workload_flops():
    w = ai.WORKLOADS
    c2 = w["gpt2_medium_b64_h16_n1024_d64_f16"]
    f, b = metrics.flops(c2.B, c2.H, metrics.kept_pairs_per_head(c2.N, c2.causal, c2.block_mask()), c2.d)
    assert f == 274_877_906_944 and b == 687_194_767_360
    c4 = w["causal_b1_h8_n65536_d128_bf16"]
    p = metrics.kept_pairs_per_head(c4.N, True, None)
    assert p == 65536 * 65537 // 2
    c5 = w["butterfly_b4_h16_n16384_d64_f16"]
    assert metrics.kept_pairs_per_head(c5.N, False, c5.block_mask()) == 1024 * 128 * 128


def test_byte_models():
    fwd, bwd = metrics.algorithmic_bytes(64, 16, 1024, 64)
    assert fwd == 4 * 2 ** 26 * 2 + 4 * 2 ** 20
    std_fwd, std_all = metrics.standard_attention_bytes(64, 16, 1024)
    assert round(std_fwd / 1e9, 2) == 8.59 and round(std_all / 1e9, 1) == 23.6


def test_varlen_pair_count_matches_oracle_visibility():
    import oracle
    from exact_io_aware_04_amd import metrics
    lq, lk = [1, 5, 9, 0, 7], [6, 5, 3, 4, 0]
    for causal in (False, True):
        brute = sum(int(oracle.kept_pairs(np.arange(a), np.arange(b), causal, None, 128, b - a).sum())
                    for a, b in zip(lq, lk))
        assert metrics.kept_pairs_varlen(lq, lk, causal) == brute
    assert metrics.kept_pairs_varlen([1], [4096], True) == 4096      # decode: one query sees every key


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_pairs_of_selected_rows_match_brute_force(causal, masked):
    n, bs = 300, 128
    mask = ai.random_block_mask(3, 0.5, 9) if masked else None
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    keep = np.ones((n, n), dtype=bool)
    if causal:
        keep &= j <= i
    if mask is not None:
        keep &= (np.asarray(mask) != 0)[i // bs, j // bs]
    rows = np.array([0, 1, 127, 128, 200, 299])
    assert metrics.kept_pairs_rows(rows, n, causal, mask, bs) == int(keep[rows].sum())
    assert metrics.kept_pairs_rows(np.arange(n), n, causal, mask, bs) == metrics.kept_pairs_per_head(n, causal, mask, bs)
