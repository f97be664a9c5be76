"""Work and traffic models used to report throughput and roofline fractions.

FLOP convention: a kept (query, key) pair costs 4 d FLOPs in the forward
(S = Q K^T and O = P V, one multiply-add each per element of d) and 10 d in
the backward (S recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K,
dK = dS^T Q). Masked pairs inside partially kept tiles are not counted.

Byte models (e = bytes per element):
  * algorithmic minimum, forward: read Q, K, V, write O (4 BHNd e) and LSE (4 BHN);
  * algorithmic minimum, backward incl. the D preprocess: read Q, K, V, dO, O
    (for D) and write dQ, dK, dV (9 BHNd e), plus LSE read, D write and read (12 BHN);
  * standard attention (the materialising baseline the pages compare against,
    page 1 IO section and page 2 "GPU 内存层级与 IO 感知"): the forward writes S,
    reads S, writes P, reads P (4 BHN^2 e); the backward reads P, writes and
    reads dP, writes dS and reads it twice (7 BHN^2 e).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

MI355X_PEAK_DENSE_F16_TFLOPS = 2500.0     # published dense fp16/bf16 MFMA peak
MI355X_HBM_GBPS = 8000.0                  # published HBM3E bandwidth


def kept_pairs_per_head(N: int, causal: bool, block_mask: Optional[np.ndarray], mask_block: int = 128) -> int:
    """Number of (query, key) pairs a head computes, counted exactly (64-bit)."""
    T = -(-N // mask_block)
    keep_tile = np.ones((T, T), dtype=bool) if block_mask is None else (np.asarray(block_mask) != 0)
    total = 0
    for ti in range(T):
        r0, r1 = ti * mask_block, min(N, (ti + 1) * mask_block)
        rows = np.arange(r0, r1, dtype=np.int64)
        for tj in np.nonzero(keep_tile[ti])[0]:
            c0, c1 = int(tj) * mask_block, min(N, (int(tj) + 1) * mask_block)
            if not causal:
                total += (r1 - r0) * (c1 - c0)
            else:
                total += int(np.clip(rows - c0 + 1, 0, c1 - c0).sum())
    return int(total)


def kept_pairs_rows(rows, N: int, causal: bool, block_mask: Optional[np.ndarray], mask_block: int = 128) -> int:
    """Kept (query, key) pairs of the given query rows of one head (N keys)."""
    rows = np.asarray(rows, dtype=np.int64)
    if block_mask is None:
        per = np.minimum(rows + 1, N) if causal else np.full(rows.shape, N, dtype=np.int64)
        return int(per.sum())
    keep_tile = np.asarray(block_mask) != 0
    total = 0
    for i in rows:
        for tj in np.nonzero(keep_tile[int(i) // mask_block])[0]:
            c0, c1 = int(tj) * mask_block, min(N, (int(tj) + 1) * mask_block)
            total += max(0, min(c1, int(i) + 1) - c0) if causal else c1 - c0
    return int(total)


def flops(B: int, H: int, pairs_per_head: int, d: int):
    """(forward, backward) algorithmic FLOPs for the whole batch."""
    pairs = B * H * pairs_per_head
    return 4 * d * pairs, 10 * d * pairs


def algorithmic_bytes(B: int, H: int, N: int, d: int, e: int = 2):
    """(forward, backward incl. preprocess) minimum HBM bytes."""
    bhn = B * H * N
    return 4 * bhn * d * e + 4 * bhn, 9 * bhn * d * e + 12 * bhn


def standard_attention_bytes(B: int, H: int, N: int, e: int = 2):
    """(forward, forward + backward) quadratic HBM bytes of materialising attention."""
    sq = B * H * N * N * e
    return 4 * sq, 11 * sq


def score_and_prob_bytes_per_head(N: int, e: int = 2) -> int:
    """Bytes to hold S and P of one head in HBM (page 2's memory example)."""
    return 2 * N * N * e


# ---------------------------------------------------------------------------
# Packed variable-length batches (grouped key/value heads)
# ---------------------------------------------------------------------------
def kept_pairs_varlen(lengths_q, lengths_k, causal: bool) -> int:
    """Kept (query, key) pairs per query head summed over the sequences. Causal
    with n_q queries and n_k keys: query i sees min(n_k, max(0, i + n_k - n_q + 1))
    keys (the queries are the last n_q key positions)."""
    total = 0
    for nq, nk in zip(lengths_q, lengths_k):
        nq, nk = int(nq), int(nk)
        if not causal:
            total += nq * nk
        else:
            i = np.arange(nq, dtype=np.int64)
            total += int(np.clip(i + (nk - nq) + 1, 0, nk).sum())
    return int(total)


def packed_bytes(total_q: int, total_k: int, hq: int, hk: int, d: int, e: int = 2):
    """(forward, backward incl. preprocess) minimum HBM bytes of a packed batch:
    forward reads Q, K, V and writes O, LSE; backward reads Q, K, V, dO, O, LSE
    and writes dQ, dK, dV, D (and reads D)."""
    q_b, kv_b, st = total_q * hq * d * e, total_k * hk * d * e, total_q * hq * 4
    return 2 * q_b + 2 * kv_b + st, 4 * q_b + 4 * kv_b + 3 * st
