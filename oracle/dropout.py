"""Attention with dropout on the probabilities, mask regenerated from a
counter-based generator (float64 attention, uint32 generator).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Sources: page 1 ("FlashAttention：不减少一次注意力计算，为什么反而更快"), the table of
key design 2 (dropout: the forward keeps the generator state, not the mask;
the backward regenerates it) and key design 3 (the saved state includes the
generator state); its discussion of reproducibility (the regenerated mask must
match the forward's). The operator with dropout rate p and keep mask M:
  O = (P o Z) V,  Z = M / (1 - p),  P = softmax(s Q K^T) (LSE unchanged),
and by the chain rule
  dV = (P o Z)^T dO,  dP = Z o (dO V^T),  D_i = sum_j P_ij dP_ij = dO_i . O_i,
  dS = P o (dP - D),  dQ = s dS K,  dK = s dS^T Q.

Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011): a 128-bit counter (c0..c3) and a
64-bit key (k0, k1) pass through 10 rounds of
  (hi0, lo0) = 0xD2511F53 * c0,  (hi1, lo1) = 0xCD9E8D57 * c2  (32 x 32 -> 64 bits),
  (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0),
with the key advanced by (0x9E3779B9, 0xBB67AE85) between rounds.
Reading (the pages fix no layout): one generator call decides a block of
2 queries x 4 keys. Element (head bh, query i, key j) uses the 16-bit half
i mod 2 (0 = low) of word j mod 4 of Philox(counter = (j div 4, i div 2, bh,
offset), key = (seed mod 2^32, seed div 2^32)); it is dropped iff that half
< floor(p 2^16) (integer comparison, so the decision is exact on both sides).
The kept fraction is 1 - floor(p 2^16) / 2^16, within 2^-16 of 1 - p; the
rescale stays 1 / (1 - p) as the method states. For a packed batch,
bh = b H + h and i, j are positions inside sequence b.
The generator is pinned to rocRAND's own Philox4x32-10 (its header
implementation, run on the host) at random counters and keys, and
statistically (keep rate, uniformity, counter and key sensitivity); the GPU
must match this implementation bit for bit.
"""
from __future__ import annotations

import numpy as np

from .attention import _probabilities, _scores, kept_pairs

M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
W0, W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10; all inputs broadcastable uint32 values.
    Returns four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    for r in range(10):
        if r > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return [x.astype(np.uint32) for x in c]


def drop_threshold(p: float) -> int:
    """floor(p 2^16), the integer below which a 16-bit draw means 'dropped'."""
    assert 0.0 <= p < 1.0
    return min(int(np.floor(p * 65536.0)), 0xFFFF)


def keep_mask(bh: int, rows, cols, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: True where element (bh, i, j) is kept."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    t = np.uint32(drop_threshold(p))
    i = rows[:, None]
    j = cols[None, :]
    words = philox4x32_10(j >> 2, i >> 1, np.int64(bh), np.int64(offset), seed & 0xFFFFFFFF,
                          (seed >> 32) & 0xFFFFFFFF)
    w = np.choose((j & 3) + np.zeros_like(i), words)
    half = (w >> (np.uint32(16) * (i & 1).astype(np.uint32))) & np.uint32(0xFFFF)
    return half >= t


def forward_head(q, k, v, scale, causal, p, seed, offset, bh, block_mask=None, mask_block=128, diag_offset=0):
    """(O, LSE) of one head with dropout; LSE is that of the scores (dropout acts after the softmax)."""
    rows, cols = np.arange(q.shape[0]), np.arange(k.shape[0])
    keep = kept_pairs(rows, cols, causal, block_mask, mask_block, diag_offset)
    prob, lse = _probabilities(_scores(q, k, scale, keep))
    z = keep_mask(bh, rows, cols, p, seed, offset) / (1.0 - p)
    return (prob * z) @ v, lse


def backward_head(q, k, v, do, scale, causal, p, seed, offset, bh, block_mask=None, mask_block=128, diag_offset=0):
    """(dQ, dK, dV, D) of one head with dropout, from the formulas in the module docstring."""
    rows, cols = np.arange(q.shape[0]), np.arange(k.shape[0])
    keep = kept_pairs(rows, cols, causal, block_mask, mask_block, diag_offset)
    prob, _ = _probabilities(_scores(q, k, scale, keep))
    z = keep_mask(bh, rows, cols, p, seed, offset) / (1.0 - p)
    dv = (prob * z).T @ do
    dp = z * (do @ v.T)
    dd = (prob * dp).sum(axis=1)
    ds = prob * (dp - dd[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv, dd


def forward(q, k, v, scale, causal, p, seed, offset=0, block_mask=None, mask_block=128):
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal, p, seed, offset, b * H + h,
                                              block_mask, mask_block)
    return o, lse


def backward(q, k, v, do, scale, causal, p, seed, offset=0, block_mask=None, mask_block=128):
    B, H, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dd = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], dd[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, p, seed, offset, b * H + h, block_mask, mask_block)
    return dq, dk, dv, dd
