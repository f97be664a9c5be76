"""Plain float64 attention: forward (O, LSE) and analytic backward (dQ, dK, dV, D).

Sources (the pages named by their titles):
  * Page 1, "FlashAttention：不减少一次注意力计算，为什么反而更快", key design 1:
    the operator S = QK^T/sqrt(d), P = softmax(S) by rows, O = PV.
  * Page 1, key design 2 (table of saved state): the saved row statistic
    L = m + log(l) (the log-sum-exp) that lets the backward rebuild P.
  * Page 1, key design 3 (the D_i identity and dS formula):
    D_i = P_i:^T dP_i: = dO_i^T O_i, dS_ij = P_ij (dP_ij - D_i),
    dV = P^T dO, dQ = dS K, dK = dS^T Q.
  * Page 2 ("FlashAttention 入门"), FA1 section: causal attention skips or
    masks keys j > i; page 1, IO section: block-sparse variant skips zero
    blocks and is exact within the kept ones.

Readings where the pages are silent or inconsistent (each is listed in the
design notes with its justification):
  * The softmax scale s is part of S, so by the chain rule dQ = s dS K and
    dK = s dS^T Q (the pages' pseudocode drops s; finite differences pin it).
  * dS keeps the -D_i term (page 2's backward display omits it; that form
    fails the finite-difference pin, see the mutation test).
  * A masked pair has score -inf before the softmax, so each row normalises
    over its kept keys only; a row with no kept key has O = 0, LSE = -inf and
    contributes nothing to any gradient.
  * LSE is the natural log of the sum of exp of the *scaled* scores.

All arrays are float64. One head is [N, d]; the batched helpers take
[B, H, N, d] and loop over heads. Packed variable-length batches with grouped
key/value heads are in oracle/varlen.py.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# Which (query, key) pairs take part
# ---------------------------------------------------------------------------
def kept_pairs(rows: np.ndarray, cols: np.ndarray, causal: bool,
               block_mask: Optional[np.ndarray], mask_block: int,
               diag_offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: True where key `col` is visible to query `row`.

    causal: key j is visible to query i iff j <= i + diag_offset. For square
    self-attention diag_offset = 0; for n_q queries against n_k keys the
    queries are read as the last n_q positions of the key sequence
    (diag_offset = n_k - n_q, a reading: the pages only note that one backend
    refuses causal attention with unequal lengths).
    block_mask: tile (i // mask_block, j // mask_block) must be nonzero.
    Both conditions combine with a logical AND.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    keep = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        keep &= cols[None, :] <= rows[:, None] + diag_offset
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        keep &= bm[(rows // mask_block)[:, None], (cols // mask_block)[None, :]]
    return keep


def _scores(q_rows, k, scale, keep):
    """S = scale * q k^T with -inf at masked pairs."""
    s = scale * (q_rows @ k.T)
    return np.where(keep, s, -np.inf)


def _probabilities(s):
    """Row softmax of S (with -inf entries) and the row log-sum-exp.

    m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i), LSE_i = m_i + ln l_i,
    P_ij = exp(S_ij - LSE_i). Rows with no finite score give P = 0, LSE = -inf.
    """
    m = s.max(axis=1)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[:, None])            # exp(-inf) = 0 at masked pairs
    ell = e.sum(axis=1)
    lse = np.where(live, m_safe + np.log(np.where(live, ell, 1.0)), -np.inf)
    lse_safe = np.where(live, lse, 0.0)
    p = np.where(live[:, None], np.exp(s - lse_safe[:, None]), 0.0)
    return p, lse


# ---------------------------------------------------------------------------
# One head
# ---------------------------------------------------------------------------
def forward_head(q, k, v, scale: float, causal: bool = False,
                 block_mask: Optional[np.ndarray] = None, mask_block: int = 128,
                 rows: Optional[Sequence[int]] = None, row_block: int = 1024,
                 diag_offset: int = 0):
    """O = softmax(scale * q k^T) v and LSE for one head (or for selected rows).

    q: [N_q, d], k, v: [N_k, d] float64. Returns (O [R, d], LSE [R]) for the R
    requested query rows (all rows by default). The score rows are
    materialised `row_block` at a time only to bound host memory.
    diag_offset: see kept_pairs (causal alignment for N_q != N_k).
    """
    n = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(n)
    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for r0 in range(0, rows.size, row_block):
        rr = rows[r0:r0 + row_block]
        keep = kept_pairs(rr, cols, causal, block_mask, mask_block, diag_offset)
        p, lse[r0:r0 + rr.size] = _probabilities(_scores(q[rr], k, scale, keep))
        o[r0:r0 + rr.size] = p @ v
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool = False,
                  block_mask: Optional[np.ndarray] = None, mask_block: int = 128,
                  row_block: int = 1024, diag_offset: int = 0,
                  rows: Optional[Sequence[int]] = None):
    """Analytic gradients of O = softmax(scale q k^T) v for one head.

    With P the probabilities and dO the incoming gradient:
      dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij, dS = P o (dP - D),
      dQ = scale dS K, dK = scale dS^T Q.
    Returns (dQ, dK, dV, D) in float64; D is computed from its definition as
    the row sum of P o dP (its equality with rowsum(dO o O) is a pin).
    `rows` restricts the sums to those query rows: dQ and D are then filled
    at those rows only (zero elsewhere) and dK, dV hold those rows'
    contributions (every row's contribution is a separate term of the sums).
    """
    n = k.shape[0]
    cols = np.arange(n)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.zeros(q.shape[0], dtype=np.float64)
    all_rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    for r0 in range(0, all_rows.size, row_block):
        rr = all_rows[r0:r0 + row_block]
        keep = kept_pairs(rr, cols, causal, block_mask, mask_block, diag_offset)
        p, _ = _probabilities(_scores(q[rr], k, scale, keep))
        dv += p.T @ do[rr]
        dp = do[rr] @ v.T
        drow = (p * dp).sum(axis=1)
        ds = p * (dp - drow[:, None])
        dq[rr] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rr])
        dd[rr] = drow
    return dq, dk, dv, dd


def backward_head_sampled(q, k, v, do, scale: float, causal: bool,
                          block_mask: Optional[np.ndarray], mask_block: int,
                          q_rows: Sequence[int], k_rows: Sequence[int],
                          first_row: int = 0, row_block: int = 1024):
    """Gradients at selected indices for a head too large to differentiate whole.

    dQ at a query row needs only that row of P plus D_i = sum_k dO_ik O_ik
    (equal to sum_j P_ij dP_ij, the D identity), all computable from that row:
      dQ_i = scale sum_j P_ij (dP_ij - D_i) K_j
    dK, dV at a key column j need that column of P, hence LSE_i and D_i of
    every query row that sees key j:
      dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i P_ij (dP_ij - D_i) Q_i
    `first_row` > 0 restricts those rows to i >= first_row; that is exact
    only for causal attention with every sampled key index >= first_row
    (P_ij = 0 for i < j), which is asserted.
    Returns (dQ[q_rows], dK[k_rows], dV[k_rows], D[q_rows]).
    """
    n = k.shape[0]
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    if first_row > 0:
        assert causal and k_rows.size and k_rows.min() >= first_row
    all_idx = np.arange(n)

    o_q, lse_q = forward_head(q, k, v, scale, causal, block_mask, mask_block, rows=q_rows,
                              row_block=row_block)
    dd_q = (do[q_rows] * o_q).sum(axis=1)
    live_q = np.isfinite(lse_q)
    keep = kept_pairs(q_rows, all_idx, causal, block_mask, mask_block)
    s = _scores(q[q_rows], k, scale, keep)
    p = np.where(live_q[:, None], np.exp(s - np.where(live_q, lse_q, 0.0)[:, None]), 0.0)
    dp = do[q_rows] @ v.T
    dq = scale * ((p * (dp - dd_q[:, None])) @ k)

    rows = np.arange(first_row, n)
    o_r, lse_r = forward_head(q, k, v, scale, causal, block_mask, mask_block, rows=rows,
                              row_block=row_block)
    dd_r = (do[rows] * o_r).sum(axis=1)
    live_r = np.isfinite(lse_r)
    keep_t = kept_pairs(rows, k_rows, causal, block_mask, mask_block)       # [R, K]
    s_t = np.where(keep_t, scale * (q[rows] @ k[k_rows].T), -np.inf)
    p_t = np.where(live_r[:, None], np.exp(s_t - np.where(live_r, lse_r, 0.0)[:, None]), 0.0)
    dp_t = do[rows] @ v[k_rows].T
    dv = p_t.T @ do[rows]
    dk = scale * ((p_t * (dp_t - dd_r[:, None])).T @ q[rows])
    return dq, dk, dv, dd_q


# ---------------------------------------------------------------------------
# Batched [B, H, N, d]
# ---------------------------------------------------------------------------
def forward(q, k, v, scale, causal=False, block_mask=None, mask_block=128):
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal,
                                              block_mask, mask_block)
    return o, lse


def backward(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128):
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dd = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], dd[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, block_mask, mask_block)
    return dq, dk, dv, dd


# ---------------------------------------------------------------------------
# Mergeable softmax state (used only by the merge pin)
# ---------------------------------------------------------------------------
def softmax_block_state(scores: np.ndarray, values: np.ndarray):
    """State of one block of a score row, as on page 3 ("Online Softmax 的具体例子"):
    m = max s, l = sum exp(s - m), O~ = sum exp(s - m) v. scores [R, c], values [c, d]."""
    m = scores.max(axis=1)
    e = np.exp(scores - m[:, None])
    return m, e.sum(axis=1), e @ values


def merge_softmax_blocks(state_a, state_b):
    """Merge two block states (page 1, key design 2 merge equations; page 3 forward
    process): m = max(m_a, m_b); l = e^{m_a-m} l_a + e^{m_b-m} l_b;
    O~ = e^{m_a-m} O~_a + e^{m_b-m} O~_b. The normalised output is O~ / l."""
    ma, la, oa = state_a
    mb, lb, ob = state_b
    m = np.maximum(ma, mb)
    ca = np.exp(ma - m)
    cb = np.exp(mb - m)
    return m, ca * la + cb * lb, ca[:, None] * oa + cb[:, None] * ob


def merge_normalised(o_parts, lse_parts):
    """Merge softmax results computed over disjoint key subsets, given as
    normalised outputs O_s and log-sum-exps LSE_s (the state page 2's FA2
    section saves, L = m + log l, in place of (m, l)): by page 1, key design 2,
    with l_s = exp(LSE_s - m) up to the common factor e^m,
      LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
    Subsets with no visible key have LSE_s = -inf and weight 0; a row with no
    visible key at all gets O = 0, LSE = -inf. o_parts [S, R, d], lse_parts [S, R]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None, :]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(live, m_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    o = np.where(live[:, None], (w[:, :, None] * o_parts).sum(axis=0) / np.where(live, tot, 1.0)[:, None], 0.0)
    return o, lse
