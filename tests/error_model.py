"""Element-wise error scales for the gradients (test infrastructure).

The kernels form every gradient element as a sum of products in fp32 whose one
factor was rounded to the 16-bit operand type: dV_jc = sum_i P_ij dO_ic with P
rounded, dK_jc = s sum_i dS_ij Q_ic and dQ_ic = s sum_j dS_ij K_jc with dS
rounded (page 1, key design 3: dV = P^T dO, dS = P o (dP - D), dQ = dS K,
dK = dS^T Q; the scale s enters through S = s Q K^T). Round-to-nearest-even
perturbs each such factor by a relative error of at most u (unit roundoff,
2^-11 for fp16, 2^-8 for bf16), independently from term to term, so the
error of a sum is a random walk whose standard deviation is at most
u * R, with R = sqrt(sum of the squared terms). Per term there are at most
three such relative errors: the rounding of the operand itself, the rounding
of P before dS is formed (d = 128 kernels), and the forward's log-sum-exp
(its row sum adds the rounded probabilities, so LSE is off by at most u in
relative terms, which rescales a whole row of the recomputed P).

Two further sources are not proportional to a term:
  * D_i = dO_i . O_i is formed from the stored 16-bit O, whose error is the
    forward's own rounding: |dO_ik| (|O_ik| + W_ik) u per element with
    W_ik = sqrt(sum_j (P_ij V_jk)^2); summed as a random walk this gives
    |dD_i| ~ u E_i, E_i = sqrt(sum_k dO_ik^2 (O_ik^2 + W_ik^2)). It enters
    dS_ij as -P_ij dD_i: into dQ_ic as s dD_i sum_j P_ij K_jc (the same sign
    for every j) and into dK_jc as s sum_i P_ij dD_i Q_ic (a random walk over
    rows). These are G below.
  * fp16 holds values below 2^-14 with a fixed spacing of 2^-24 (subnormal
    range), so a rounded probability can be off by 2^-25 in absolute terms:
    the floor F = sqrt(sum over kept pairs of the squared other factor).

The bound a test applies to each element is then
    |GPU - oracle| <= C u (R + G) + 2 u |oracle| + C eta F + eps,
with C = 8 (eight standard deviations: a Gaussian tail of 1e-15, against
<= 1e8 compared elements; where one term dominates, its worst case of three
roundings is 3 u R), 2 u |oracle| for the final rounding of the gradient and
the LSE scaling of a dQ row, eta = 2^-25 for fp16 (0 for bf16) and eps a
floor at fp32 accumulation level. A wrong tile, row, sign or index moves an
element by a sizeable fraction of R (a missing 64-key tile out of 1024 keys:
~R/4), far outside this bound.

Dropout: the terms carry the keep mask Z = M / (1 - p): dV uses P o Z,
dP = Z o (dO V^T), and O = (P o Z) V.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence

import numpy as np

from oracle.attention import _probabilities, _scores, kept_pairs

C_SIGMA = 8.0
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
SUBNORMAL_FLOOR = {"f16": 2.0 ** -25, "bf16": 0.0}


@dataclasses.dataclass
class Scales:
    """Per-element error scales of one gradient tensor (same shape as the tensor)."""
    r: np.ndarray      # sqrt(sum of squared terms)
    g: np.ndarray      # propagated error of D (scale of it, divided by u)
    f: np.ndarray      # subnormal floor (scale, divided by eta)

    @staticmethod
    def combine(parts: Sequence["Scales"]) -> "Scales":
        """Scales of a sum of independent gradients (grouped key/value heads)."""
        return Scales(np.sqrt(sum(p.r ** 2 for p in parts)), np.sqrt(sum(p.g ** 2 for p in parts)),
                      np.sqrt(sum(p.f ** 2 for p in parts)))


def gradient_scales_head(q, k, v, do, scale: float, causal: bool = False,
                         block_mask: Optional[np.ndarray] = None, mask_block: int = 128,
                         diag_offset: int = 0, z: Optional[Callable] = None,
                         q_rows: Optional[Sequence[int]] = None, k_cols: Optional[Sequence[int]] = None,
                         first_row: int = 0, row_block: int = 512):
    """Error scales of dQ (at q_rows) and dK, dV (at k_cols) for one head.

    q, do: [N_q, d]; k, v: [N_k, d] float64 inputs. z(rows, cols), when given,
    returns the dropout multiplier block M / (1 - p). `first_row` > 0 drops the
    contributions of rows i < first_row to dK, dV: exact for causal attention
    when every k_col >= first_row + diag_offset (those rows see none of the
    keys). Returns {"dq": Scales, "dk": Scales, "dv": Scales}.
    """
    nq, nk = q.shape[0], k.shape[0]
    q_rows = np.arange(nq) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_cols = np.arange(nk) if k_cols is None else np.asarray(k_cols, dtype=np.int64)
    rows_needed = np.union1d(np.arange(first_row, nq), q_rows)
    want_q = np.zeros(nq, dtype=bool)
    want_q[q_rows] = True
    d = q.shape[1]
    k2, absk = k ** 2, np.abs(k)
    rq2 = np.zeros((nq, d))
    fq2 = np.zeros((nq, d))
    gq = np.zeros((nq, d))
    rv2 = np.zeros((k_cols.size, d))
    fv2 = np.zeros((k_cols.size, d))
    rk2 = np.zeros((k_cols.size, d))
    fk2 = np.zeros((k_cols.size, d))
    gk2 = np.zeros((k_cols.size, d))
    for r0 in range(0, rows_needed.size, row_block):
        rr = rows_needed[r0:r0 + row_block]
        # keys past the last one any row of the block sees contribute exactly zero
        ncol = nk if not causal else int(min(nk, max(rr.max() + diag_offset + 1, 0)))
        cols = np.arange(ncol)
        keep = kept_pairs(rr, cols, causal, block_mask, mask_block, diag_offset)
        p, _ = _probabilities(_scores(q[rr], k[:ncol], scale, keep))
        zz = z(rr, cols) if z is not None else 1.0
        pz = p * zz
        o = pz @ v[:ncol]
        w2 = (pz ** 2) @ (v[:ncol] ** 2)
        drow = (do[rr] * o).sum(axis=1)                       # D_i = dO_i . O_i
        e_d = np.sqrt((do[rr] ** 2 * (o ** 2 + w2)).sum(axis=1))
        sel = want_q[rr]
        if sel.any():
            dp = (do[rr][sel] @ v[:ncol].T) * (zz[sel] if z is not None else 1.0)
            ds = p[sel] * (dp - drow[sel][:, None])
            rq2[rr[sel]] = (ds ** 2) @ k2[:ncol]
            fq2[rr[sel]] = keep[sel].astype(np.float64) @ k2[:ncol]
            gq[rr[sel]] = e_d[sel][:, None] * (p[sel] @ absk[:ncol])
        live = rr >= first_row
        cin = np.nonzero(k_cols < ncol)[0]
        if live.any() and cin.size:
            kc = k_cols[cin]
            xr, dor, pl = q[rr][live], do[rr][live], p[live][:, kc]
            pzl = pz[live][:, kc]
            dpc = (dor @ v[kc].T) * (zz[live][:, kc] if z is not None else 1.0)
            dsc = pl * (dpc - drow[live][:, None])
            kpc = keep[live][:, kc].astype(np.float64)
            rv2[cin] += (pzl ** 2).T @ (dor ** 2)
            fv2[cin] += kpc.T @ (dor ** 2)
            rk2[cin] += (dsc ** 2).T @ (xr ** 2)
            fk2[cin] += kpc.T @ (xr ** 2)
            gk2[cin] += ((pl * e_d[live][:, None]) ** 2).T @ (xr ** 2)
    s = abs(scale)
    return {
        "dq": Scales(s * np.sqrt(rq2[q_rows]), s * gq[q_rows], s * np.sqrt(fq2[q_rows])),
        "dk": Scales(s * np.sqrt(rk2), s * np.sqrt(gk2), s * np.sqrt(fk2)),
        "dv": Scales(np.sqrt(rv2), np.zeros_like(rv2), np.sqrt(fv2)),
    }


def elementwise_bound(ref: np.ndarray, sc: Scales, dtype: str) -> np.ndarray:
    """|GPU - oracle| allowed per element (module docstring)."""
    u, eta = UNIT_ROUNDOFF[dtype], SUBNORMAL_FLOOR[dtype]
    a = np.abs(ref)
    eps = 1e-6 * (float(a.max()) if a.size else 0.0) + 1e-12
    return C_SIGMA * u * (sc.r + sc.g) + 2.0 * u * a + C_SIGMA * eta * sc.f + eps
