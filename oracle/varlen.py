"""Packed variable-length batches with grouped key/value heads (float64).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Sources: page 2 ("FlashAttention 入门"), "padding and shapes" paragraph of its
usage section (variable-length sequences packed without padding through
cumulative sequence offsets; query and key lengths may differ) and its
library-interface paragraph (multi-query / grouped-query attention); page 1,
key designs 1-3 for the operator itself, evaluated per sequence and head by
oracle.attention.

Layout (token-major, the packed form the pages describe):
  q [total_q, Hq, d], k and v [total_k, Hk, d], Hq a multiple of Hk;
  sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
  cu_k[b] .. cu_k[b+1]-1; query head h reads key/value head h // (Hq / Hk).
  O and dQ have q's layout, dK and dV k's; LSE and D are [total_q, Hq].
Readings (the pages are silent):
  * causal attention with n_q != n_k keys places the queries at the last n_q
    key positions: query i sees key j iff j <= i + (n_k - n_q); queries
    with no visible key give O = 0, LSE = -inf.
  * dK and dV of a key/value head sum the contributions of every query head
    that reads it (the chain rule for a shared parameter).
  * with dropout (p > 0; oracle.dropout), the mask of query head h of
    sequence b is that of head bh = b Hq + h at the positions i, j inside
    the sequence.
"""
from __future__ import annotations

import numpy as np

from . import dropout as _dropout
from .attention import backward_head, forward_head


def _spans(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[b]), int(cu[b + 1])) for b in range(cu.size - 1)]


def forward(q, k, v, cu_q, cu_k, scale: float, causal: bool = False, p: float = 0.0, seed: int = 0,
            offset: int = 0):
    """Returns (O [total_q, Hq, d], LSE [total_q, Hq]); p > 0 applies dropout."""
    total_q, hq, d = q.shape
    hk = k.shape[1]
    assert hq % hk == 0
    grp = hq // hk
    o = np.zeros_like(q)
    lse = np.full((total_q, hq), -np.inf)
    for b, ((sq, eq), (sk, ek)) in enumerate(zip(_spans(cu_q), _spans(cu_k))):
        if eq == sq:
            continue
        off = (ek - sk) - (eq - sq)
        for h in range(hq):
            if ek == sk:
                continue                        # no keys: O = 0, LSE = -inf
            args = (q[sq:eq, h], k[sk:ek, h // grp], v[sk:ek, h // grp], scale, causal)
            if p > 0:
                o[sq:eq, h], lse[sq:eq, h] = _dropout.forward_head(*args, p, seed, offset, b * hq + h,
                                                                   diag_offset=off)
            else:
                o[sq:eq, h], lse[sq:eq, h] = forward_head(*args, diag_offset=off)
    return o, lse


def backward(q, k, v, do, cu_q, cu_k, scale: float, causal: bool = False, p: float = 0.0, seed: int = 0,
             offset: int = 0):
    """Returns (dQ, dK, dV, D) with dK, dV summed over the query heads of each group; p > 0
    applies dropout."""
    total_q, hq, d = q.shape
    hk = k.shape[1]
    grp = hq // hk
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.zeros((total_q, hq))
    for bi, ((sq, eq), (sk, ek)) in enumerate(zip(_spans(cu_q), _spans(cu_k))):
        if eq == sq or ek == sk:
            continue
        off = (ek - sk) - (eq - sq)
        for h in range(hq):
            g = h // grp
            args = (q[sq:eq, h], k[sk:ek, g], v[sk:ek, g], do[sq:eq, h], scale, causal)
            if p > 0:
                a, b_, c, e = _dropout.backward_head(*args, p, seed, offset, bi * hq + h, diag_offset=off)
            else:
                a, b_, c, e = backward_head(*args, diag_offset=off)
            dq[sq:eq, h] = a
            dk[sk:ek, g] += b_
            dv[sk:ek, g] += c
            dd[sq:eq, h] = e
    return dq, dk, dv, dd
