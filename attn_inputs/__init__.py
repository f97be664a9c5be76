"""Seeded synthetic inputs for the attention kernels and for the oracle.

This module is the only code that the HIP path and the oracle share. It holds
no attention arithmetic: it draws the random tensors, rounds them to the
16-bit storage formats, and builds the fixed block masks. Both sides consume
the same bits; the oracle upcasts them to float64 (exactly representable), the
device path copies them to HBM unchanged.

Workloads follow the attention shapes the FlashAttention pages talk about:
the GPT-2-medium attention shape of the Fig. 2 ablation (page 1, "核心机制消融"
section: batch 64, 16 heads, length 1024, head dimension 64) plus long-context
causal and fixed butterfly block-sparse variants (page 1, "IO 复杂度" section,
block-sparse IO bound; page 2, FA1 section, "因果掩码几乎免费").
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F16 = "f16"
BF16 = "bf16"
MASK_BLOCK = 128


# ---------------------------------------------------------------------------
# 16-bit rounding (round to nearest, ties to even)
# ---------------------------------------------------------------------------
def round_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16 bit patterns, round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns with round-to-nearest-even.

    bfloat16 keeps the top 16 bits of the binary32 encoding. Adding
    0x7FFF plus the lowest kept bit before truncating rounds halfway cases to
    the even neighbour; overflow past the largest finite value carries into
    the exponent and yields infinity, as IEEE rounding requires. NaNs map to a
    quiet NaN. Every non-NaN pattern is at most 0xFF800000 (-inf), so the sum
    stays within 32 bits.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    nan = np.isnan(f)
    has_nan = bool(nan.any())
    b = f.view(np.uint32)
    if has_nan:
        b = np.where(nan, np.uint32(0), b)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if has_nan:
        r[nan] = np.uint16(0x7FC0)
    return r


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of 16-bit storage patterns to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return round_to_f16_bits(x)
    if dtype == BF16:
        return round_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Block masks
# ---------------------------------------------------------------------------
def butterfly_block_mask(n_tiles: int) -> np.ndarray:
    """uint8 [n_tiles, n_tiles]: tile (i, j) kept iff i == j or i XOR j is a power of two.

    This is the fixed butterfly pattern used for the block-sparse workload
    (page 1 names butterfly sparsity for block-sparse FlashAttention; the
    exact rule over 128x128 tiles is this workload's own choice).
    """
    i = np.arange(n_tiles, dtype=np.int64)[:, None]
    j = np.arange(n_tiles, dtype=np.int64)[None, :]
    x = i ^ j
    keep = (x == 0) | ((x & (x - 1)) == 0)
    return keep.astype(np.uint8)


def random_block_mask(n_tiles: int, density: float, seed: int) -> np.ndarray:
    """Seeded random uint8 tile mask (diagonal always kept) for parity tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = (rng.random((n_tiles, n_tiles)) < density).astype(np.uint8)
    np.fill_diagonal(m, 1)
    return m


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    mask: Optional[str]      # None | "butterfly"
    mult: float              # multiplier applied to the N(0,1) draws before rounding
    seed: int
    backward: bool

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def block_mask(self) -> Optional[np.ndarray]:
        if self.mask is None:
            return None
        if self.mask == "butterfly":
            return butterfly_block_mask(-(-self.N // MASK_BLOCK))
        raise ValueError(self.mask)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_fwd_n256_d64_f16", 1, 1, 256, 64, F16, False, None, 1.0, 1001, False),
        Workload("gpt2_medium_b64_h16_n1024_d64_f16", 64, 16, 1024, 64, F16, False, None, 1.0, 1002, True),
        Workload("causal_b2_h32_n8192_d128_bf16", 2, 32, 8192, 128, BF16, True, None, 0.5, 1003, True),
        Workload("causal_b1_h8_n65536_d128_bf16", 1, 8, 65536, 128, BF16, True, None, 1.0, 1004, True),
        Workload("butterfly_b4_h16_n16384_d64_f16", 4, 16, 16384, 64, F16, False, "butterfly", 1.0, 1005, True),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclasses.dataclass
class Drawn:
    """Bit patterns (uint16, [B,H,N,d]) for q, k, v and optionally do."""
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]

    def f64(self, name: str, b: Optional[int] = None, h: Optional[int] = None) -> np.ndarray:
        """float64 copy of a whole tensor, or of head (b, h) only."""
        x = getattr(self, name)
        if b is not None:
            x = x[b, h]
        return bits_to_f64(x, self.dtype)


def draw(B: int, H: int, N: int, d: int, dtype: str, seed: int,
         mult: float = 1.0, with_do: bool = True) -> Drawn:
    """Draw q, k, v (and do) i.i.d. N(0,1) in fp32 from PCG64(seed), in that order,
    multiply by `mult`, round to `dtype` with round-to-nearest-even."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(4 if with_do else 3):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out.append(round_bits(x, dtype))
    return Drawn(dtype, out[0], out[1], out[2], out[3] if with_do else None)


def draw_ramped_keys(B: int, H: int, N: int, d: int, dtype: str, seed: int, lo: float, hi: float,
                     q_mult: float = 1.0) -> Drawn:
    """Like draw(), but key row j is multiplied by lo + (hi - lo) j / (N - 1) (and q by
    q_mult) before rounding, so that scores grow along the key axis: each query row's
    running maximum keeps rising as later key tiles arrive."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    ramp = (lo + (hi - lo) * np.arange(N, dtype=np.float32) / np.float32(max(N - 1, 1))).astype(np.float32)
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(q_mult)
    k = rng.standard_normal(shape, dtype=np.float32) * ramp[None, None, :, None]
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32)
    return Drawn(dtype, *(round_bits(x, dtype) for x in (q, k, v, do)))


def draw_workload(w: Workload, with_do: Optional[bool] = None) -> Drawn:
    if with_do is None:
        with_do = w.backward
    return draw(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.mult, with_do)



# ---------------------------------------------------------------------------
# Packed variable-length batches (token-major [total, heads, d])
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PackedDrawn:
    """16-bit bit patterns of packed q [total_q, Hq, d], k and v [total_k, Hk, d],
    do [total_q, Hq, d], and the cumulative offsets (int32, batch + 1)."""
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        return bits_to_f64(getattr(self, name), self.dtype)


def cumulative(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def draw_packed(lengths_q, lengths_k, hq: int, hk: int, d: int, dtype: str, seed: int,
                mult: float = 1.0) -> PackedDrawn:
    """Draw packed q, k, v, do i.i.d. N(0,1) in fp32 from PCG64(seed), in that
    order, multiply by `mult` and round to `dtype` (round-to-nearest-even)."""
    cu_q, cu_k = cumulative(lengths_q), cumulative(lengths_k)
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = [(int(cu_q[-1]), hq, d), (int(cu_k[-1]), hk, d), (int(cu_k[-1]), hk, d), (int(cu_q[-1]), hq, d)]
    out = []
    for shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out.append(round_bits(x, dtype))
    return PackedDrawn(dtype, out[0], out[1], out[2], out[3], cu_q, cu_k)


def length_mix(batch: int, max_len: int, seed: int, min_len: int = 1) -> np.ndarray:
    """Sequence lengths for a packed batch: uniform in [min_len, max_len] from
    PCG64(seed), with the first entry pinned to max_len so the maximum is hit."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(min_len, max_len + 1, size=batch)
    lens[0] = max_len
    return lens.astype(np.int64)


@dataclasses.dataclass(frozen=True)
class PackedWorkload:
    """A packed variable-length batch used to measure the grouped-head and
    split-KV paths (synthetic: the pages fix no such workload).
    decode: one query per sequence against a key/value cache of length
    U[max_k/2, max_k]; otherwise query and key lengths are equal, U[max_q/8, max_q]."""
    name: str
    batch: int
    hq: int
    hk: int
    d: int
    dtype: str
    causal: bool
    max_q: int
    max_k: int
    decode: bool
    seed: int
    n_splits: int = 1
    backward: bool = True

    def lengths(self):
        if self.decode:
            return np.ones(self.batch, dtype=np.int64), length_mix(self.batch, self.max_k, self.seed, self.max_k // 2)
        lens = length_mix(self.batch, self.max_q, self.seed, self.max_q // 8)
        return lens, lens.copy()


PACKED_WORKLOADS = {w.name: w for w in [
    PackedWorkload("varlen_gqa_b16_hq32_hk8_max4096_d128_bf16", 16, 32, 8, 128, BF16, True, 4096, 4096, False, 2001),
    PackedWorkload("decode_splitkv_b32_hq32_hk8_k16384_d128_bf16", 32, 32, 8, 128, BF16, True, 1, 16384, True, 2002,
                   n_splits=8, backward=False),
]}
