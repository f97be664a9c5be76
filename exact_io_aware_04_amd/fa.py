"""Python binding of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: every step of the attention computation runs in the
HIP kernels behind the C entry points. PyTorch provides device memory and the
stream. There is no fallback: if the shared library is missing or fails to
load, importing this module raises.

The low-level functions keep the C names (`fa_fwd`, `fa_bwd_preprocess`,
`fa_bwd`, `fa_fwd_varlen`, `fa_bwd_varlen`, their `_dropout` forms,
`fa_fwd_splitkv`, `fa_status_string`, ...) and take
integer device addresses. `forward` / `backward` (dense [B, H, N, d]) and
`forward_varlen` / `backward_varlen` (packed token-major, grouped heads) are
thin conveniences over torch tensors that allocate the outputs and call the
same entry points.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_F16 = 0
FA_BF16 = 1
FA_OK = 0
STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_DTYPE", -4: "FA_ERR_HEADDIM",
    -5: "FA_ERR_MASK", -6: "FA_ERR_ALIGN", -7: "FA_ERR_HIP", -8: "FA_ERR_SCALE", -9: "FA_ERR_DROPOUT",
    -10: "FA_ERR_SCRATCH",
}
EXPORTED = ("fa_fwd", "fa_bwd_preprocess", "fa_bwd", "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_varlen",
            "fa_bwd_varlen", "fa_fwd_varlen_dropout", "fa_bwd_varlen_dropout", "fa_fwd_splitkv",
            "fa_fwd_splitkv_noalloc", "fa_status_string")
FA_MAX_SPLITS = 256
FA_NOALLOC_SCRATCH_BYTES = 32 << 20


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime with the same SONAME as the system one.
    # Importing torch first makes libfa.so bind to that already-loaded
    # runtime; loading libfa.so first would map a second HIP/HSA runtime into
    # the process, and the two then fight over the device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
            "or python exact_io_aware_04_amd/build.py). There is no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp]
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.fa_fwd_dropout.restype = i
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, f, u64, u32, vp]
    lib.fa_bwd_dropout.restype = i
    lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, f, u64, u32, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_varlen_dropout.restype = i
    lib.fa_fwd_varlen_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, f, u64, u32, vp]
    lib.fa_bwd_varlen_dropout.restype = i
    lib.fa_bwd_varlen_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i,
                                          f, u64, u32, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp, vp, vp]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i]
    return lib


_lib = _load()


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fa_status_string(status)} ({status})")
        self.status = status


# ---------------------------------------------------------------------------
# C entry points (same names and argument order as include/fa.h)
# ---------------------------------------------------------------------------
def fa_fwd(q, k, v, o, lse, B, H, N, d, dt, scale, causal, block_mask, mask_block, stream) -> int:
    return _lib.fa_fwd(q, k, v, o, lse, B, H, N, d, dt, scale, causal, block_mask, mask_block, stream)


def fa_bwd_preprocess(o, dO, D, B, H, N, d, dt, stream) -> int:
    return _lib.fa_bwd_preprocess(o, dO, D, B, H, N, d, dt, stream)


def fa_bwd(q, k, v, dO, lse, D, dq, dk, dv, B, H, N, d, dt, scale, causal, block_mask, mask_block,
           stream) -> int:
    return _lib.fa_bwd(q, k, v, dO, lse, D, dq, dk, dv, B, H, N, d, dt, scale, causal, block_mask,
                       mask_block, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, dt, scale, causal, block_mask, mask_block, p_drop, seed, offset,
                   stream) -> int:
    return _lib.fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, dt, scale, causal, block_mask, mask_block, p_drop, seed,
                               offset, stream)


def fa_bwd_dropout(q, k, v, dO, lse, D, dq, dk, dv, B, H, N, d, dt, scale, causal, block_mask, mask_block, p_drop,
                   seed, offset, stream) -> int:
    return _lib.fa_bwd_dropout(q, k, v, dO, lse, D, dq, dk, dv, B, H, N, d, dt, scale, causal, block_mask,
                               mask_block, p_drop, seed, offset, stream)


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk, d, dt,
                  scale, causal, stream) -> int:
    return _lib.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk, d,
                              dt, scale, causal, stream)


def fa_bwd_varlen(q, k, v, dO, lse, D, dq, dk, dv, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk,
                  d, dt, scale, causal, stream) -> int:
    return _lib.fa_bwd_varlen(q, k, v, dO, lse, D, dq, dk, dv, cu_q, cu_k, batch, total_q, total_k, max_q,
                              max_k, Hq, Hk, d, dt, scale, causal, stream)


def fa_fwd_varlen_dropout(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk, d, dt,
                          scale, causal, p_drop, seed, offset, stream) -> int:
    return _lib.fa_fwd_varlen_dropout(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk,
                                      d, dt, scale, causal, p_drop, seed, offset, stream)


def fa_bwd_varlen_dropout(q, k, v, dO, lse, D, dq, dk, dv, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq,
                          Hk, d, dt, scale, causal, p_drop, seed, offset, stream) -> int:
    return _lib.fa_bwd_varlen_dropout(q, k, v, dO, lse, D, dq, dk, dv, cu_q, cu_k, batch, total_q, total_k, max_q,
                                      max_k, Hq, Hk, d, dt, scale, causal, p_drop, seed, offset, stream)


def fa_fwd_splitkv(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk, d, dt, scale,
                   causal, n_splits, o_partial, lse_partial, stream) -> int:
    return _lib.fa_fwd_splitkv(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk, d, dt,
                               scale, causal, n_splits, o_partial, lse_partial, stream)


def splitkv_noalloc_bytes(total_q: int, hq: int, d: int, n_splits: int) -> int:
    """Scratch bytes fa_fwd_splitkv_noalloc needs (it refuses more than FA_NOALLOC_SCRATCH_BYTES)."""
    rows = n_splits * total_q * hq
    return ((rows * d * 4 + 255) & ~255) + rows * 4


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk, d, dt,
                           scale, causal, n_splits, stream) -> int:
    return _lib.fa_fwd_splitkv_noalloc(q, k, v, o, lse, cu_q, cu_k, batch, total_q, total_k, max_q, max_k, Hq, Hk,
                                       d, dt, scale, causal, n_splits, stream)


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(status).decode()


# ---------------------------------------------------------------------------
# torch conveniences
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def _check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FAError(status, where)


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _shape(q):
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("expected contiguous [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _expect(t, shape, dtype, like, name: str):
    """Every buffer handed to the library must be contiguous, of the given shape and
    dtype, and on q's device: the C entry points only see pointers and sizes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != like.device:
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)} on {like.device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _expect_mask(block_mask, N: int, mask_block: int, like):
    if block_mask is None:
        return
    t = -(-N // mask_block) if mask_block > 0 else 0
    _expect(block_mask, (t, t), _torch().uint8, like, "block_mask")


def _dense_args(q, k, v, block_mask, mask_block, **others):
    """Shape checks of the dense entry points; `others` maps names to (tensor, kind)
    with kind 'qkv' ([B, H, N, d], q's dtype) or 'row' ([B, H, N] float32)."""
    torch = _torch()
    B, H, N, d = _shape(q)
    _expect(k, q.shape, q.dtype, q, "k")
    _expect(v, q.shape, q.dtype, q, "v")
    for name, (t, kind) in others.items():
        if kind == "qkv":
            _expect(t, q.shape, q.dtype, q, name)
        else:
            _expect(t, (B, H, N), torch.float32, q, name)
    _expect_mask(block_mask, N, mask_block, q)
    return B, H, N, d


def forward(q, k, v, scale: Optional[float] = None, causal: bool = False, block_mask=None,
            mask_block: int = 128, out=None, lse=None, stream=None):
    """Run fa_fwd on [B, H, N, d] torch tensors; returns (o, lse)."""
    torch = _torch()
    B, H, N, d = _dense_args(q, k, v, block_mask, mask_block, out=(out, "qkv"), lse=(lse, "row"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                _dt(q), float(scale), int(bool(causal)), _ptr(block_mask), mask_block, _stream(stream))
    _check(st, "fa_fwd")
    return o, lse


def backward(q, k, v, o, lse, dO, scale: Optional[float] = None, causal: bool = False, block_mask=None,
             mask_block: int = 128, D=None, stream=None, out=None):
    """Run fa_bwd_preprocess then fa_bwd; returns (dq, dk, dv, D). `out` = optional (dq, dk, dv)."""
    torch = _torch()
    grads = out if out is not None else (None, None, None)
    B, H, N, d = _dense_args(q, k, v, block_mask, mask_block, o=(o, "qkv"), dO=(dO, "qkv"), lse=(lse, "row"),
                             D=(D, "row"), dq=(grads[0], "qkv"), dk=(grads[1], "qkv"), dv=(grads[2], "qkv"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = _dt(q)
    s = _stream(stream)
    if D is None:
        D = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fa_bwd_preprocess(o.data_ptr(), dO.data_ptr(), D.data_ptr(), B, H, N, d, dt, s), "fa_bwd_preprocess")
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dO.data_ptr(), lse.data_ptr(), D.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, dt,
                float(scale), int(bool(causal)), _ptr(block_mask), mask_block, s)
    _check(st, "fa_bwd")
    return dq, dk, dv, D


def _varlen_shapes(q, k, v, cu_q, cu_k):
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("expected contiguous token-major [total, heads, d] tensors")
    if tuple(v.shape) != tuple(k.shape) or k.dtype != q.dtype or v.dtype != q.dtype or k.shape[2] != q.shape[2]:
        raise ValueError("k and v must share shape [total_k, Hk, d] and q's dtype and d")
    for c in (cu_q, cu_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous() or c.device != q.device:
            raise ValueError("cu_seqlens must be contiguous int32 device tensors")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold batch + 1 offsets")
    return int(cu_q.numel() - 1), int(q.shape[0]), int(k.shape[0]), int(q.shape[1]), int(k.shape[1]), int(q.shape[2])


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   scale: Optional[float] = None, causal: bool = False, stream=None, out=None, lse=None,
                   p_drop: float = 0.0, seed: int = 0, offset: int = 0):
    """fa_fwd_varlen on packed tensors q [total_q, Hq, d], k/v [total_k, Hk, d];
    returns (o [total_q, Hq, d], lse [total_q, Hq]) (optionally into `out`, `lse`).
    p_drop > 0 calls fa_fwd_varlen_dropout with (p_drop, seed, offset)."""
    torch = _torch()
    batch, tq, tk, hq, hk, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _expect(out, q.shape, q.dtype, q, "out")
    _expect(lse, (tq, hq), torch.float32, q, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu_seqlens_q.data_ptr(),
            cu_seqlens_k.data_ptr(), batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hk, d, _dt(q),
            float(scale), int(bool(causal)))
    if p_drop > 0:
        _check(fa_fwd_varlen_dropout(*args, float(p_drop), int(seed), int(offset), _stream(stream)),
               "fa_fwd_varlen_dropout")
    else:
        _check(fa_fwd_varlen(*args, _stream(stream)), "fa_fwd_varlen")
    return o, lse


def backward_varlen(q, k, v, o, lse, dO, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    scale: Optional[float] = None, causal: bool = False, stream=None, out=None,
                    p_drop: float = 0.0, seed: int = 0, offset: int = 0):
    """fa_bwd_preprocess over the packed rows, then fa_bwd_varlen (fa_bwd_varlen_dropout
    when p_drop > 0: the forward's p_drop, seed, offset); returns (dq, dk, dv, D).
    `out` = optional (dq, dk, dv)."""
    torch = _torch()
    batch, tq, tk, hq, hk, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    grads = out if out is not None else (None, None, None)
    for name, t, like in (("o", o, q), ("dO", dO, q), ("dq", grads[0], q), ("dk", grads[1], k), ("dv", grads[2], v)):
        _expect(t, like.shape, q.dtype, q, name)
    _expect(lse, (tq, hq), torch.float32, q, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = _dt(q)
    s = _stream(stream)
    D = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    if tq > 0:
        _check(fa_bwd_preprocess(o.data_ptr(), dO.data_ptr(), D.data_ptr(), 1, hq, tq, d, dt, s), "fa_bwd_preprocess")
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dO.data_ptr(), lse.data_ptr(), D.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch, tq, tk,
            int(max_seqlen_q), int(max_seqlen_k), hq, hk, d, dt, float(scale), int(bool(causal)))
    if p_drop > 0:
        _check(fa_bwd_varlen_dropout(*args, float(p_drop), int(seed), int(offset), s), "fa_bwd_varlen_dropout")
    else:
        _check(fa_bwd_varlen(*args, s), "fa_bwd_varlen")
    return dq, dk, dv, D


def splitkv_workspace(total_q: int, hq: int, d: int, n_splits: int, device):
    """Partial-result buffers for fa_fwd_splitkv: (o_partial, lse_partial) in float32."""
    torch = _torch()
    return (torch.empty((n_splits, total_q, hq, d), dtype=torch.float32, device=device),
            torch.empty((n_splits, total_q, hq), dtype=torch.float32, device=device))


def forward_splitkv(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, n_splits: int,
                    scale: Optional[float] = None, causal: bool = False, workspace=None, stream=None):
    """fa_fwd_splitkv on packed tensors; returns (o, lse) like forward_varlen."""
    torch = _torch()
    batch, tq, tk, hq, hk, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    opart, lpart = splitkv_workspace(tq, hq, d, n_splits, q.device) if workspace is None else workspace
    _expect(opart, (n_splits, tq, hq, d), torch.float32, q, "workspace[0]")
    _expect(lpart, (n_splits, tq, hq), torch.float32, q, "workspace[1]")
    st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch, tq, tk, int(max_seqlen_q),
                        int(max_seqlen_k), hq, hk, d, _dt(q), float(scale), int(bool(causal)), int(n_splits),
                        opart.data_ptr(), lpart.data_ptr(), _stream(stream))
    _check(st, "fa_fwd_splitkv")
    return o, lse


def forward_dropout(q, k, v, p_drop: float, seed: int, offset: int = 0, scale: Optional[float] = None,
                    causal: bool = False, block_mask=None, mask_block: int = 128, stream=None):
    """fa_fwd_dropout on [B, H, N, d] tensors; returns (o, lse)."""
    torch = _torch()
    B, H, N, d = _dense_args(q, k, v, block_mask, mask_block)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, _dt(q),
                        float(scale), int(bool(causal)), _ptr(block_mask), mask_block, float(p_drop), int(seed),
                        int(offset), _stream(stream))
    _check(st, "fa_fwd_dropout")
    return o, lse


def backward_dropout(q, k, v, o, lse, dO, p_drop: float, seed: int, offset: int = 0, scale: Optional[float] = None,
                     causal: bool = False, block_mask=None, mask_block: int = 128, stream=None):
    """fa_bwd_preprocess then fa_bwd_dropout (same p_drop, seed, offset as the forward); returns (dq, dk, dv, D)."""
    torch = _torch()
    B, H, N, d = _dense_args(q, k, v, block_mask, mask_block, o=(o, "qkv"), dO=(dO, "qkv"), lse=(lse, "row"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = _dt(q)
    s = _stream(stream)
    D = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fa_bwd_preprocess(o.data_ptr(), dO.data_ptr(), D.data_ptr(), B, H, N, d, dt, s), "fa_bwd_preprocess")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), dO.data_ptr(), lse.data_ptr(), D.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, dt, float(scale), int(bool(causal)),
                        _ptr(block_mask), mask_block, float(p_drop), int(seed), int(offset), s)
    _check(st, "fa_bwd_dropout")
    return dq, dk, dv, D
