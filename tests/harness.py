"""GPU-test helpers: move seeded 16-bit inputs to the device, run the C ABI
through the Python binding, bring results back as float64, and compare with
the oracle under the stated tolerances.

Tolerances (written here once, used by every parity test):
  * O: max |GPU - oracle| <= 2e-3 for fp16, <= 1e-2 for bf16.
  * dQ, dK, dV, per tensor: ||GPU - oracle||_F / ||oracle||_F <= 2e-2, and
    max |GPU - oracle| / max |oracle| <= 4 u (u = unit roundoff of the 16-bit
    type: the random walk of the operand roundings reaches ~6 u R at its
    largest element against a largest |oracle| of ~5.5 R on unstructured
    inputs, plus u for the final rounding); and, element by element, the
    rounding bound of tests/error_model.py (which also bounds every row).
    Where the exact gradient is no larger than its rounding bound (norms over
    the tensor; e.g. dQ of rows that see a single key, exactly 0), the two
    relative measures are undefined and only the element-wise bound applies.
  * LSE: max |GPU - oracle| on rows with a visible key <= 2e-3 (fp16) /
    4e-3 (bf16); rows without one must be -inf on both sides. The row sum l
    adds the probabilities rounded to the operand type (unit roundoff u), so
    |d ln l| <= u (2^-11 fp16, 2^-8 bf16 = 3.9e-3), plus ~1e-5 of fp32 and
    hardware exp2 / log error.
  * D (preprocess): max |GPU - sum(dO * O_gpu)| <= 1e-3 * (1 + |D|), computed
    from the GPU's own stored O, which is what the preprocess reads.
"""
from __future__ import annotations

import sys

import numpy as np

import attn_inputs as ai
from error_model import UNIT_ROUNDOFF, elementwise_bound

O_TOL = {ai.F16: 2e-3, ai.BF16: 1e-2}
GRAD_REL_TOL = 2e-2
# LSE: the kernels add the probabilities rounded to the operand type (RNE, unit
# roundoff u = 2^-11 fp16, 2^-8 bf16) into the row sum l, so |d ln l| <= u; plus
# fp32 / hardware exp2-log error (~1e-5). fp16 keeps the looser 2e-3.
LSE_TOL = {ai.F16: 2e-3, ai.BF16: 4e-3}
# max |GPU - oracle| / max |oracle| per gradient tensor, in units of u
GRAD_MAX_RATIO_U = 4.0


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.float16 if dtype == ai.F16 else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).cuda()


def from_dev(t, dtype: str) -> np.ndarray:
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return ai.bits_to_f64(bits, dtype)


def mask_dev(mask):
    import torch
    if mask is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()


def run_gpu(dr: ai.Drawn, scale: float, causal: bool, mask=None, backward: bool = True, poison: bool = True):
    """fa_fwd (+ fa_bwd_preprocess, fa_bwd) on the drawn inputs. Returns float64 numpy arrays.
    With `poison`, every output buffer starts as NaN, so an element a kernel fails to write
    fails the comparison."""
    import torch
    from exact_io_aware_04_amd import fa
    q, k, v = (to_dev(getattr(dr, n), dr.dtype) for n in "qkv")
    bm = mask_dev(mask)
    B, H, N, d = dr.q.shape
    o = torch.full_like(q, float("nan")) if poison else None
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device) if poison else None
    o, lse = fa.forward(q, k, v, scale, causal, bm, out=o, lse=lse)
    out = {"o_dev": o, "lse_dev": lse}
    if backward:
        do = to_dev(dr.do, dr.dtype)
        grads = tuple(torch.full_like(t, float("nan")) for t in (q, k, v)) if poison else None
        dq, dk, dv, D = fa.backward(q, k, v, o, lse, do, scale, causal, bm, out=grads)
        out.update(dq=dq, dk=dk, dv=dv, D=D)
    torch.cuda.synchronize()
    res = {"o": from_dev(o, dr.dtype), "lse": lse.double().cpu().numpy()}
    if backward:
        for n in ("dq", "dk", "dv"):
            res[n] = from_dev(out[n], dr.dtype)
        res["D"] = out["D"].double().cpu().numpy()
    return res


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    na = float(np.linalg.norm(a - b))
    return na / nb if nb > 0 else na


def check_forward(o, lse, o_ref, lse_ref, dtype, what=""):
    assert np.isfinite(o).all(), f"{what}: non-finite O (unwritten output?)"
    err = float(np.abs(o - o_ref).max()) if o.size else 0.0
    assert err <= O_TOL[dtype], f"{what}: O max-abs error {err:.3e} > {O_TOL[dtype]}"
    live = np.isfinite(lse_ref)
    assert (np.isneginf(lse) == ~live).all(), f"{what}: LSE -inf pattern differs"
    lerr = float(np.abs(lse[live] - lse_ref[live]).max()) if live.any() else 0.0
    assert lerr <= LSE_TOL[dtype], f"{what}: LSE max-abs error {lerr:.3e}"
    return err, lerr


def check_grads(res, ref, what="", scales=None, dtype=None, max_ratio: bool = True):
    """Gradient parity: the relative Frobenius error per tensor; with `dtype`, the
    largest error against the largest reference value; with `scales` (from
    error_model.gradient_scales_head), every element against its rounding bound.
    Returns {name: {"fro", "max_ratio", "worst"}} (worst = largest error / bound)."""
    errs = {}
    for n in ("dq", "dk", "dv"):
        g, r = res[n], ref[n]
        assert g.shape == r.shape, f"{what}: {n} shape {g.shape} vs {r.shape}"
        assert np.isfinite(g).all(), f"{what}: non-finite {n}"
        diff = np.abs(g - r)
        bound = elementwise_bound(r, scales[n], dtype) if scales is not None and r.size else None
        # A gradient whose exact value is no larger than its own rounding bound
        # (e.g. dQ of a row that sees one key: dS = P (dP - D) = 0, so only the
        # rounding of the stored O, through D, remains) has no meaningful
        # relative error; there the element-wise bound alone applies.
        relative = bound is None or float(np.linalg.norm(r)) > float(np.linalg.norm(bound))
        e = rel_fro(g, r)
        info = {"fro": e}
        if relative:
            assert e <= GRAD_REL_TOL, f"{what}: {n} relative error {e:.3e} > {GRAD_REL_TOL}"
        if dtype is not None and r.size:
            mref = float(np.abs(r).max())
            ratio = float(diff.max()) / mref if mref > 0 else 0.0
            info["max_ratio"] = ratio
            lim = GRAD_MAX_RATIO_U * UNIT_ROUNDOFF[dtype]
            if max_ratio and mref > 0 and relative:
                assert ratio <= lim, f"{what}: {n} max|d|/max|ref| {ratio:.3e} > {lim:.3e}"
        if bound is not None:
            q = diff / bound
            worst = int(np.argmax(q))
            info["worst"] = float(q.flat[worst])
            if q.flat[worst] > 1.0:
                idx = np.unravel_index(worst, r.shape)
                bad = int((q > 1.0).sum())
                raise AssertionError(
                    f"{what}: {n} beyond its rounding bound at {bad} element(s); worst {idx}: "
                    f"gpu {g[idx]:.6e} oracle {r[idx]:.6e} |d| {diff[idx]:.3e} bound {bound[idx]:.3e}")
        errs[n] = info
    return errs


def report(what: str, errs) -> None:
    say(f"    {what}: " + "  ".join(
        f"{n} fro {e['fro']:.2e} max {e.get('max_ratio', float('nan')):.2e} worst {e.get('worst', float('nan')):.2f}"
        for n, e in errs.items()))


def check_D(D, do, o_gpu, what=""):
    ref = (do * o_gpu).sum(axis=-1)
    err = float((np.abs(D - ref) / (1 + np.abs(ref))).max())
    assert err <= 1e-3, f"{what}: D error {err:.3e}"
