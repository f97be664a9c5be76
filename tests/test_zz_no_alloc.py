"""fa_fwd_splitkv_noalloc: the split-KV forward whose partial results live in
the library's static device scratch instead of caller workspace.

Through the raw C entry point: two calls in a row (the second with a smaller
input) must give the bits of fa_fwd_splitkv with caller workspace (same
kernels, same arithmetic) and match the oracle within the O / LSE tolerances;
sizes beyond the scratch are refused before any HIP call.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle.varlen as ov
from harness import LSE_TOL, O_TOL, from_dev, say, to_dev

A = 1 << 20          # fake, never-dereferenced 16-byte-aligned address


def test_scratch_limit_is_refused_before_any_hip_call():
    from exact_io_aware_04_amd import fa
    # 2048 rows x 32 heads x 8 splits x 129 floats = 270 MB of partials > 32 MiB
    tq, hq, hk, d, splits = 2048, 32, 8, 128, 8
    assert fa.splitkv_noalloc_bytes(tq, hq, d, splits) > fa.FA_NOALLOC_SCRATCH_BYTES
    st = fa.fa_fwd_splitkv_noalloc(A, A, A, A, A, A, A, 2048, tq, 4096, 1, 4096, hq, hk, d, fa.FA_BF16,
                                   0.088, 1, splits, None)
    assert st == -10 and fa.STATUS[st] == "FA_ERR_SCRATCH"
    assert "scratch" in fa.fa_status_string(st)
    # the usual argument checks come first
    assert fa.fa_fwd_splitkv_noalloc(None, A, A, A, A, A, A, 1, 1, 8, 1, 8, 4, 4, 64, 0, 0.1, 0, 1, None) == -1
    assert fa.fa_fwd_splitkv_noalloc(A, A, A, A, A, A, A, 1, 1, 8, 1, 8, 4, 4, 64, 0, 0.1, 0, 0, None) == -2
    assert fa.fa_fwd_splitkv_noalloc(A, A, A, A, A, A, A, 1, 1, 8, 1, 8, 4, 4, 96, 0, 0.1, 0, 1, None) == -4


CASES = [
    # (name, lengths_q, lengths_k, Hq, Hk, d, dtype, causal, n_splits)
    ("decode_gqa_32seq", [1] * 32, list(range(8192, 8192 + 32 * 257, 257)), 32, 8, 128, ai.BF16, True, 8),
    ("smaller_mixed", [1, 4, 2], [700, 33, 1500], 8, 2, 64, ai.F16, False, 3),
]


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).cuda()


@pytest.mark.gpu
def test_noalloc_matches_workspace_path_on_consecutive_calls():
    import torch
    from exact_io_aware_04_amd import fa
    for name, lq, lk, hq, hk, d, dtype, causal, splits in CASES:
        seed = 60_000 + d + splits
        say(f"[noalloc] {name}: {len(lq)} seqs Hq={hq} Hk={hk} d={d} {dtype} causal={causal} splits={splits}")
        pk = ai.draw_packed(lq, lk, hq, hk, d, dtype, seed)
        q, k, v = (to_dev(getattr(pk, n), pk.dtype) for n in ("q", "k", "v"))
        cu_q, cu_k = _dev_i32(pk.cu_q), _dev_i32(pk.cu_k)
        tq, tk, mq, mk = q.shape[0], k.shape[0], max(lq), max(lk)
        scale = 1.0 / np.sqrt(d)
        assert fa.splitkv_noalloc_bytes(tq, hq, d, splits) <= fa.FA_NOALLOC_SCRATCH_BYTES
        o_ws, lse_ws = fa.forward_splitkv(q, k, v, cu_q, cu_k, mq, mk, splits, scale, causal)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((tq, hq), float("nan"), dtype=torch.float32, device=q.device)
        code = fa.FA_BF16 if dtype == ai.BF16 else fa.FA_F16
        st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       cu_q.data_ptr(), cu_k.data_ptr(), len(lq), tq, tk, mq, mk, hq, hk, d, code,
                                       scale, int(causal), splits, torch.cuda.current_stream().cuda_stream)
        assert st == 0, fa.fa_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ws.view(torch.int16)), f"{name}: O differs from the workspace path"
        assert torch.equal(lse, lse_ws), f"{name}: LSE differs from the workspace path"
        o_ref, lse_ref = ov.forward(pk.f64("q"), pk.f64("k"), pk.f64("v"), pk.cu_q, pk.cu_k, scale, causal)
        og, lg = from_dev(o, dtype), lse.double().cpu().numpy()
        err = float(np.abs(og - o_ref).max())
        assert err <= O_TOL[dtype], f"{name}: O error {err:.3e}"
        lerr = float(np.abs(lg - lse_ref).max())
        assert lerr <= LSE_TOL[dtype], f"{name}: LSE error {lerr:.3e}"
        say(f"    {name}: bitwise equal to the workspace path; O error {err:.2e}, LSE error {lerr:.2e}")
