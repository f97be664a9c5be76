"""C ABI: the library loads, exports every declared symbol, and validates its
arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_io_aware_04_amd.fa", reason="libfa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fa_[a-z_0-9]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings():
    for code, name in fa.STATUS.items():
        assert fa.fa_status_string(code).startswith(name)
    assert "unknown" in fa.fa_status_string(123)


# Fake, never-dereferenced addresses: validation rejects before any HIP call.
A = 1 << 20          # 16-byte aligned
MIS = A + 8          # misaligned


def fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=16, d=64, dt=fa.FA_F16, scale=0.125, causal=0,
                block_mask=None, mask_block=128, stream=None)
    args.update(kw)
    return fa.fa_fwd(*args.values())


def bwd(**kw):
    args = dict(q=A, k=A, v=A, dO=A, lse=A, D=A, dq=A, dk=A, dv=A, B=1, H=1, N=16, d=64,
                dt=fa.FA_F16, scale=0.125, causal=0, block_mask=None, mask_block=128, stream=None)
    args.update(kw)
    return fa.fa_bwd(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=-1), -2), (dict(N=0), -2), (dict(B=1 << 20, H=1 << 10, N=1 << 20), -2), (dict(N=1 << 22, d=128), -2), (dict(N=1 << 23), -2),
    (dict(dt=2), -3), (dict(dt=-1), -3),
    (dict(d=32), -4), (dict(d=96), -4), (dict(d=256), -4),
    (dict(block_mask=A, mask_block=64), -5),
    (dict(q=MIS), -6), (dict(lse=MIS), -6),
    (dict(scale=0.0), -8), (dict(scale=-1.0), -8), (dict(scale=float("inf")), -8), (dict(scale=float("nan")), -8),
])
def test_fwd_validation(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dq=None), -1), (dict(D=None), -1), (dict(dv=None), -1),
    (dict(N=0), -2), (dict(dt=7), -3), (dict(d=80), -4),
    (dict(block_mask=A, mask_block=256), -5),
    (dict(dk=MIS), -6), (dict(dq=MIS), -6),
    (dict(scale=0.0), -8),
])
def test_bwd_validation(kw, code):
    assert bwd(**kw) == code


def fwd_dropout(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=16, d=64, dt=fa.FA_F16, scale=0.125, causal=0,
                block_mask=None, mask_block=128, p=0.1, seed=1, offset=0, stream=None)
    args.update(kw)
    return fa.fa_fwd_dropout(*args.values())


def bwd_dropout(**kw):
    args = dict(q=A, k=A, v=A, dO=A, lse=A, D=A, dq=A, dk=A, dv=A, B=1, H=1, N=16, d=64, dt=fa.FA_F16, scale=0.125,
                causal=0, block_mask=None, mask_block=128, p=0.1, seed=1, offset=0, stream=None)
    args.update(kw)
    return fa.fa_bwd_dropout(*args.values())


DROPOUT_CASES = [
    (dict(q=None), -1), (dict(p=-0.1), -9), (dict(p=1.0), -9), (dict(p=float("nan")), -9), (dict(p=float("inf")), -9),
    (dict(N=0), -2), (dict(d=32), -4), (dict(dt=5), -3), (dict(block_mask=A, mask_block=64), -5), (dict(lse=MIS), -6),
    (dict(scale=0.0), -8),
]


@pytest.mark.parametrize("kw,code", DROPOUT_CASES)
def test_fwd_dropout_validation(kw, code):
    assert fwd_dropout(**kw) == code


@pytest.mark.parametrize("kw,code", DROPOUT_CASES + [(dict(dk=None), -1), (dict(D=MIS), -6)])
def test_bwd_dropout_validation(kw, code):
    assert bwd_dropout(**kw) == code


def fwd_varlen(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, cu_q=A, cu_k=A, batch=2, total_q=40, total_k=50, max_q=30, max_k=30,
                Hq=4, Hk=2, d=64, dt=fa.FA_BF16, scale=0.125, causal=1, stream=None)
    args.update(kw)
    return fa.fa_fwd_varlen(*args.values())


def bwd_varlen(**kw):
    args = dict(q=A, k=A, v=A, dO=A, lse=A, D=A, dq=A, dk=A, dv=A, cu_q=A, cu_k=A, batch=2, total_q=40,
                total_k=50, max_q=30, max_k=30, Hq=4, Hk=2, d=128, dt=fa.FA_F16, scale=0.125, causal=0,
                stream=None)
    args.update(kw)
    return fa.fa_bwd_varlen(*args.values())


VARLEN_CASES = [
    (dict(q=None), -1), (dict(cu_q=None), -1), (dict(cu_k=None), -1),
    (dict(batch=0), -2), (dict(total_q=-1), -2), (dict(max_q=0), -2), (dict(max_k=0), -2),
    (dict(Hq=3, Hk=2), -2), (dict(Hk=0), -2), (dict(max_q=1 << 20, Hq=64), -2), (dict(max_k=1 << 20, Hk=64), -2),
    # many one-token sequences with grouped heads: the 8-wave forward grid (256-row
    # blocks of 512 threads) would pass 2^32 work-items although 128-row blocks would not
    (dict(batch=1_500_000, total_q=1_500_000, total_k=1_500_000, max_q=1, max_k=1, Hq=8, Hk=1), -2),
    (dict(dt=3), -3), (dict(d=96), -4),
    (dict(o=MIS), -6), (dict(scale=0.0), -8),
]


@pytest.mark.parametrize("kw,code", VARLEN_CASES)
def test_fwd_varlen_validation(kw, code):
    assert fwd_varlen(**kw) == code


@pytest.mark.parametrize("kw,code", [c for c in VARLEN_CASES if "o" not in c[0]] + [
    (dict(dk=None), -1), (dict(D=None), -1), (dict(dv=MIS), -6)])
def test_bwd_varlen_validation(kw, code):
    assert bwd_varlen(**kw) == code


def fwd_varlen_dropout(p_drop=0.1, seed=7, offset=0, **kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, cu_q=A, cu_k=A, batch=2, total_q=40, total_k=50, max_q=30, max_k=30,
                Hq=4, Hk=2, d=64, dt=fa.FA_BF16, scale=0.125, causal=1)
    args.update(kw)
    return fa.fa_fwd_varlen_dropout(*args.values(), p_drop, seed, offset, None)


def bwd_varlen_dropout(p_drop=0.1, seed=7, offset=0, **kw):
    args = dict(q=A, k=A, v=A, dO=A, lse=A, D=A, dq=A, dk=A, dv=A, cu_q=A, cu_k=A, batch=2, total_q=40,
                total_k=50, max_q=30, max_k=30, Hq=4, Hk=2, d=128, dt=fa.FA_F16, scale=0.125, causal=0)
    args.update(kw)
    return fa.fa_bwd_varlen_dropout(*args.values(), p_drop, seed, offset, None)


VARLEN_DROPOUT_CASES = [(dict(p_drop=-0.1), -9), (dict(p_drop=1.0), -9), (dict(p_drop=float("nan")), -9),
                        (dict(q=None, p_drop=float("nan")), -1)]


@pytest.mark.parametrize("kw,code", VARLEN_CASES + VARLEN_DROPOUT_CASES)
def test_fwd_varlen_dropout_validation(kw, code):
    assert fwd_varlen_dropout(**kw) == code


@pytest.mark.parametrize("kw,code", [c for c in VARLEN_CASES if "o" not in c[0]] + VARLEN_DROPOUT_CASES + [
    (dict(dk=None), -1), (dict(D=None), -1), (dict(dv=MIS), -6)])
def test_bwd_varlen_dropout_validation(kw, code):
    assert bwd_varlen_dropout(**kw) == code


def fwd_splitkv(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, cu_q=A, cu_k=A, batch=2, total_q=2, total_k=5000, max_q=1, max_k=4096,
                Hq=8, Hk=2, d=128, dt=fa.FA_BF16, scale=0.125, causal=0, n_splits=8, o_part=A, lse_part=A,
                stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv(*args.values())


@pytest.mark.parametrize("kw,code", VARLEN_CASES + [
    (dict(o_part=None), -1), (dict(lse_part=None), -1), (dict(n_splits=0), -2),
    (dict(n_splits=fa.FA_MAX_SPLITS + 1), -2), (dict(lse_part=MIS), -6), (dict(o_part=MIS), -6)])
def test_fwd_splitkv_validation(kw, code):
    assert fwd_splitkv(**kw) == code


def test_preprocess_validation():
    assert fa.fa_bwd_preprocess(None, A, A, 1, 1, 16, 64, 0, None) == -1
    assert fa.fa_bwd_preprocess(A, A, A, 1, 1, 0, 64, 0, None) == -2
    assert fa.fa_bwd_preprocess(A, A, A, 1, 1, 16, 64, 5, None) == -3
    assert fa.fa_bwd_preprocess(A, A, A, 1, 1, 16, 48, 0, None) == -4
    assert fa.fa_bwd_preprocess(A, MIS, A, 1, 1, 16, 64, 0, None) == -6


def test_binding_keeps_a_single_hip_runtime():
    """The binding loads torch's HIP runtime before libfa.so, so only one
    libamdhip64 / libhsa-runtime64 is mapped, whatever is imported first."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from exact_io_aware_04_amd import fa\n"
        "import torch\n"
        "maps = open('/proc/self/maps').read().splitlines()\n"
        "libs = {l.split()[-1] for l in maps if 'amdhip64' in l or 'hsa-runtime64' in l}\n"
        "print(len([x for x in libs if 'amdhip64' in x]), len([x for x in libs if 'hsa-runtime64' in x]))\n"
    ) % ROOT
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["1", "1"], out.stdout


def test_binding_rejects_mismatched_buffers():
    """The torch wrappers check every buffer they hand to the C entry points
    (shape, dtype, contiguity, device) before any HIP call."""
    import torch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.float16)
    k, v, o, do = (torch.zeros_like(q) for _ in range(4))
    lse = torch.zeros((1, 2, 64), dtype=torch.float32)
    bad = [
        lambda: fa.forward(q, k[:, :, :32], v),                                   # k shorter than q
        lambda: fa.forward(q, k, v.to(torch.bfloat16)),                           # dtype mismatch
        lambda: fa.forward(q, k, v, out=torch.zeros((1, 2, 64, 32), dtype=torch.float16)),
        lambda: fa.forward(q, k, v, lse=torch.zeros((1, 2, 64), dtype=torch.float16)),
        lambda: fa.forward(q, k, v, block_mask=torch.ones((2, 2), dtype=torch.uint8)),   # needs 1 x 1
        lambda: fa.forward(q, k, v.transpose(2, 3)),                              # not contiguous
        lambda: fa.backward(q, k, v, o, lse, do[:, :1]),
        lambda: fa.backward(q, k, v, o, lse[:, :, :10], do),
        lambda: fa.backward(q, k, v, o, lse, do, out=(torch.zeros_like(q), torch.zeros_like(q), q[:, :1])),
        lambda: fa.forward_dropout(q, k[:, :1], v, 0.1, 1),
        lambda: fa.backward_dropout(q, k, v, o[:, :, :8], lse, do, 0.1, 1),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
