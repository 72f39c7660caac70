"""The C-ABI library loads, exports every symbol include/attn.h declares, and
rejects invalid arguments before any HIP call (so these run without a GPU)."""
import ctypes
import math
import os
import re

import pytest

from exact_tiled_softmax_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(attn_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.LIB_PATH):
        from exact_tiled_softmax_amd import build
        build.build()
    return attn.load()


def test_header_declares_the_expected_entry_points():
    assert set(declared_functions()) == set(attn.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_codes(lib):
    for code in (0, -1, -2, -3, 12345):
        s = attn.strerror(code)
        assert isinstance(s, str) and s
    assert lib.attn_last_hip_error() == 0


NZ = 16  # a non-null dummy pointer; validation fails before it could be used


def fwd_call(lib, q=NZ, k=NZ, v=NZ, o=NZ, lse=NZ, B=1, H=1, Tq=8, Tk=8, d=64, dv=64, scale=0.125, causal=0):
    return lib.attn_fwd(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale, causal, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
                                dict(B=0), dict(H=-1), dict(Tq=0), dict(Tk=0), dict(d=0), dict(dv=0),
                                dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=-1.0),
                                dict(B=1 << 20, H=1 << 20)])
def test_fwd_invalid_args(lib, kw):
    assert fwd_call(lib, **kw) == attn.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("d,dv", [(32, 32), (64, 128), (128, 64), (96, 96), (256, 256)])
def test_fwd_unsupported_head_dims(lib, d, dv):
    assert fwd_call(lib, d=d, dv=dv) == attn.ATTN_ERR_UNSUPPORTED


def test_fwd_splits_rejects_negative(lib):
    assert lib.attn_fwd_splits(NZ, NZ, NZ, NZ, NZ, 1, 1, 8, 8, 64, 64, 0.1, 0, -1, None) == attn.ATTN_ERR_INVALID_ARG


def test_bwd_invalid_and_unsupported(lib):
    args = [NZ] * 9 + [1, 1, 8, 8, 64, 64, 0.125, 1, None]
    for i in range(9):
        a = list(args)
        a[i] = None
        assert lib.attn_bwd(*a) == attn.ATTN_ERR_INVALID_ARG
    a = list(args)
    a[13] = a[14] = 80
    assert lib.attn_bwd(*a) == attn.ATTN_ERR_UNSUPPORTED
    a = list(args)
    a[15] = math.nan
    assert lib.attn_bwd(*a) == attn.ATTN_ERR_INVALID_ARG


def test_bwd_dlse_validates(lib):
    args = [NZ] * 10 + [1, 1, 8, 8, 64, 64, 0.125, 1, None]
    for i in range(10):  # every pointer, dlse (index 5) included, is required
        a = list(args)
        a[i] = None
        assert lib.attn_bwd_dlse(*a) == attn.ATTN_ERR_INVALID_ARG
    a = list(args)
    a[14] = a[15] = 96
    assert lib.attn_bwd_dlse(*a) == attn.ATTN_ERR_UNSUPPORTED


def test_fwd_state_validates(lib):
    args = [NZ] * 6 + [1, 1, 8, 8, 64, 64, 0.125, 1, 0, 0, None]
    for i in range(6):
        a = list(args)
        a[i] = None
        assert lib.attn_fwd_state(*a) == attn.ATTN_ERR_INVALID_ARG
    for i, bad in ((6, 0), (8, 0), (12, -0.5), (14, -1), (15, -3)):  # B, Tq, scale, q_offset, k_offset
        a = list(args)
        a[i] = bad
        assert lib.attn_fwd_state(*a) == attn.ATTN_ERR_INVALID_ARG
    a = list(args)
    a[10] = a[11] = 80
    assert lib.attn_fwd_state(*a) == attn.ATTN_ERR_UNSUPPORTED


def test_merge_states_validates(lib):
    args = [NZ, NZ, NZ, 2, NZ, NZ, 1, 1, 8, 64, None]
    for i in (0, 1, 2, 4, 5):
        a = list(args)
        a[i] = None
        assert lib.attn_merge_states(*a) == attn.ATTN_ERR_INVALID_ARG
    for i, bad in ((3, 0), (6, 0), (8, -1), (9, 0)):
        a = list(args)
        a[i] = bad
        assert lib.attn_merge_states(*a) == attn.ATTN_ERR_INVALID_ARG
    a = list(args)
    a[9] = 96
    assert lib.attn_merge_states(*a) == attn.ATTN_ERR_UNSUPPORTED


def test_fwd_standard_validates(lib):
    args = [NZ] * 5 + [1, 2, 64, 64, 128, 128, 0.088, 1, None]
    for i in range(5):
        a = list(args)
        a[i] = None
        assert lib.attn_fwd_standard(*a) == attn.ATTN_ERR_INVALID_ARG
    for i, bad in ((5, 0), (7, 0), (11, float("inf"))):
        a = list(args)
        a[i] = bad
        assert lib.attn_fwd_standard(*a) == attn.ATTN_ERR_INVALID_ARG
    a = list(args)
    a[9] = 96
    a[10] = 96
    assert lib.attn_fwd_standard(*a) == attn.ATTN_ERR_UNSUPPORTED


def test_decode_validates(lib):
    # q k v kv_lens o lse B H Tq Tk d dv scale causal stream; kv_lens may be null
    args = [NZ, NZ, NZ, None, NZ, NZ, 2, 4, 1, 4096, 128, 128, 0.088, 1, None]
    for i in (0, 1, 2, 4, 5):
        a = list(args)
        a[i] = None
        assert lib.attn_decode(*a) == attn.ATTN_ERR_INVALID_ARG
    for i, bad in ((6, 0), (8, 0), (9, 0), (12, -1.0), (12, float("nan"))):
        a = list(args)
        a[i] = bad
        assert lib.attn_decode(*a) == attn.ATTN_ERR_INVALID_ARG
    for i, bad in ((8, attn.DECODE_MAX_QUERIES + 1), (10, 96), (11, 64)):
        a = list(args)
        a[i] = bad
        assert lib.attn_decode(*a) == attn.ATTN_ERR_UNSUPPORTED
    assert lib.attn_decode_splits(*args[:-1], -1, None) == attn.ATTN_ERR_INVALID_ARG


def test_f32_entry_points_validate(lib):
    base = [NZ] * 5 + [1, 1, 8, 8, 64, 64, 0.125, 0]
    for fn in (lib.attn_fwd_f32, lib.attn_fwd_f32_unrescaled):
        assert fn(*base, -1, None) == attn.ATTN_ERR_INVALID_ARG
        assert fn(*([None] + base[1:]), 0, None) == attn.ATTN_ERR_INVALID_ARG
        b = list(base)
        b[10] = 129
        assert fn(*b, 0, None) == attn.ATTN_ERR_UNSUPPORTED
    assert lib.attn_fwd_f32(*base, -1, None) == attn.ATTN_ERR_INVALID_ARG
    assert lib.attn_fwd_f32(*base, 1025, None) == attn.ATTN_ERR_INVALID_ARG
    b = list(base)
    b[9] = 129
    assert lib.attn_fwd_f32(*b, 0, None) == attn.ATTN_ERR_UNSUPPORTED
    bb = [NZ] * 9 + [1, 1, 8, 8, 64, 200, 0.125, 0, None]
    assert lib.attn_bwd_f32(*bb) == attn.ATTN_ERR_UNSUPPORTED
    bb[5] = None
    assert lib.attn_bwd_f32(*bb) == attn.ATTN_ERR_INVALID_ARG


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(attn, "_lib", None)
    monkeypatch.setattr(attn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        attn.load()


# ---- the binding refuses wrongly shaped buffers before any launch ----------
# (CPU tensors: the shape check runs first, so these need no GPU)

def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def _f32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


B_, H_, TQ_, TK_, D_ = 2, 3, 40, 50, 64


@pytest.mark.parametrize("which,bad", [("out", (B_, H_, TQ_ - 1, D_)), ("out", (B_, H_, TQ_, D_ * 2)),
                                       ("lse", (B_, H_, TQ_ - 1)), ("lse", (B_, H_, TQ_, 1))])
def test_fwd_refuses_misshaped_outputs(lib, which, bad):
    q, k, v = _bf(B_, H_, TQ_, D_), _bf(B_, H_, TK_, D_), _bf(B_, H_, TK_, D_)
    kw = {which: (_bf(*bad) if which == "out" else _f32(*bad))}
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        attn.fwd(q, k, v, **kw)
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        attn.fwd_standard(q, k, v, **kw)


@pytest.mark.parametrize("which", ["o", "dout", "lse", "dq", "dk", "dv", "dlse"])
def test_bwd_refuses_misshaped_buffers(lib, which):
    q, k, v = _bf(B_, H_, TQ_, D_), _bf(B_, H_, TK_, D_), _bf(B_, H_, TK_, D_)
    args = dict(o=_bf(B_, H_, TQ_, D_), lse=_f32(B_, H_, TQ_), dout=_bf(B_, H_, TQ_, D_))
    # dk and dv have the key count, dq the query count: swapping them must fail
    bad = {"o": _bf(B_, H_, TK_, D_), "dout": _bf(B_, H_, TQ_, D_ + 8), "lse": _f32(B_, H_, TK_),
           "dq": _bf(B_, H_, TK_, D_), "dk": _bf(B_, H_, TQ_, D_), "dv": _bf(B_, H_, TK_ - 1, D_),
           "dlse": _f32(B_, H_ + 1, TQ_)}[which]
    kw = {}
    if which in args:
        args[which] = bad
    else:
        kw[which] = bad
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        attn.bwd(q, k, v, args["o"], args["lse"], args["dout"], **kw)


@pytest.mark.parametrize("which", ["acc", "m", "l"])
def test_fwd_state_refuses_misshaped_outputs(lib, which):
    q, k, v = _bf(B_, H_, TQ_, D_), _bf(B_, H_, TK_, D_), _bf(B_, H_, TK_, D_)
    bad = {"acc": _f32(B_, H_, TQ_, D_ - 1), "m": _f32(B_, H_, TK_), "l": _f32(B_, H_ + 1, TQ_)}[which]
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        attn.fwd_state(q, k, v, **{which: bad})


@pytest.mark.parametrize("which", ["out", "lse"])
def test_merge_states_refuses_misshaped_outputs(lib, which):
    acc, m, l = _f32(3, B_, H_, TQ_, D_), _f32(3, B_, H_, TQ_), _f32(3, B_, H_, TQ_)
    bad = {"out": _bf(B_, H_, TQ_ + 1, D_), "lse": _f32(B_, H_, TQ_, 1)}[which]
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        attn.merge_states(acc, m, l, **{which: bad})


def test_f32_and_decode_refuse_misshaped_buffers(lib):
    import torch
    q, k, v = _f32(1, 2, 9, 16), _f32(1, 2, 11, 16), _f32(1, 2, 11, 16)
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.fwd_f32(q, k, v, lse=_f32(1, 2, 8))
    with pytest.raises(ValueError, match="o must have shape"):
        attn.bwd_f32(q, k, v, _f32(1, 2, 11, 16), _f32(1, 2, 9), _f32(1, 2, 9, 16))
    qd, kd, vd = _bf(3, 2, 1, 64), _bf(3, 2, 100, 64), _bf(3, 2, 100, 64)
    with pytest.raises(ValueError, match="kv_lens must have shape"):
        attn.decode(qd, kd, vd, kv_lens=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="out must have shape"):
        attn.decode(qd, kd, vd, out=_bf(3, 2, 2, 64))


def test_backward_row_count_limit_is_the_abi_limit(lib):
    # the largest B*H*Tq the ABI accepts: argument checks pass (the call then
    # stops at the first null pointer check, before any HIP call), and one
    # row more is refused
    nz = NZ
    rows_max = 2**31 - 1
    assert lib.attn_bwd(nz, nz, nz, nz, nz, nz, nz, nz, None, 1, 1, rows_max, 8, 64, 64, 0.125, 0, None) \
        == attn.ATTN_ERR_INVALID_ARG  # null dv_grad
    assert lib.attn_bwd(nz, nz, nz, nz, nz, nz, nz, nz, nz, 2, 1, rows_max, 8, 64, 64, 0.125, 0, None) \
        == attn.ATTN_ERR_INVALID_ARG  # B*H*Tq past 2^31 - 1
