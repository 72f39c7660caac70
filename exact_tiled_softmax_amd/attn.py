"""Thin ctypes binding of libattn.so (include/attn.h).

Argument marshalling only: tensors are passed as device pointers and the
current torch stream as the hipStream_t; every step of the computation runs in
the library's HIP kernels.  There is no fallback: if libattn.so is missing or
the GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ATTN_LIB", os.path.join(_PKG, "libattn.so"))

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_HIP = -3
ATTN_ERR_TOO_LARGE = -4
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("attn_fwd", "attn_fwd_splits", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_dlse", "attn_fwd_state", "attn_merge_states",
            "attn_decode", "attn_decode_splits", "attn_fwd_standard", "attn_fwd_f32", "attn_fwd_f32_unrescaled", "attn_bwd_f32", "attn_strerror", "attn_last_hip_error", "attn_profile_start",
            "attn_profile_stop", "attn_profile_query")

# kernel kinds of attn_profile_query (include/attn.h)
KERNEL_FWD = 0
KERNEL_FWD_AUX = 1
KERNEL_BWD_PREP = 2
KERNEL_BWD_DKDV = 3
KERNEL_BWD_DQ = 4
KERNEL_DECODE = 5
KERNEL_STANDARD = 6
KERNEL_NAMES = {0: "fwd", 1: "fwd_aux", 2: "bwd_prep", 3: "bwd_dkdv", 4: "bwd_dq", 5: "decode", 6: "standard"}
DECODE_MAX_QUERIES = 4

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libattn.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with `python -m exact_tiled_softmax_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    dims = [I, I, I, I, I, I, F, I]  # B H Tq Tk d dv scale causal
    lib.attn_fwd.argtypes = [P, P, P, P, P, *dims, P]
    lib.attn_fwd_splits.argtypes = [P, P, P, P, P, *dims, I, P]
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, *dims, P]
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, *dims, P]
    lib.attn_bwd_dlse.argtypes = [P, P, P, P, P, P, P, P, P, P, *dims, P]
    lib.attn_fwd_state.argtypes = [P, P, P, P, P, P, *dims, I, I, P]
    lib.attn_merge_states.argtypes = [P, P, P, I, P, P, I, I, I, I, P]
    lib.attn_decode.argtypes = [P, P, P, P, P, P, *dims, P]
    lib.attn_fwd_standard.argtypes = [P, P, P, P, P, *dims, P]
    lib.attn_decode_splits.argtypes = [P, P, P, P, P, P, *dims, I, P]
    lib.attn_fwd_f32.argtypes = [P, P, P, P, P, *dims, I, P]
    lib.attn_fwd_f32_unrescaled.argtypes = [P, P, P, P, P, *dims, I, P]
    lib.attn_bwd_f32.argtypes = [P, P, P, P, P, P, P, P, P, *dims, P]
    for fn in ("attn_fwd", "attn_fwd_splits", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_dlse", "attn_fwd_state", "attn_merge_states",
               "attn_decode", "attn_decode_splits", "attn_fwd_standard", "attn_fwd_f32", "attn_fwd_f32_unrescaled", "attn_bwd_f32"):
        getattr(lib, fn).restype = I
    lib.attn_strerror.argtypes = [I]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = I
    lib.attn_profile_start.argtypes = []
    lib.attn_profile_start.restype = I
    lib.attn_profile_stop.argtypes = []
    lib.attn_profile_stop.restype = I
    lib.attn_profile_query.argtypes = [I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.attn_profile_query.restype = I
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().attn_strerror(code).decode()


def _check(fn: str, rc: int) -> None:
    if rc != ATTN_OK:
        msg = strerror(rc)
        if rc == ATTN_ERR_HIP:
            msg += f" (hipError {load().attn_last_hip_error()})"
        raise AttnError(fn, rc, msg)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dims(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, dim]")
    B, H, Tq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape[:2] != (B, H) or k.shape[3] != d or v.shape[2] != k.shape[2]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, H, Tq, k.shape[2], d, v.shape[3]


def _shapes(**named) -> None:
    """Refuse caller-supplied buffers whose shape differs from the one the
    call's dimensions imply (name=(tensor or None, shape)); runs before any
    other check, so a mismatch is reported as such."""
    for name, (t, shape) in named.items():
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device, shape=None) -> None:
    """Check a tensor handed to the library: dtype, device, contiguity and,
    when given, its exact shape (the kernels read and write the full extent
    the dimensions imply, so a smaller buffer would be overrun)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q, k, v, scale=None, causal=False, out=None, lse=None, num_splits=None):
    """bf16 forward: returns (o [B,H,Tq,dv] bf16, lse [B,H,Tq] fp32)."""
    lib = load()
    B, H, Tq, Tk, d, dv = _dims(q, k, v)
    _shapes(out=(out, (B, H, Tq, dv)), lse=(lse, (B, H, Tq)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Tq, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev, (B, H, Tq, dv))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Tq, Tk, d, dv, float(scale), int(bool(causal)))
    if num_splits is None:
        _check("attn_fwd", lib.attn_fwd(*args, _stream(dev)))
    else:
        _check("attn_fwd_splits", lib.attn_fwd_splits(*args, int(num_splits), _stream(dev)))
    return out, lse


def bwd(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None, dlse=None, noalloc=False):
    """bf16 backward: returns (dq, dk, dv) bf16 with the shapes of q, k, v.
    dlse (optional, fp32 [B,H,Tq]): upstream gradient on the LSE output.
    noalloc=True calls attn_bwd_noalloc (workspace in the library's static
    scratch; no dlse)."""
    lib = load()
    B, H, Tq, Tk, d, dvd = _dims(q, k, v)
    _shapes(o=(o, (B, H, Tq, dvd)), dout=(dout, (B, H, Tq, dvd)), lse=(lse, (B, H, Tq)), dq=(dq, (B, H, Tq, d)),
            dk=(dk, (B, H, Tk, d)), dv=(dv, (B, H, Tk, dvd)), dlse=(dlse, (B, H, Tq)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, dev)
    _need(o, "o", torch.bfloat16, dev, (B, H, Tq, dvd))
    _need(dout, "dout", torch.bfloat16, dev, (B, H, Tq, dvd))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, shp in ((dq, "dq", (B, H, Tq, d)), (dk, "dk", (B, H, Tk, d)), (dv, "dv", (B, H, Tk, dvd))):
        _need(t, n, torch.bfloat16, dev, shp)
    tail = (_ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, Tq, Tk, d, dvd, float(scale), int(bool(causal)),
            _stream(dev))
    if noalloc:
        if dlse is not None:
            raise ValueError("attn_bwd_noalloc takes no dlse")
        _check("attn_bwd_noalloc", lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), *tail))
    elif dlse is None:
        _check("attn_bwd", lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), *tail))
    else:
        _need(dlse, "dlse", torch.float32, dev, (B, H, Tq))
        _check("attn_bwd_dlse", lib.attn_bwd_dlse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dlse), *tail))
    return dq, dk, dv


def fwd_state(q, k, v, scale=None, causal=False, q_offset=0, k_offset=0, acc=None, m=None, l=None):
    """Partial online-softmax state of the keys k, v for the queries q:
    returns (acc [B,H,Tq,dv] fp32, m [B,H,Tq] fp32 natural-log, l [B,H,Tq] fp32),
    written into acc, m, l when given (e.g. slices of stacked buffers for
    merge_states)."""
    lib = load()
    B, H, Tq, Tk, d, dv = _dims(q, k, v)
    _shapes(acc=(acc, (B, H, Tq, dv)), m=(m, (B, H, Tq)), l=(l, (B, H, Tq)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if acc is None:
        acc = torch.empty((B, H, Tq, dv), dtype=torch.float32, device=dev)
    if m is None:
        m = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    if l is None:
        l = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    _need(acc, "acc", torch.float32, dev, (B, H, Tq, dv))
    _need(m, "m", torch.float32, dev, (B, H, Tq))
    _need(l, "l", torch.float32, dev, (B, H, Tq))
    rc = lib.attn_fwd_state(_ptr(q), _ptr(k), _ptr(v), _ptr(acc), _ptr(m), _ptr(l), B, H, Tq, Tk, d, dv,
                            float(scale), int(bool(causal)), int(q_offset), int(k_offset), _stream(dev))
    _check("attn_fwd_state", rc)
    return acc, m, l


def merge_states(acc, m, l, out=None, lse=None):
    """Merge n partial states stacked on dim 0 (acc [n,B,H,Tq,dv], m and l
    [n,B,H,Tq], fp32) into (o [B,H,Tq,dv] bf16, lse [B,H,Tq] fp32), written
    into out and lse when given."""
    lib = load()
    if acc.dim() != 5 or m.dim() != 4 or l.dim() != 4 or m.shape != acc.shape[:4] or l.shape != m.shape:
        raise ValueError("acc must be [n,B,H,Tq,dv] and m, l [n,B,H,Tq]")
    n, B, H, Tq, dv = acc.shape
    _shapes(out=(out, (B, H, Tq, dv)), lse=(lse, (B, H, Tq)))
    dev = acc.device
    for t, nm in ((acc, "acc"), (m, "m"), (l, "l")):
        _need(t, nm, torch.float32, dev)
    o = torch.empty((B, H, Tq, dv), dtype=torch.bfloat16, device=dev) if out is None else out
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    _need(o, "out", torch.bfloat16, dev, (B, H, Tq, dv))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    rc = lib.attn_merge_states(_ptr(acc), _ptr(m), _ptr(l), n, _ptr(o), _ptr(lse), B, H, Tq, dv, _stream(dev))
    _check("attn_merge_states", rc)
    return o, lse


def fwd_standard(q, k, v, scale=None, causal=False, out=None, lse=None):
    """Standard attention with the score matrix materialised in HBM (bf16 in
    and out, as fwd): returns (o, lse).  For the IO comparison."""
    lib = load()
    B, H, Tq, Tk, d, dv = _dims(q, k, v)
    _shapes(out=(out, (B, H, Tq, dv)), lse=(lse, (B, H, Tq)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, H, Tq, dv), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.bfloat16, dev, (B, H, Tq, dv))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    rc = lib.attn_fwd_standard(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Tq, Tk, d, dv, float(scale),
                               int(bool(causal)), _stream(dev))
    _check("attn_fwd_standard", rc)
    return out, lse


def decode(q, k, v, kv_lens=None, scale=None, causal=False, out=None, lse=None, num_splits=None):
    """bf16 decode: the Tq (<= 4) newest queries q [B,H,Tq,d] of each sequence
    against the key/value cache k, v [B,H,Tk,d]; kv_lens (int32 [B] on the
    device, optional) gives each sequence's cache length.  Returns
    (o [B,H,Tq,dv] bf16, lse [B,H,Tq] fp32)."""
    lib = load()
    B, H, Tq, Tk, d, dv = _dims(q, k, v)
    _shapes(out=(out, (B, H, Tq, dv)), lse=(lse, (B, H, Tq)), kv_lens=(kv_lens, (B,)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, dev)
    if kv_lens is not None:
        _need(kv_lens, "kv_lens", torch.int32, dev, (B,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Tq, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev, (B, H, Tq, dv))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    lens = 0 if kv_lens is None else _ptr(kv_lens)
    args = (_ptr(q), _ptr(k), _ptr(v), lens, _ptr(out), _ptr(lse), B, H, Tq, Tk, d, dv, float(scale),
            int(bool(causal)))
    if num_splits is None:
        _check("attn_decode", lib.attn_decode(*args, _stream(dev)))
    else:
        _check("attn_decode_splits", lib.attn_decode_splits(*args, int(num_splits), _stream(dev)))
    return out, lse


def fwd_f32(q, k, v, scale=None, causal=False, block_n=0, out=None, lse=None, rescale=True):
    """fp32 forward with the key-block size `block_n` (0 = default).
    rescale=False calls attn_fwd_f32_unrescaled (the chunk-wise mode without
    a running max: a negative control that overflows for large scores)."""
    lib = load()
    B, H, Tq, Tk, d, dv = _dims(q, k, v)
    _shapes(out=(out, (B, H, Tq, dv)), lse=(lse, (B, H, Tq)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, H, Tq, dv), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.float32, dev, (B, H, Tq, dv))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    fn = "attn_fwd_f32" if rescale else "attn_fwd_f32_unrescaled"
    rc = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Tq, Tk, d, dv, float(scale),
                          int(bool(causal)), int(block_n), _stream(dev))
    _check(fn, rc)
    return out, lse


def bwd_f32(q, k, v, o, lse, dout, scale=None, causal=False):
    """fp32 backward: returns (dq, dk, dv)."""
    lib = load()
    B, H, Tq, Tk, d, dvd = _dims(q, k, v)
    _shapes(o=(o, (B, H, Tq, dvd)), dout=(dout, (B, H, Tq, dvd)), lse=(lse, (B, H, Tq)))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.float32, dev)
    _need(o, "o", torch.float32, dev, (B, H, Tq, dvd))
    _need(dout, "dout", torch.float32, dev, (B, H, Tq, dvd))
    _need(lse, "lse", torch.float32, dev, (B, H, Tq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rc = lib.attn_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                          B, H, Tq, Tk, d, dvd, float(scale), int(bool(causal)), _stream(dev))
    _check("attn_bwd_f32", rc)
    return dq, dk, dv


def profile_start() -> None:
    """Start recording HIP events around every kernel the library launches."""
    _check("attn_profile_start", load().attn_profile_start())


def profile_stop() -> None:
    _check("attn_profile_stop", load().attn_profile_stop())


def profile_query(kind: int):
    """(total_ms, launches) of the kernels of `kind` recorded since profile_start()."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int(0)
    _check("attn_profile_query", load().attn_profile_query(int(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
