"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws and lays out numbers; it holds none of the attention
arithmetic.  Every (workload, tensor, batch, head) slice comes from its own
numpy PCG64 stream seeded by SeedSequence([workload_id, tensor_id, b, h]), so
one head can be regenerated alone (the CPU checks of large workloads use that).
Values are drawn as float32 normals and, for bf16 workloads, rounded to
bfloat16 with round-to-nearest-even; the checks then use the exact float64
values of those rounded numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, mask, dtype and input distribution."""

    name: str
    wid: int
    B: int
    H: int
    Tq: int
    Tk: int
    d: int
    dv: int
    causal: bool
    dtype: str  # "bf16" or "f32"
    sigma: dict = field(default_factory=dict)  # per-tensor std, default 1
    # decode workloads: Tq newest queries against Tk cache slots, sequence b
    # using the first kv_lens(w)[b] of them
    decode: bool = False

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))

    def shape(self, name: str) -> tuple:
        if name == "q":
            return (self.B, self.H, self.Tq, self.d)
        if name == "k":
            return (self.B, self.H, self.Tk, self.d)
        if name == "v":
            return (self.B, self.H, self.Tk, self.dv)
        if name == "do":
            return (self.B, self.H, self.Tq, self.dv)
        raise KeyError(name)


# The five workloads: a tiny fp32 head, a d=64 forward, the d=128 causal
# sequence-8192 forward (the headline), a d=128 causal backward at 4096, and a
# short-query / 65536-key case with wide score range (Q std 2).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_t64_d64", 1, 1, 1, 64, 64, 64, 64, False, "f32"),
        Workload("fwd_bf16_b4h16_t2048_d64", 2, 4, 16, 2048, 2048, 64, 64, False, "bf16"),
        Workload("causal_bf16_b2h32_t8192_d128", 3, 2, 32, 8192, 8192, 128, 128, True, "bf16"),
        Workload("bwd_causal_bf16_b2h16_t4096_d128", 4, 2, 16, 4096, 4096, 128, 128, True, "bf16"),
        Workload("longkv_bf16_b1h64_tq256_tk65536_d128", 5, 1, 64, 256, 65536, 128, 128, False, "bf16",
                 sigma={"q": 2.0}),
        # decode: one new query per sequence against a 32768-slot cache, 8
        # sequences of mixed lengths (kv_lens), 32 heads
        Workload("decode_bf16_b8h32_tk32768_d128", 6, 8, 32, 1, 32768, 128, 128, True, "bf16", decode=True),
        # index range: K and V hold 128 * 131072 * 128 = 2^31 elements each, so
        # element offsets of the last heads pass the int32 range
        Workload("index_bf16_b1h128_tq128_tk131072_d128", 7, 1, 128, 128, 131072, 128, 128, False, "bf16"),
    ]
}


def kv_lens(w: Workload) -> np.ndarray:
    """Cache lengths of a decode workload's sequences (int32 [B]): seeded
    uniform draws in [Tk/8, Tk], the last sequence at the full Tk."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.wid, 99])))
    lens = g.integers(w.Tk // 8, w.Tk, size=w.B, endpoint=True).astype(np.int32)
    lens[-1] = w.Tk
    return lens


def head_normal(wid: int, tensor: str, b: int, h: int, rows: int, cols: int, sigma: float = 1.0) -> np.ndarray:
    """float32 [rows, cols] normal(0, sigma) draws for one head of one tensor."""
    ss = np.random.SeedSequence([wid, TENSOR_IDS[tensor], b, h])
    g = np.random.Generator(np.random.PCG64(ss))
    x = g.standard_normal((rows, cols), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """Round float32 values to bfloat16 (round-to-nearest-even), CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def exact_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a (CPU or device) bf16/f32 tensor."""
    return t.detach().to("cpu", torch.float64).numpy()


def make_tensor(w: Workload, tensor: str, device="cpu", heads=None) -> torch.Tensor:
    """The full [B, H, T, dim] tensor of a workload, built head by head in the
    workload's dtype on `device`.  `heads` optionally restricts generation to a
    list of (b, h) pairs (other heads are left zero)."""
    B, H, T, D = w.shape(tensor)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.zeros((B, H, T, D), dtype=tdt, device=device)
    sig = w.sigma.get(tensor, 1.0)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        x = head_normal(w.wid, tensor, b, h, T, D, sig)
        t = to_bf16(x) if w.dtype == "bf16" else torch.from_numpy(x)
        out[b, h].copy_(t)
    return out


def make_head(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """Exact float64 values of one head of one tensor (same numbers as
    make_tensor produces for that head)."""
    _, _, T, D = w.shape(tensor)
    x = head_normal(w.wid, tensor, b, h, T, D, w.sigma.get(tensor, 1.0))
    if w.dtype == "bf16":
        return exact_f64(to_bf16(x))
    return x.astype(np.float64)


def random_problem(seed: int, B: int, H: int, Tq: int, Tk: int, d: int, dv: int, dtype: str = "f32",
                   sigma_q: float = 1.0):
    """Small seeded problem (q, k, v, do) as CPU tensors of `dtype` for the
    parity tests at odd shapes."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + seed, B, H, Tq, Tk, d, dv])))
    q = g.standard_normal((B, H, Tq, d), dtype=np.float32) * np.float32(sigma_q)
    k = g.standard_normal((B, H, Tk, d), dtype=np.float32)
    v = g.standard_normal((B, H, Tk, dv), dtype=np.float32)
    do = g.standard_normal((B, H, Tq, dv), dtype=np.float32)
    conv = to_bf16 if dtype == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)))
    return conv(q), conv(k), conv(v), conv(do)


def adversarial_problem(seed: int, Tq: int, Tk: int, d: int, dv: int, split: int, high_first: bool,
                        alpha: float = 100.0, separated: bool = True):
    """fp32 single-head problem whose scores jump between key blocks.

    Column 0 of K is +100 on keys [0, split) and -100 on keys [split, 2*split)
    (the pattern repeats every 2*split keys; swapped when high_first is
    False), and column 0 of Q is alpha*(|q0| + 1), so with scale 1/sqrt(d) the
    scores sit above +1000 in one block and below -1000 in the next.

    separated=True: only column 0 of Q is scaled, and the first key of every
    block gets +10 more in column 0, so each block has one key whose score
    leads the others by at least 125 and the softmax of every row is decided
    by a single key (an fp32 score near 1250 carries about 6e-5 of rounding,
    which a mix of near-tied keys would pass on to the output).
    separated=False: all of Q is multiplied by alpha, leaving about +-100 of
    noise between the keys of a block (near ties occur)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2000 + seed, Tq, Tk, d, dv, split])))
    q = g.standard_normal((Tq, d), dtype=np.float32)
    k = g.standard_normal((Tk, d), dtype=np.float32)
    v = g.standard_normal((Tk, dv), dtype=np.float32)
    do = g.standard_normal((Tq, dv), dtype=np.float32)
    q[:, 0] = np.abs(q[:, 0]) + 1.0
    if separated:
        q[:, 0] *= np.float32(alpha)
    else:
        q *= np.float32(alpha)
    idx = np.arange(Tk)
    hi = (idx // split) % 2 == 0
    if not high_first:
        hi = ~hi
    k[:, 0] = np.where(hi, 100.0, -100.0).astype(np.float32)
    if separated:
        k[idx % split == 0, 0] += np.float32(10.0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).reshape((1, 1) + a.shape)
    return t(q), t(k), t(v), t(do)
