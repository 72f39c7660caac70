"""GPU parity of attn_decode (the newest Tq <= 4 queries of each sequence
against its key/value cache) through the C ABI, against the float64 oracle's
decode_forward.

Cache slots at and past each sequence's length are filled with NaN: the
library must never read them, so every output must stay finite.

Tolerances as for the other bf16 entry points: 2e-2 on O, 1e-2 on LSE.
"""
import math

import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import WORKLOADS, exact_f64, kv_lens, make_head, make_tensor, random_problem
from oracle import decode_forward
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_LSE_BF16 = 1e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


def f64(t):
    return exact_f64(t)


def poisoned_cache(k, v, lens):
    """Copies of k, v with NaN in every slot at or past each sequence's length."""
    kp, vp = k.clone(), v.clone()
    for b, n in enumerate(lens):
        kp[b, :, n:] = float("nan")
        vp[b, :, n:] = float("nan")
    return kp, vp


def run_decode(dev, q, k, v, lens, causal, num_splits=None, scale=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
    o, lse = attn.decode(q.to(dev), k.to(dev), v.to(dev), kv_lens=lens_d, causal=causal, num_splits=num_splits,
                         scale=scale)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


def check(o, lse, ro, rl):
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), "rows without an allowed key"
    assert np.all(o[empty] == 0)
    assert np.all(np.isfinite(o))
    assert_close("O", o, ro, TOL_BF16)
    assert_close("LSE", lse[~empty], rl[~empty], TOL_LSE_BF16)


CASES = [
    # B, H, Tq, Tk, d, lens
    (2, 3, 1, 1000, 128, [1000, 377]),
    (3, 2, 1, 700, 64, [700, 1, 64]),
    (2, 2, 2, 513, 128, [513, 2]),
    (2, 2, 3, 300, 128, [300, 200]),
    (2, 1, 4, 257, 64, [257, 129]),
    (1, 1, 1, 1, 128, [1]),
    (4, 2, 4, 4100, 128, [4100, 3, 0, 2049]),  # a sequence shorter than Tq and an empty one
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_decode_matches_oracle(dev, case, causal):
    B, H, Tq, Tk, d, lens = case
    q, k, v, _ = random_problem(21, B, H, Tq, Tk, d, d, "bf16")
    kp, vp = poisoned_cache(k, v, lens)
    o, lse = run_decode(dev, q, kp, vp, lens, causal)
    ro, rl = decode_forward(f64(q), f64(k), f64(v), 1 / math.sqrt(d), kv_lens=lens, causal=causal)
    check(o, lse, ro, rl)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
@pytest.mark.parametrize("tq", [1, 3])
def test_bf16_decode_key_splits(dev, splits, tq):
    B, H, Tk, d = 2, 2, 3000, 128
    lens = [3000, 1111]
    q, k, v, _ = random_problem(22, B, H, tq, Tk, d, d, "bf16", sigma_q=2.0)
    kp, vp = poisoned_cache(k, v, lens)
    o, lse = run_decode(dev, q, kp, vp, lens, True, num_splits=splits)
    ro, rl = decode_forward(f64(q), f64(k), f64(v), 1 / math.sqrt(d), kv_lens=lens, causal=True)
    check(o, lse, ro, rl)


def test_bf16_decode_without_lengths_uses_whole_cache(dev):
    q, k, v, _ = random_problem(23, 2, 4, 2, 777, 64, 64, "bf16")
    o, lse = run_decode(dev, q, k, v, None, True)
    ro, rl = decode_forward(f64(q), f64(k), f64(v), 1 / 8.0, causal=True)
    check(o, lse, ro, rl)


def test_bf16_decode_lengths_out_of_range_are_clamped(dev):
    q, k, v, _ = random_problem(24, 3, 1, 1, 200, 128, 128, "bf16")
    o, lse = run_decode(dev, q, k, v, [-5, 10 ** 9, 50], False)
    ro, rl = decode_forward(f64(q), f64(k), f64(v), 1 / math.sqrt(128), kv_lens=[0, 200, 50])
    check(o, lse, ro, rl)


def test_bf16_decode_scale_zero_and_large_scores(dev):
    q, k, v, _ = random_problem(25, 1, 2, 1, 2000, 128, 128, "bf16")
    o, lse = run_decode(dev, q, k, v, None, False, scale=0.0)
    ro, rl = decode_forward(f64(q), f64(k), f64(v), 0.0)
    check(o, lse, ro, rl)
    # scores spread over hundreds: the lazy reference max has to move many times
    o, lse = run_decode(dev, q * 30, k, v, None, False)
    ro, rl = decode_forward(f64(q * 30), f64(k), f64(v), 1 / math.sqrt(128))
    check(o, lse, ro, rl)


def test_bf16_decode_deterministic(dev):
    q, k, v, _ = random_problem(26, 2, 2, 2, 5000, 128, 128, "bf16")
    lens = torch.tensor([5000, 2500], dtype=torch.int32, device=dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = attn.decode(qd, kd, vd, kv_lens=lens, causal=True)
    o2, l2 = attn.decode(qd, kd, vd, kv_lens=lens, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_bf16_decode_full_size_workload_sampled(dev):
    """The decode benchmark workload (8 sequences of mixed lengths, 32 heads,
    32768 cache slots, d = 128) in the launch configuration the benchmark uses;
    every output row is checked for finiteness, sampled (sequence, head) rows
    against the oracle."""
    w = WORKLOADS["decode_bf16_b8h32_tk32768_d128"]
    lens = kv_lens(w)
    q, k, v = (make_tensor(w, n, device=dev) for n in ("q", "k", "v"))
    o, lse = attn.decode(q, k, v, kv_lens=torch.from_numpy(lens).to(dev), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(o.float())) and torch.all(torch.isfinite(lse))
    rng = np.random.default_rng(7)
    picks = [(b, int(rng.integers(w.H))) for b in range(w.B)] + [(w.B - 1, 0), (0, w.H - 1)]
    for b, h in picks:
        n = int(lens[b])
        qh = make_head(w, "q", b, h)[None, None]
        kh = make_head(w, "k", b, h)[None, None, :n]
        vh = make_head(w, "v", b, h)[None, None, :n]
        ro, rl = decode_forward(qh, kh, vh, w.scale, causal=w.causal)
        assert_close(f"O[{b},{h}]", f64(o[b, h])[None, None], ro, TOL_BF16)
        assert_close(f"LSE[{b},{h}]", f64(lse[b, h])[None, None], rl, TOL_LSE_BF16)
