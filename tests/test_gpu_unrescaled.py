"""GPU check of the negative control attn_fwd_f32_unrescaled (the chunk-wise
mode of "The Hidden Recurrence in Softmax Attention" before the rescale)
against the float64 oracle's chunkwise_unrescaled, through the C ABI.

For modest scores the un-rescaled mode is exact (tolerance 1e-5, as for the
other fp32 entry points).  Past about 88.7 fp32 exp overflows: the rows whose
largest score exceeds that come out inf or nan, while attn_fwd_f32 (the
online softmax with its running max) stays finite and correct on the very
same input.
"""
import math

import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import adversarial_problem, exact_f64, random_problem
from oracle import chunkwise_unrescaled, dense_forward
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
FP32_EXP_LIMIT = math.log(np.finfo(np.float32).max)  # about 88.72


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_n", [1, 7, 64, 128])
def test_unrescaled_matches_oracle_for_modest_scores(dev, causal, block_n):
    q, k, v, _ = random_problem(31, 1, 2, 70, 150, 64, 48, "f32")
    o, lse = attn.fwd_f32(q.to(dev), k.to(dev), v.to(dev), causal=causal, block_n=block_n, rescale=False)
    torch.cuda.synchronize()
    o, lse = exact_f64(o), exact_f64(lse)
    for h in range(2):
        ro, rl = chunkwise_unrescaled(exact_f64(q)[0, h], exact_f64(k)[0, h], exact_f64(v)[0, h], block_n,
                                      1 / 8.0, causal)
        assert_close("O", o[0, h], ro, TOL_F32)
        assert_close("LSE", lse[0, h], rl, TOL_F32)
    ro, rl = dense_forward(exact_f64(q), exact_f64(k), exact_f64(v), 1 / 8.0, causal)
    assert_close("O vs dense", o, ro, TOL_F32)


@pytest.mark.parametrize("causal", [False, True])
def test_unrescaled_overflows_where_the_online_softmax_does_not(dev, causal):
    """The adversarial input (scores above +1000 on some key blocks): rows whose
    largest allowed score passes the fp32 exp range turn non-finite in the
    un-rescaled mode, every row of the rescaled forward stays finite and
    matches the oracle."""
    # one high-score key block (split 128 of 256 keys): its top key leads every row
    q, k, v, _ = adversarial_problem(0, 64, 256, 64, 64, 128, True)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    bad_o, bad_lse = attn.fwd_f32(qd, kd, vd, scale=1 / 8.0, causal=causal, block_n=64, rescale=False)
    good_o, good_lse = attn.fwd_f32(qd, kd, vd, scale=1 / 8.0, causal=causal, block_n=64)
    torch.cuda.synchronize()
    s = exact_f64(q)[0, 0] @ exact_f64(k)[0, 0].T / 8.0
    if causal:
        s = np.where(np.arange(256)[None, :] > np.arange(64)[:, None], -np.inf, s)
    overflow_rows = s.max(axis=1) > FP32_EXP_LIMIT + 1.0
    safe_rows = s.max(axis=1) < FP32_EXP_LIMIT - 1.0
    assert overflow_rows.any()
    bad = exact_f64(bad_o)[0, 0]
    assert np.all(~np.isfinite(bad[overflow_rows]).all(axis=1))
    assert np.all(~np.isfinite(exact_f64(bad_lse)[0, 0][overflow_rows]))
    ro, rl = dense_forward(exact_f64(q), exact_f64(k), exact_f64(v), 1 / 8.0, causal)
    assert np.all(np.isfinite(exact_f64(good_o))) and np.all(np.isfinite(exact_f64(good_lse)))
    assert_close("O (rescaled)", exact_f64(good_o), ro, TOL_F32)
    assert_close("LSE (rescaled)", exact_f64(good_lse), rl, TOL_F32)
    if safe_rows.any():
        assert_close("O (un-rescaled, safe rows)", bad[safe_rows], ro[0, 0][safe_rows], TOL_F32)


def test_unrescaled_threshold(dev):
    """One key scored just under the fp32 exp limit stays finite; just over it
    overflows (single key, so the row sum is that one exponential)."""
    d = 64
    for target, finite in ((86.0, True), (90.0, False)):
        q = torch.zeros((1, 1, 1, d), dtype=torch.float32)
        k = torch.zeros((1, 1, 1, d), dtype=torch.float32)
        q[..., 0] = target
        k[..., 0] = 1.0
        v = torch.ones((1, 1, 1, d), dtype=torch.float32)
        o, lse = attn.fwd_f32(q.to(dev), k.to(dev), v.to(dev), scale=1.0, rescale=False)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o).all()) == finite
        if finite:
            assert abs(float(lse) - target) < 1e-4 and torch.allclose(o.cpu(), v)
