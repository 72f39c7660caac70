"""GPU parity of attn_fwd_standard (standard attention with the score matrix
materialised in HBM) through the C ABI, against the float64 oracle's dense
forward and against the tiled forward.

Tolerances as for the other bf16 entry points: 2e-2 on O, 1e-2 on LSE.
"""
import math

import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import exact_f64, random_problem
from oracle import dense_forward
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_LSE_BF16 = 1e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


SHAPES = [
    (1, 2, 300, 333, 64, 64),
    (2, 1, 513, 257, 128, 128),
    (1, 2, 200, 700, 128, 128),
    (1, 1, 1, 1, 128, 128),
    (1, 1, 1, 300, 64, 64),
    (1, 1, 300, 1, 64, 64),
    (1, 1, 64, 64, 128, 128),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_standard_matches_oracle(dev, shape, causal):
    B, H, Tq, Tk, d, dv = shape
    q, k, v, _ = random_problem(41, B, H, Tq, Tk, d, dv, "bf16", sigma_q=1.5)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = attn.fwd_standard(qd, kd, vd, causal=causal)
    fo, flse = attn.fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    ro, rl = dense_forward(exact_f64(q), exact_f64(k), exact_f64(v), 1 / math.sqrt(d), causal)
    assert_close("O", exact_f64(o), ro, TOL_BF16)
    assert_close("LSE", exact_f64(lse), rl, TOL_LSE_BF16)
    # the tiled and the materialised forward agree with each other as well
    assert_close("O vs tiled", exact_f64(o), exact_f64(fo), TOL_BF16)
    assert np.max(np.abs(exact_f64(lse) - exact_f64(flse))) < 1e-3


def test_standard_scale_zero(dev):
    q, k, v, _ = random_problem(42, 1, 1, 70, 70, 64, 64, "bf16")
    o, lse = attn.fwd_standard(q.to(dev), k.to(dev), v.to(dev), scale=0.0, causal=True)
    torch.cuda.synchronize()
    ro, rl = dense_forward(exact_f64(q), exact_f64(k), exact_f64(v), 0.0, True)
    assert_close("O", exact_f64(o), ro, TOL_BF16)
    assert_close("LSE", exact_f64(lse), rl, TOL_LSE_BF16)
