"""Pins of the bf16 error model used by the large-score parity tests
(tests/_bounds.py), on the CPU.

A float64 emulation of the bf16 path's rounding steps (P rounded to bf16
before P V, O rounded on output, D formed from that O, P and dS rounded to
bf16 before the gradient products, gradients rounded on output; every sum in
float64) is compared with the float64 oracle.  The model must bound the
emulated error (it is an error bound) and must not be vacuous (its sigma is
the size of the errors it models, not orders above them).  A model that drops
the term D inherits from the bf16 O is exceeded at large scores, which is
why the term is there.
"""
import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd.inputs import exact_f64, random_problem
from oracle import causal_blocked, dense_backward
from tests._bounds import N_SIGMA, U_BF16, bf16_backward_parts, bf16_backward_sigma


def bf(x):
    """Round float64 values to bf16 (nearest even) and back."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def emulated_bf16_backward(q, k, v, do, scale, causal):
    s = scale * (q @ k.T)
    if causal:
        s = np.where(causal_blocked(s.shape[0], s.shape[1]), -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = bf((bf(e) @ v) / l)
    p = e / l
    ds = p * (do @ v.T - np.sum(do * o, axis=1, keepdims=True))
    dq = bf(scale * bf(ds) @ k)
    dk = bf(scale * bf(ds).T @ q)
    dv = bf(bf(p).T @ do)
    return dq, dk, dv


CASES = [(seed, sq, causal) for seed in (12, 13) for sq in (1.0, 4.0, 8.0) for causal in (False, True)]


@pytest.mark.parametrize("seed,sigma_q,causal", CASES)
def test_model_bounds_the_emulated_bf16_backward(seed, sigma_q, causal):
    q, k, v, do = (exact_f64(t)[0, 0] for t in random_problem(seed, 1, 1, 200, 300, 128, 128, "bf16",
                                                               sigma_q=sigma_q))
    sc = 1 / np.sqrt(128)
    ref = dense_backward(q, k, v, do, sc, causal)
    got = emulated_bf16_backward(q, k, v, do, sc, causal)
    sig = bf16_backward_sigma(q, k, v, do, sc, causal)
    for name, x, r, s in zip(("dQ", "dK", "dV"), got, ref, sig):
        err = np.abs(x - r)
        bound = N_SIGMA * s + U_BF16 * np.abs(r)
        assert np.all(err <= bound), f"{name}: max err/bound {np.max(err / (bound + 1e-300)):.3f}"
        # not vacuous: the errors use a fair share of the modelled spread
        live = s > 0
        ratio = np.sqrt(np.mean(err[live] ** 2)) / np.sqrt(np.mean(s[live] ** 2))
        assert 0.2 < ratio < 2.0, f"{name}: rms(err)/rms(sigma) = {ratio:.3f}"


def test_dropping_the_d_term_is_exceeded_at_large_scores():
    q, k, v, do = (exact_f64(t)[0, 0] for t in random_problem(12, 1, 1, 300, 700, 128, 128, "bf16", sigma_q=8.0))
    sc = 1 / np.sqrt(128)
    ref = dense_backward(q, k, v, do, sc, False)
    got = emulated_bf16_backward(q, k, v, do, sc, False)
    u2 = U_BF16 ** 2 / 3
    p, o, ds = bf16_backward_parts(q, k, v, do, sc, False)
    s_dk_no_d = np.sqrt(sc ** 2 * u2 * (ds ** 2).T @ (q ** 2))
    err = np.abs(got[1] - ref[1])
    assert np.any(err > N_SIGMA * s_dk_no_d + U_BF16 * np.abs(ref[1]))
    # and the stated bf16 tolerance alone does not hold there either
    assert np.any((err > 2e-2) & (err > 2e-2 * np.abs(ref[1])))


def test_parts_match_the_oracle_gradients():
    # the model's P and dS give the oracle's gradients back
    q, k, v, do = (exact_f64(t)[0, 0] for t in random_problem(3, 1, 1, 50, 70, 16, 16, "bf16", sigma_q=3.0))
    sc = 0.3
    for causal in (False, True):
        p, o, ds = bf16_backward_parts(q, k, v, do, sc, causal)
        rq, rk, rv = dense_backward(q, k, v, do, sc, causal)
        np.testing.assert_allclose(sc * ds @ k, rq, atol=1e-12)
        np.testing.assert_allclose(sc * ds.T @ q, rk, atol=1e-12)
        np.testing.assert_allclose(p.T @ do, rv, atol=1e-12)
