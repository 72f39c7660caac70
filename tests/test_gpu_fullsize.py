"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (attn_fwd then attn_bwd through the C ABI, default split choice).

The oracle cannot run the whole workloads in seconds, so it checks sampled
outputs of whole heads: O and LSE rows, dQ rows (each needs only its own score
row) and dK/dV rows of sampled keys (each needs that key's column of P, formed
from complete rows chunk by chunk).  Besides the element-wise tolerance, every
sampled row with at least 64 contributing terms must match as a row: its
largest error at most 0.06 of the row's RMS (the magnitude-aware bound derived
in tests/_bounds.py), and LSE must match to 1e-4 absolute; a row that is off
by a constant factor of 10% fails either check even where most of its
elements are smaller than the absolute tolerance.  Properties that hold at any size are
checked on every head: sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 (every row of
dS sums to zero), and all outputs finite.
"""
import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import WORKLOADS, exact_f64, make_head, make_tensor
from oracle import backward_dkdv_cols, backward_dq_rows, forward_rows
from tests._bounds import LSE_ABS_BOUND, assert_rows_match
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_LSE = 1e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


def sample_idx(n, extra_seed):
    g = np.random.Generator(np.random.PCG64(extra_seed))
    fixed = [0, 1, 63, 64, 255, 256, n // 2, n - 2, n - 1]
    rnd = g.choice(n, size=min(n, 23), replace=False)
    return np.unique(np.clip(np.concatenate([fixed, rnd]), 0, n - 1))


def run_workload(w, dev, with_bwd):
    print(f"[fullsize] {w.name}: generating inputs", flush=True)
    names = ("q", "k", "v", "do") if with_bwd else ("q", "k", "v")
    t = {n: make_tensor(w, n).to(dev) for n in names}
    print(f"[fullsize] {w.name}: attn_fwd" + (" + attn_bwd" if with_bwd else ""), flush=True)
    o, lse = attn.fwd(t["q"], t["k"], t["v"], scale=w.scale, causal=w.causal)
    grads = None
    if with_bwd:
        grads = attn.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    return t, o, lse, grads


def check_heads(w, o, lse, grads, heads, seed):
    for b, h in heads:
        q, k, v = (make_head(w, n, b, h) for n in ("q", "k", "v"))
        rows = sample_idx(w.Tq, seed + 17 * h + b)
        ro, rl = forward_rows(q, k, v, rows, w.scale, w.causal)
        xo, xl = exact_f64(o[b, h])[rows], exact_f64(lse[b, h])[rows]
        assert_close(f"O[{b},{h}]", xo, ro, TOL)
        assert_close(f"LSE[{b},{h}]", xl, rl, TOL_LSE)
        assert np.max(np.abs(xl - rl)) <= LSE_ABS_BOUND, f"LSE[{b},{h}]: max abs err {np.max(np.abs(xl - rl)):.2e}"
        # rows that see at least 64 keys (causal: query index >= 63)
        many = rows >= 63 if w.causal else np.ones(len(rows), bool)
        assert_rows_match(f"O[{b},{h}] rows", xo[many], ro[many])
        if grads is None:
            continue
        do = make_head(w, "do", b, h)
        dq, dk, dv = grads
        rq = backward_dq_rows(q, k, v, do, rows, w.scale, w.causal)
        xq = exact_f64(dq[b, h])[rows]
        assert_close(f"dQ[{b},{h}]", xq, rq, TOL)
        assert_rows_match(f"dQ[{b},{h}] rows", xq[many], rq[many])
        cols = sample_idx(w.Tk, seed + 31 * h + b + 5)
        rk, rv = backward_dkdv_cols(q, k, v, do, cols, w.scale, w.causal)
        xk, xv = exact_f64(dk[b, h])[cols], exact_f64(dv[b, h])[cols]
        assert_close(f"dK[{b},{h}]", xk, rk, TOL)
        assert_close(f"dV[{b},{h}]", xv, rv, TOL)
        # keys seen by at least 64 queries (causal: key index <= Tq - 64)
        kmany = cols <= w.Tq - 64 if w.causal else np.ones(len(cols), bool)
        assert_rows_match(f"dK[{b},{h}] rows", xk[kmany], rk[kmany])
        assert_rows_match(f"dV[{b},{h}] rows", xv[kmany], rv[kmany])


def check_properties(t, o, lse, grads):
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    if grads is None:
        return
    dq, dk, dv = grads
    for g in grads:
        assert torch.isfinite(g.float()).all()
    sdv = dv.double().sum(dim=2)
    sdo = t["do"].double().sum(dim=2)
    scale_v = dv.double().abs().sum(dim=2) + 1.0
    assert ((sdv - sdo).abs() <= 1e-2 * scale_v).all(), float(((sdv - sdo).abs() / scale_v).max())
    sdk = dk.double().sum(dim=2)
    scale_k = dk.double().abs().sum(dim=2) + 1.0
    assert (sdk.abs() <= 1e-2 * scale_k).all(), float((sdk.abs() / scale_k).max())


def test_fwd_d64_t2048(dev):
    w = WORKLOADS["fwd_bf16_b4h16_t2048_d64"]
    t, o, lse, _ = run_workload(w, dev, with_bwd=False)
    check_properties(t, o, lse, None)
    check_heads(w, o, lse, None, [(0, 0), (3, 15)], 100)


def test_causal_d128_t8192_fwd_bwd(dev):
    w = WORKLOADS["causal_bf16_b2h32_t8192_d128"]
    t, o, lse, grads = run_workload(w, dev, with_bwd=True)
    check_properties(t, o, lse, grads)
    check_heads(w, o, lse, grads, [(0, 0), (1, 31)], 200)


def test_bwd_causal_d128_t4096(dev):
    w = WORKLOADS["bwd_causal_bf16_b2h16_t4096_d128"]
    t, o, lse, grads = run_workload(w, dev, with_bwd=True)
    check_properties(t, o, lse, grads)
    check_heads(w, o, lse, grads, [(0, 0), (1, 15)], 300)


def test_longkv_tq256_tk65536(dev):
    w = WORKLOADS["longkv_bf16_b1h64_tq256_tk65536_d128"]
    t, o, lse, grads = run_workload(w, dev, with_bwd=True)
    check_properties(t, o, lse, grads)
    check_heads(w, o, lse, grads, [(0, 0), (0, 63)], 400)

