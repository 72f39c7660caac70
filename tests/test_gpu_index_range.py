"""GPU parity with more than 2^31 elements in one tensor.

K, V, dK and dV of the index-range workload hold 2^31 elements each, so any
32-bit element offset in the kernels would wrap on the last heads.
"""
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import WORKLOADS, exact_f64, make_head, make_tensor
from oracle import dense_backward, dense_forward
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL = 2e-2
TOL_LSE = 1e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


def test_more_than_2_31_elements_per_tensor(dev):
    """K, V, dK and dV of 2^31 elements each (4 GiB in bf16): head 127 starts
    at element 127 * 2^24 and its last keys lie past element 2^31 - 1, so any
    32-bit element offset would wrap.  Heads 0 and 127 carry their seeded
    values (the others stay zero) and are checked whole against the oracle;
    every output must be finite."""
    w = WORKLOADS["index_bf16_b1h128_tq128_tk131072_d128"]
    heads = [(0, 0), (0, w.H - 1)]
    print(f"[index] {w.name}: generating heads {heads}", flush=True)
    t = {n: make_tensor(w, n, device=dev, heads=heads) for n in ("q", "k", "v", "do")}
    assert t["k"].numel() >= 2 ** 31 and t["v"].numel() >= 2 ** 31
    print(f"[index] {w.name}: attn_fwd + attn_bwd", flush=True)
    o, lse = attn.fwd(t["q"], t["k"], t["v"], scale=w.scale, causal=w.causal)
    dq, dk, dv = attn.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    for x in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(x.float() if x.dtype != torch.float32 else x).all())
    for b, h in heads:
        q, k, v, do = (make_head(w, n, b, h) for n in ("q", "k", "v", "do"))
        ro, rl = dense_forward(q, k, v, w.scale, w.causal)
        assert_close(f"O[{b},{h}]", exact_f64(o[b, h]), ro, TOL)
        assert_close(f"LSE[{b},{h}]", exact_f64(lse[b, h]), rl, TOL_LSE)
        rq, rk, rv = dense_backward(q, k, v, do, w.scale, w.causal)
        assert_close(f"dQ[{b},{h}]", exact_f64(dq[b, h]), rq, TOL)
        assert_close(f"dK[{b},{h}]", exact_f64(dk[b, h]), rk, TOL)
        assert_close(f"dV[{b},{h}]", exact_f64(dv[b, h]), rv, TOL)
