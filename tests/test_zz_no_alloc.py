"""attn_bwd_noalloc (the backward whose workspace is the library's static
scratch array) against attn_bwd on the same inputs, through the C ABI: two
calls in a row on one GPU, the second with a smaller input, each checked to
the bf16 tolerance (2e-2 on dQ, dK, dV) and, since both entry points take the
same key-range split plan at these sizes, for identical bits.  The first call
splits the dQ key range (fp32 partials in the scratch); the second does not.
"""
import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import exact_f64, random_problem
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


def run_both(dev, shape, causal, seed):
    B, H, Tq, Tk, d, dv = shape
    print(f"[noalloc] shape {shape} causal={causal} seed={seed}", flush=True)
    q, k, v, do = (t.to(dev) for t in random_problem(seed, B, H, Tq, Tk, d, dv, "bf16"))
    o, lse = attn.fwd(q, k, v, causal=causal)
    ref = attn.bwd(q, k, v, o, lse, do, causal=causal)
    got = attn.bwd(q, k, v, o, lse, do, causal=causal, noalloc=True)
    torch.cuda.synchronize()
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(name, exact_f64(x), exact_f64(r), TOL_BF16)
        assert torch.equal(x.view(torch.int16), r.view(torch.int16)), f"{name} differs from attn_bwd"


def test_noalloc_two_calls_second_smaller(dev):
    # few query blocks, many keys: the dQ kernel splits its key range and keeps
    # fp32 partials in the scratch
    run_both(dev, (1, 2, 130, 3000, 128, 128), False, 21)
    # a smaller problem on the same scratch, which still holds the first
    # call's partials
    run_both(dev, (1, 1, 100, 200, 64, 64), True, 22)


def test_noalloc_refuses_too_large_before_any_launch(dev):
    # row statistics alone would exceed the scratch: refused, nothing launched
    nz = 16
    lib = attn.load()
    rc = lib.attn_bwd_noalloc(nz, nz, nz, nz, nz, nz, nz, nz, nz, 1, 129, 65536, 64, 128, 128, 0.088, 1, None)
    assert rc == attn.ATTN_ERR_TOO_LARGE
