"""Calls on separate HIP streams and around synchronisations.

The C ABI only enqueues work on the caller's stream and takes its workspace
stream-ordered from the library's own memory pool (include/attn.h, "Stream"
and "Workspace"): calls on different streams may overlap, and memory freed by
one call is handed to the next only in stream order.  Each check runs the same
calls once on the current stream, one after the other, and again overlapped on
two side streams or with a synchronisation after every call, and requires
bit-identical outputs.  Every kernel sums each output element in a fixed
order, so any difference would come from two calls sharing memory they should
not.  The shapes are chosen so that every call takes a workspace: the forward
and decode with key-range splits, the backward with a key-split dQ (few query
blocks against many keys), whose fp32 partials are the largest workspace.
"""
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import random_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


def _problem(seed, dev, B=1, H=6, Tq=96, Tk=6000, d=128):
    return [t.to(dev) for t in random_problem(seed, B, H, Tq, Tk, d, d, "bf16")]


def _fwd_bwd(q, k, v, do, causal):
    o, lse = attn.fwd(q, k, v, causal=causal, num_splits=3)
    o1, lse1 = attn.fwd(q, k, v, causal=causal)
    dq, dk, dv = attn.bwd(q, k, v, o1, lse1, do, causal=causal)
    return [o, lse, o1, lse1, dq, dk, dv]


def _decode(qd, k, v, lens):
    return list(attn.decode(qd, k, v, kv_lens=lens, num_splits=4))


def _bits(ts):
    return [t.clone() for t in ts]


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def test_overlapped_streams_match_sequential(dev):
    pa = _problem(1, dev)
    pb = _problem(2, dev, H=4, Tq=64, Tk=9000)
    lens = torch.tensor([5000], dtype=torch.int32, device=dev)
    qd = pa[0][:, :, :2].contiguous()  # two newest queries per head for decode
    ref_a = _bits(_fwd_bwd(*pa, causal=False))
    ref_b = _bits(_fwd_bwd(*pb, causal=True))
    ref_d = _bits(_decode(qd, pa[1], pa[2], lens))
    torch.cuda.synchronize()

    main = torch.cuda.current_stream(dev)
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)  # default priority
    s1.wait_stream(main)
    s2.wait_stream(main)
    outs = {}
    for rep in range(3):
        with torch.cuda.stream(s1):
            outs[("a", rep)] = _fwd_bwd(*pa, causal=False)
            outs[("d", rep)] = _decode(qd, pa[1], pa[2], lens)
        with torch.cuda.stream(s2):
            outs[("b", rep)] = _fwd_bwd(*pb, causal=True)
    main.wait_stream(s1)
    main.wait_stream(s2)
    torch.cuda.synchronize()
    for rep in range(3):
        _same(outs[("a", rep)], ref_a)
        _same(outs[("b", rep)], ref_b)
        _same(outs[("d", rep)], ref_d)


def test_synchronised_calls_match(dev):
    p = _problem(3, dev)
    ref = _bits(_fwd_bwd(*p, causal=True))
    for _ in range(3):
        torch.cuda.synchronize()
        _same(_fwd_bwd(*p, causal=True), ref)
    torch.cuda.synchronize()
