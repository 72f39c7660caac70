"""GPU parity of the key-range state entry points (attn_fwd_state,
attn_merge_states) and of the backward with an upstream LSE gradient
(attn_bwd_dlse), through the C ABI, against the float64 oracle.

The state of a key range is (m, l, acc); merging the states of disjoint key
ranges by rescaling to the common max gives attention over their union ("The
Hidden Recurrence in Softmax Attention", section "Chunk-wise Mode with Online
Softmax Re-scale").  The library keeps a lazy reference max, so m itself is
only checked to lie within 8 ln 2 below the exact row max; acc / l and
m + ln l do not depend on the reference and are compared with the oracle's.

Tolerances as for the other bf16 entry points: 2e-2 on O, acc / l, dQ, dK, dV;
1e-2 on LSE and m + ln l.
"""
import math

import numpy as np
import pytest
import torch

from exact_tiled_softmax_amd import attn
from exact_tiled_softmax_amd.inputs import exact_f64, random_problem
from oracle import attention_state, dense_backward, dense_forward, merge_states
from tests._util import assert_close

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_LSE_BF16 = 1e-2
LAZY_MAX_GAP = 8 * math.log(2.0)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    attn.load()
    return torch.device("cuda:0")


def f64(t):
    return exact_f64(t)


def check_state(name, got, ref):
    """Compare one key range's state from the GPU with the oracle's exact one."""
    acc, m, l = (f64(x) for x in got)
    rm, rl, racc = ref
    empty = rl == 0
    assert np.array_equal(np.isneginf(m), empty), f"{name}: rows without an allowed key"
    assert np.all(l[empty] == 0) and np.all(acc[empty] == 0), f"{name}: empty rows must be zero"
    live = ~empty
    if not np.any(live):
        return
    # lazy reference: not above the row max, at most 8 ln 2 below it (plus fp32 score rounding)
    slack = 1e-3 * (1 + np.abs(rm[live]))
    assert np.all(m[live] <= rm[live] + slack), f"{name}: reference above the row max"
    assert np.all(m[live] >= rm[live] - LAZY_MAX_GAP - slack), f"{name}: reference too far below the row max"
    assert_close(f"{name} acc/l", acc[live] / l[live][:, None], racc[live] / rl[live][:, None], TOL_BF16)
    assert_close(f"{name} m+ln l", m[live] + np.log(l[live]), rm[live] + np.log(rl[live]), TOL_LSE_BF16)


def shard_problem(seed, B, H, T, d, q_off, Tq, sigma_q=1.0):
    """Full-length Q, K, V of T positions and the query shard [q_off, q_off + Tq)."""
    q, k, v, _ = random_problem(seed, B, H, T, T, d, d, "bf16", sigma_q=sigma_q)
    return q, k, v, q[:, :, q_off:q_off + Tq].contiguous()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 130, 390, 700), (0, 64, 128, 300, 301, 700)])
def test_bf16_key_range_states_merge_to_full_attention(dev, d, causal, cuts):
    B, H, T, q_off, Tq = 1, 2, cuts[-1], 350, 300
    qfull, k, v, q = shard_problem(11, B, H, T, d, q_off, Tq, sigma_q=1.5)
    scale = 1 / math.sqrt(d)
    qd = q.to(dev)
    states, refs = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        kc, vc = k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous()
        states.append(attn.fwd_state(qd, kc.to(dev), vc.to(dev), causal=causal, q_offset=q_off, k_offset=a))
        refs.append(attention_state(f64(q), f64(kc), f64(vc), scale, causal, q_offset=q_off, k_offset=a))
    acc = torch.stack([s[0] for s in states])
    m = torch.stack([s[1] for s in states])
    l = torch.stack([s[2] for s in states])
    o, lse = attn.merge_states(acc, m, l)
    torch.cuda.synchronize()
    for i, (got, ref) in enumerate(zip(states, refs)):
        bh = lambda x: x.reshape((B * H,) + x.shape[2:])
        for h in range(B * H):
            check_state(f"range {i} head {h}", tuple(bh(x)[h] for x in got), tuple(bh(x)[h] for x in ref))
    ro, rl = dense_forward(f64(qfull), f64(k), f64(v), scale, causal)
    assert_close("O", f64(o), ro[:, :, q_off:q_off + Tq], TOL_BF16)
    assert_close("LSE", f64(lse), rl[:, :, q_off:q_off + Tq], TOL_LSE_BF16)
    # the oracle's own merge of its exact states agrees with its dense forward
    mo, ml = merge_states([r[0] for r in refs], [r[1] for r in refs], [r[2] for r in refs])
    assert np.allclose(mo, ro[:, :, q_off:q_off + Tq], atol=1e-12)


def test_bf16_state_of_a_range_after_every_query_is_empty(dev):
    B, H, T, d = 1, 1, 400, 128
    _, k, v, q = shard_problem(12, B, H, T, d, 0, 100)
    acc, m, l = attn.fwd_state(q.to(dev), k[:, :, 200:].contiguous().to(dev), v[:, :, 200:].contiguous().to(dev),
                               causal=True, q_offset=0, k_offset=200)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(m)) and torch.all(l == 0) and torch.all(acc == 0)
    o, lse = attn.merge_states(acc[None], m[None], l[None])
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_bf16_single_state_merge_matches_forward(dev):
    """One state spanning all keys, merged alone, is the forward itself."""
    q, k, v, _ = random_problem(13, 2, 2, 333, 515, 128, 128, "bf16")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    acc, m, l = attn.fwd_state(qd, kd, vd, causal=True)
    o, lse = attn.merge_states(acc[None], m[None], l[None])
    fo, flse = attn.fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    # same arithmetic up to where the final log is taken: O within one bf16 step
    assert torch.allclose(o.float(), fo.float(), rtol=2.0**-7, atol=1e-6)
    assert torch.allclose(lse, flse, rtol=0, atol=1e-5)
    ro, rl = dense_forward(f64(q), f64(k), f64(v), 1 / math.sqrt(128), True)
    assert_close("O", f64(o), ro, TOL_BF16)
    assert_close("LSE", f64(lse), rl, TOL_LSE_BF16)


@pytest.mark.parametrize("shape", [(1, 2, 300, 333, 128, 128), (2, 1, 513, 257, 64, 64), (1, 1, 1, 300, 128, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_bwd_with_lse_gradient(dev, shape, causal):
    B, H, Tq, Tk, d, dv = shape
    q, k, v, do = random_problem(14, B, H, Tq, Tk, d, dv, "bf16")
    dlse = torch.from_numpy(np.random.default_rng(15).standard_normal((B, H, Tq)).astype(np.float32))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn.fwd(qd, kd, vd, causal=causal)
    dq, dk, dvv = attn.bwd(qd, kd, vd, o, lse, dod, causal=causal, dlse=dlse.to(dev))
    torch.cuda.synchronize()
    rq, rk, rv = dense_backward(f64(q), f64(k), f64(v), f64(do), 1 / math.sqrt(d), causal, dlse=dlse.double().numpy())
    assert_close("dQ", f64(dq), rq, TOL_BF16)
    assert_close("dK", f64(dk), rk, TOL_BF16)
    assert_close("dV", f64(dvv), rv, TOL_BF16)


def test_bf16_bwd_zero_lse_gradient_equals_plain_bwd(dev):
    q, k, v, do = random_problem(16, 1, 2, 300, 333, 128, 128, "bf16")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn.fwd(qd, kd, vd, causal=True)
    g0 = attn.bwd(qd, kd, vd, o, lse, dod, causal=True)
    g1 = attn.bwd(qd, kd, vd, o, lse, dod, causal=True, dlse=torch.zeros_like(lse))
    torch.cuda.synchronize()
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bf16_states_written_into_stacked_buffers(dev):
    """fwd_state writing into slices of one stacked buffer, and merge_states
    writing into caller buffers, give bit-for-bit what the allocating calls
    give (the form the benchmark's key-range path uses)."""
    cuts = (0, 200, 333, 515)
    q, k, v, _ = random_problem(14, 1, 3, 300, 515, 128, 128, "bf16")
    qd = q.to(dev)
    ks = [k[:, :, a:b].contiguous().to(dev) for a, b in zip(cuts[:-1], cuts[1:])]
    vs = [v[:, :, a:b].contiguous().to(dev) for a, b in zip(cuts[:-1], cuts[1:])]
    n = len(ks)
    acc = torch.full((n, 1, 3, 300, 128), float("nan"), dtype=torch.float32, device=dev)
    m = torch.full((n, 1, 3, 300), float("nan"), dtype=torch.float32, device=dev)
    l = torch.full_like(m, float("nan"))
    sep = []
    for j, a in enumerate(cuts[:-1]):
        attn.fwd_state(qd, ks[j], vs[j], causal=True, k_offset=a, acc=acc[j], m=m[j], l=l[j])
        sep.append(attn.fwd_state(qd, ks[j], vs[j], causal=True, k_offset=a))
    o = torch.empty((1, 3, 300, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, 3, 300), dtype=torch.float32, device=dev)
    attn.merge_states(acc, m, l, out=o, lse=lse)
    o2, lse2 = attn.merge_states(torch.stack([s[0] for s in sep]), torch.stack([s[1] for s in sep]),
                                 torch.stack([s[2] for s in sep]))
    torch.cuda.synchronize()
    for j in range(n):
        assert torch.equal(acc[j], sep[j][0]) and torch.equal(m[j], sep[j][1]) and torch.equal(l[j], sep[j][2])
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    ro, rl = dense_forward(f64(q), f64(k), f64(v), 1 / math.sqrt(128), True)
    assert_close("O", f64(o), ro, TOL_BF16)
    assert_close("LSE", f64(lse), rl, TOL_LSE_BF16)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_state_of_a_long_range_computed_in_splits(dev, d):
    """Few queries against a long key range without the mask: the call splits
    the range inside (as the forward does) and merges the split states into
    one state, which must still be the exact state of the whole range."""
    B, H, Tq, Tk = 1, 2, 100, 4200
    q, k, v, _ = random_problem(15, B, H, Tq, Tk, d, d, "bf16", sigma_q=1.5)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    acc, m, l = attn.fwd_state(qd, kd, vd, causal=False)
    o, lse = attn.merge_states(acc[None], m[None], l[None])
    torch.cuda.synchronize()
    ref = attention_state(f64(q), f64(k), f64(v), scale, False)
    bh = lambda x: x.reshape((B * H,) + x.shape[2:])
    for h in range(B * H):
        check_state(f"head {h}", tuple(bh(x)[h] for x in (acc, m, l)), tuple(bh(x)[h] for x in ref))
    ro, rl = dense_forward(f64(q), f64(k), f64(v), scale, False)
    assert_close("O", f64(o), ro, TOL_BF16)
    assert_close("LSE", f64(lse), rl, TOL_LSE_BF16)
