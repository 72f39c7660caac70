#!/usr/bin/env python3
"""Benchmark of exact tiled-softmax attention on one MI355X.

Metric: attention TFLOP/s for the forward and for forward+backward, bf16,
d = 128, L = 8192, causal, and the fraction of the dense bf16 MFMA peak.

A step is one pass of the whole hot path over one batch of synthetic input:
attn_fwd (O, LSE) followed by attn_bwd (dQ, dK, dV), on the workload
B=2, H=32, Tq=Tk=8192, d=dv=128, causal, Q/K/V/dO ~ N(0,1) in bf16, scale
1/sqrt(d).  Inputs are resident in HBM before the timed region starts.

Throughput counts algorithmic flops only: with `pairs` the number of unmasked
(query, key) pairs, forward = 2*pairs*(d+dv) (Q K^T and P V) and backward =
2*pairs*(3d+2dv) (Q K^T recomputed, dO V^T, P^T dO, dS K, dS^T Q).

Prints one JSON line.  Also reports the dominant kernel against its roofline
(HIP-event durations recorded by the library on the launch stream) and the
float64 CPU oracle timed on a bounded sample of the same workload.

--workload decode_bf16_b8h32_tk32768_d128 times attn_decode instead (one new
query per sequence against a key/value cache of mixed lengths): the metric is
then HBM GB/s of the algorithmic bytes (every cached key and value row read
once, q read, o and lse written) against the 8 TB/s HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
HEADLINE = "causal_bf16_b2h32_t8192_d128"
BWD_TARGET = "bwd_causal_bf16_b2h16_t4096_d128"  # the causal backward workload reported beside it
# further workloads timed beside the headline: head dim 64 (non-causal) and
# few queries against a long key range
SIDE_TARGETS = ("fwd_bf16_b4h16_t2048_d64", "longkv_bf16_b1h64_tq256_tk65536_d128")
METRIC = "attention TFLOP/s fwd & fwd+bwd, bf16 d=128 L=8192 causal; % of MFMA peak"


def unmasked_pairs(tq: int, tk: int, causal: bool) -> int:
    """(query, key) pairs that are not blocked, per head (causal: key <= query)."""
    if not causal:
        return tq * tk
    n = min(tq, tk)
    # rows 0..n-1 see i+1 keys; rows n..tq-1 see all tk keys
    return n * (n + 1) // 2 + (tq - n) * tk


def kernel_flops(w):
    """Per kernel: (algorithmic flops it carries, flops it executes).  The
    backward's algorithmic flops (Q K^T recomputed, dO V^T, P^T dO, dS K,
    dS^T Q) are split between its two kernels: dK/dV carries Q K^T, dO V^T,
    P^T dO and dS^T Q; dQ carries dS K and executes Q K^T and dO V^T again."""
    pairs = unmasked_pairs(w.Tq, w.Tk, w.causal) * w.B * w.H
    return {
        "fwd": (2 * pairs * (w.d + w.dv), 2 * pairs * (w.d + w.dv)),
        "bwd_dkdv": (2 * pairs * (2 * w.d + 2 * w.dv), 2 * pairs * (2 * w.d + 2 * w.dv)),
        "bwd_dq": (2 * pairs * w.d, 2 * pairs * (2 * w.d + w.dv)),
    }


def work(w):
    pairs = unmasked_pairs(w.Tq, w.Tk, w.causal) * w.B * w.H
    fwd = 2 * pairs * (w.d + w.dv)
    bwd = 2 * pairs * (3 * w.d + 2 * w.dv)
    e = 2  # bf16 bytes
    bh = w.B * w.H
    fwd_bytes = bh * (e * (w.Tq * w.d + w.Tk * w.d + w.Tk * w.dv + w.Tq * w.dv) + 4 * w.Tq)
    bwd_bytes = bh * (e * (2 * w.Tq * w.d + 2 * w.Tk * w.d + 2 * w.Tk * w.dv + 2 * w.Tq * w.dv) + 4 * w.Tq)
    return pairs, fwd, bwd, fwd_bytes, bwd_bytes


def kernel_bytes(w):
    """Algorithmic HBM bytes per launch of each kernel: what it must read
    (every input once) and write (every output once).  The dQ kernel reads
    O and LSE besides its own inputs and writes the row statistics the dK/dV
    kernel reads (8 bytes per query row: -LSE/scale and -D, fp32)."""
    e = 2  # bf16 bytes
    bh = w.B * w.H
    qo = e * (w.Tq * w.d + w.Tq * w.dv)  # Q and dO (or Q and O)
    kv = e * (w.Tk * w.d + w.Tk * w.dv)  # K and V
    return {
        "fwd": bh * (qo + kv + 4 * w.Tq),
        "bwd_prep": 0,
        "bwd_dkdv": bh * (qo + kv + 8 * w.Tq + kv),
        "bwd_dq": bh * (qo + kv + e * w.Tq * w.dv + 4 * w.Tq + 8 * w.Tq + e * w.Tq * w.d),
    }


def kernel_source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "exact_tiled_softmax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"decode": ["decode_bf16.hip", "attn_common.hpp"],
                  "fwd": ["fwd_bf16.hip", "attn_common.hpp", "tile_stream.hpp"],
                  "bwd_dkdv": ["bwd_bf16.hip", "attn_common.hpp", "tile_stream.hpp"],
                  "bwd_dq": ["bwd_bf16.hip", "attn_common.hpp", "tile_stream.hpp"]}
KERNEL_SYMBOL = {"decode": "decode_bf16_kernel", "fwd": "fwd_bf16_kernel", "bwd_dkdv": "bwd_dkdv_kernel", "bwd_dq": "bwd_dq_kernel"}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_SYMBOL[kernel]}_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_digest(KERNEL_SOURCES[kernel]):
        return None
    return float(m_b.group(1))


def host_workers() -> int:
    """Worker processes for the CPU oracle: the cores this process may run on,
    capped by OMP_NUM_THREADS when it is set (the host's share of CPUs)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _oracle_head(args):
    """One pool task: the float64 oracle's dense forward + backward of one
    head, with single-threaded BLAS; returns (start, end) of the oracle call
    on the shared monotonic clock."""
    w, b, h = args
    from threadpoolctl import threadpool_limits

    import numpy as np

    from exact_tiled_softmax_amd.inputs import make_head
    from oracle import dense_backward, dense_forward

    q, k, v, do = (make_head(w, n, b, h) for n in ("q", "k", "v", "do"))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        o, _ = dense_forward(q, k, v, w.scale, w.causal)
        dq, _, _ = dense_backward(q, k, v, do, w.scale, w.causal)
        t1 = time.perf_counter()
    assert np.isfinite(o).all() and np.isfinite(dq).all()
    return t0, t1


def cpu_baseline(w, budget_s: float):
    """The float64 oracle (dense forward + backward) on whole heads of the
    workload: a pool of single-threaded workers, one per host core, each
    taking one head at a time; as many rounds of heads as fit in about
    `budget_s` seconds (at least one).  Must run before the process touches
    the GPU (the pool forks)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    workers = host_workers()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_head_flops = 2 * unmasked_pairs(w.Tq, w.Tk, w.causal) * ((w.d + w.dv) + (3 * w.d + 2 * w.dv))
    done, spans = 0, []
    t_begin = time.perf_counter()
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork")) as ex:
        while done < len(heads):
            batch = heads[done:done + workers]
            spans += list(ex.map(_oracle_head, [(w, b, h) for b, h in batch]))
            done += len(batch)
            if time.perf_counter() - t_begin >= budget_s:
                break
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    return {
        "value": done * per_head_flops / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "blas_threads_per_core": 1,
        "kind": "oracle",
        "sample": (f"{done} of {w.B * w.H} heads of {w.name} (first: b,h={heads[0]}), forward+backward in float64 "
                   f"numpy with full score rows, one head per worker process, {workers} single-threaded workers, "
                   f"{wall:.1f} s wall; same algorithmic flop count as the GPU"),
    }


def decode_bytes(w, lens):
    """Algorithmic HBM bytes of one decode call: each sequence's cached key and
    value rows (bf16) read once, q read, o (bf16) and lse (fp32) written."""
    e = 2
    kv = int(sum(int(n) for n in lens)) * w.H * e * (w.d + w.dv)
    return kv + w.B * w.H * w.Tq * (e * w.d + e * w.dv + 4)


def cpu_baseline_decode(w, lens, budget_s: float):
    """The float64 oracle decode over the whole workload (every sequence, all
    heads), repeated until about `budget_s` seconds of oracle time have run
    (one pass takes well under a second); one process, single-threaded BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from exact_tiled_softmax_amd.inputs import make_head
    from oracle import decode_forward

    seqs = []
    for b in range(w.B):
        n = int(lens[b])
        q = np.stack([make_head(w, "q", b, h) for h in range(w.H)])[None]
        k = np.stack([make_head(w, "k", b, h)[:n] for h in range(w.H)])[None]
        v = np.stack([make_head(w, "v", b, h)[:n] for h in range(w.H)])[None]
        seqs.append((n, q, k, v))
    passes, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while passes == 0 or elapsed < budget_s:
            for n, q, k, v in seqs:
                t0 = time.perf_counter()
                o, lse = decode_forward(q, k, v, w.scale, kv_lens=[n], causal=w.causal)
                elapsed += time.perf_counter() - t0
                assert np.isfinite(o).all()
            passes += 1
    return {
        "value": passes * decode_bytes(w, lens) / elapsed / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "blas_threads_per_core": 1,
        "kind": "oracle",
        "sample": (f"the whole workload {w.name} ({w.B} sequences x {w.H} heads, cache lengths "
                   f"{[int(x) for x in lens]}) {passes} times, float64 numpy in one single-threaded process, "
                   f"{elapsed:.1f} s; same algorithmic byte count as the GPU"),
    }


def bench_decode(args, w, cpu) -> int:
    import torch

    from exact_tiled_softmax_amd import attn
    from exact_tiled_softmax_amd.inputs import kv_lens, make_tensor

    dev = torch.device("cuda:0")
    lens_np = kv_lens(w)
    print(f"[bench] building inputs for {w.name}", file=sys.stderr, flush=True)
    q, k, v = (make_tensor(w, n).to(dev) for n in ("q", "k", "v"))
    lens = torch.from_numpy(lens_np).to(dev)
    o = torch.empty((w.B, w.H, w.Tq, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device=dev)

    def step():
        attn.decode(q, k, v, kv_lens=lens, scale=w.scale, causal=w.causal, out=o, lse=lse,
                    num_splits=args.decode_splits or None)

    n_warm = warm_up(step, args.warmup, args.warmup_min_s)
    print(f"[bench] warmup done ({n_warm} steps); timing {args.steps} steps", file=sys.stderr, flush=True)
    attn.profile_start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn.profile_stop()
    kern = {name: attn.profile_query(kind) for kind, name in attn.KERNEL_NAMES.items()}

    nbytes = decode_bytes(w, lens_np)
    ms_step = (t1 - t0) * 1e3 / args.steps
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    dom_ms = kern["decode"][0] / max(1, kern["decode"][1])
    achieved = nbytes / (dom_ms * 1e-3) / 1e9
    roofline = {
        "kernel": KERNEL_SYMBOL["decode"],
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic("decode", w.name),
        "avg_launch_ms": round(dom_ms, 4),
        "launches": kern["decode"][1],
        "algorithmic_bytes_per_launch": nbytes,
    }
    line = {
        "metric": "decode HBM GB/s (algorithmic bytes), bf16 d=128, 1 query against a mixed-length KV cache",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": args.warmup_min_s,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Tq": w.Tq, "Tk": w.Tk, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "kv_lens": [int(x) for x in lens_np], "step": "attn_decode"},
        "kernel_ms_per_step": {n: round(kern[n][0] / args.steps, 4) for n in kern if kern[n][1]},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def standard_bytes(w):
    """HBM bytes of the materialised path per call: S written (fp32), read twice
    by the two-pass row softmax, P written and read (bf16, keys padded to 64),
    plus Q, K, V read, V^T written and read, O and LSE written."""
    bh, tkp = w.B * w.H, (w.Tk + 63) // 64 * 64
    mat = bh * w.Tq * (w.Tk * 4 * 3 + tkp * 2 * 2)
    io = bh * (2 * (w.Tq * w.d + w.Tk * w.d + w.Tk * w.dv + 2 * tkp * w.dv + w.Tq * w.dv) + 4 * w.Tq)
    return mat + io


def bench_standard(args, w) -> int:
    """The IO comparison: the tiled forward and the materialised standard
    forward timed on the same inputs, one after the other.  The compared
    times are the kernels' own (the library's HIP events); wall times per
    call are reported beside them."""
    import torch

    from exact_tiled_softmax_amd import attn
    from exact_tiled_softmax_amd.inputs import make_tensor

    dev = torch.device("cuda:0")
    print(f"[bench] building inputs for {w.name}", file=sys.stderr, flush=True)
    q, k, v = (make_tensor(w, n).to(dev) for n in ("q", "k", "v"))
    o = torch.empty((w.B, w.H, w.Tq, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device=dev)
    res, wall = {}, {}
    kinds = {"tiled": ("fwd", "fwd_aux"), "standard": ("standard",)}
    for name, fn in (("tiled", attn.fwd), ("standard", attn.fwd_standard)):
        warm_up(lambda: fn(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse), args.warmup, args.warmup_min_s)
        attn.profile_start()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
        torch.cuda.synchronize()
        wall[name] = (time.perf_counter() - t0) * 1e3 / args.steps
        attn.profile_stop()
        # kernel time from the library's HIP events: the wall time of the
        # standard path also holds the mapping of its workspace, which the
        # driver sometimes takes hundreds of ms over
        res[name] = sum(attn.profile_query(kind)[0] for kind, n in attn.KERNEL_NAMES.items()
                        if n in kinds[name]) / args.steps
        print(f"[bench] {name}: {res[name]:.3f} ms of kernels, {wall[name]:.3f} ms wall per call", file=sys.stderr,
              flush=True)
    _, fwd_fl, _, fwd_b, _ = work(w)
    std_b = standard_bytes(w)
    line = {
        "metric": "attention forward TFLOP/s, tiled vs materialised standard attention (IO comparison)",
        "value": round(fwd_fl / (res["standard"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": args.warmup_min_s,
        "ms_per_step": round(res["standard"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Tq": w.Tq, "Tk": w.Tk, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "step": "attn_fwd_standard"},
        "io_comparison": {
            "tiled_ms": round(res["tiled"], 4),
            "standard_ms": round(res["standard"], 4),
            "tiled_wall_ms": round(wall["tiled"], 4),
            "standard_wall_ms": round(wall["standard"], 4),
            "standard_over_tiled_time": round(res["standard"] / res["tiled"], 2),
            "tiled_algorithmic_bytes": fwd_b,
            "standard_hbm_bytes_model": std_b,
            "standard_over_tiled_bytes": round(std_b / fwd_b, 1),
            "standard_GBs_at_model": round(std_b / (res["standard"] * 1e-3) / 1e9, 1),
        },
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_states(args, w) -> int:
    """Forward through key-range states (the chunk-wise mode's state and its
    rescale merge, P1 "Chunk-wise Mode with Online Softmax Re-scale"): the
    key range is cut into N equal ranges, attn_fwd_state computes each
    range's partial state (acc, m, l) into one stacked buffer, and
    attn_merge_states merges the N states into O and LSE, as a forward whose
    keys arrive in pieces (sequence sharding) would.  Timed beside the
    one-shot attn_fwd on the same inputs; kernel times from the library's
    HIP events (states: the forward kernel kind, merge: the auxiliary kind)."""
    import torch

    from exact_tiled_softmax_amd import attn
    from exact_tiled_softmax_amd.inputs import make_tensor

    n = args.state_merge
    dev = torch.device("cuda:0")
    print(f"[bench] building inputs for {w.name}", file=sys.stderr, flush=True)
    q, k, v = (make_tensor(w, nm).to(dev) for nm in ("q", "k", "v"))
    bounds = [(i * w.Tk // n, (i + 1) * w.Tk // n) for i in range(n)]
    if any(b <= a for a, b in bounds):
        print(f"--state-merge {n}: more ranges than keys", file=sys.stderr)
        return 2
    # each range's keys as their own buffers, as a shard would hold them
    ks = [k[:, :, a:b].contiguous() for a, b in bounds]
    vs = [v[:, :, a:b].contiguous() for a, b in bounds]
    acc = torch.empty((n, w.B, w.H, w.Tq, w.dv), dtype=torch.float32, device=dev)
    m = torch.empty((n, w.B, w.H, w.Tq), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    o = torch.empty((w.B, w.H, w.Tq, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device=dev)
    o1, lse1 = torch.empty_like(o), torch.empty_like(lse)

    def states():
        for j, (a, _) in enumerate(bounds):
            attn.fwd_state(q, ks[j], vs[j], scale=w.scale, causal=w.causal, q_offset=0, k_offset=a, acc=acc[j],
                           m=m[j], l=l[j])

    def merge():
        attn.merge_states(acc, m, l, out=o, lse=lse)

    def one_shot():
        attn.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o1, lse=lse1)

    # kernel time per call of each part (a state call that splits its range
    # launches the forward kernel and a merge of its splits)
    res = {}
    for name, fn in (("one_shot", one_shot), ("states", states), ("merge", merge)):
        warm_up(fn, args.warmup, args.warmup_min_s)
        attn.profile_start()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        attn.profile_stop()
        res[name] = sum(attn.profile_query(kind)[0] for kind, kn in attn.KERNEL_NAMES.items()
                        if kn in ("fwd", "fwd_aux")) / args.steps
    _, fwd_fl, _, _, _ = work(w)
    one_ms, st_ms, mg_ms = res["one_shot"], res["states"], res["merge"]
    merge_bytes = n * w.B * w.H * w.Tq * (w.dv + 2) * 4 + w.B * w.H * w.Tq * (w.dv * 2 + 4)
    do = (o.float() - o1.float()).abs().max().item()
    dl = (lse - lse1).abs().max().item()
    line = {
        "metric": f"attention forward TFLOP/s through {n} key-range states and their merge",
        "value": round(fwd_fl / ((st_ms + mg_ms) * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": args.warmup_min_s,
        "ms_per_step": round(st_ms + mg_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Tq": w.Tq, "Tk": w.Tk, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "key_ranges": n, "step": "attn_fwd_state x N + attn_merge_states"},
        "states": {
            "states_ms": round(st_ms, 4),
            "merge_ms": round(mg_ms, 4),
            "merge_GBs": round(merge_bytes / (mg_ms * 1e-3) / 1e9, 1) if mg_ms > 0 else None,
            "merge_bytes": merge_bytes,
            "one_shot_fwd_ms": round(one_ms, 4),
            "one_shot_tflops": round(fwd_fl / (one_ms * 1e-3) / 1e12, 2),
            "states_plus_merge_over_one_shot": round((st_ms + mg_ms) / one_ms, 3),
            "max_abs_diff_o_vs_one_shot": do,
            "max_abs_diff_lse_vs_one_shot": dl,
        },
    }
    print(json.dumps(line), flush=True)
    return 0


def warm_up(step, steps, min_s):
    """Run `step` at least `steps` times and, beyond that, until at least
    `min_s` seconds of back-to-back work have run.  From idle the GPU's clock
    takes longer than a few short steps to reach its loaded level: five
    warm-up steps of the L=4096 workload (3.4 ms) left its kernels 14% slower
    than after 200.  Returns the number of warm-up steps run."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while n < steps or time.perf_counter() - t0 < min_s:
        step()
        n += 1
        if n >= steps:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_steps(attn, w, dev, steps, warmup, flush_mib=0, warmup_min_s=0.0):
    """Warm up, then time `steps` fwd+bwd steps of workload w with inputs
    resident on `dev`.  Returns ({kernel: (total_ms, launches)} from the
    library's HIP events, wall ms per step).  With flush_mib > 0 a buffer of
    that size is written before every step and the step time is the
    attention kernels' own event time."""
    import torch

    from exact_tiled_softmax_amd.inputs import make_tensor

    print(f"[bench] building inputs for {w.name}", file=sys.stderr, flush=True)
    q, k, v, do = (make_tensor(w, n).to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty((w.B, w.H, w.Tq, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device=dev)
    dq, dk, dvg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    flush = torch.empty(flush_mib << 18, dtype=torch.float32, device=dev) if flush_mib > 0 else None

    def step():
        if flush is not None:
            flush.fill_(1.0)
        attn.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
        attn.bwd(q, k, v, o, lse, do, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dvg)

    n_warm = warm_up(step, warmup, warmup_min_s)
    print(f"[bench] {w.name}: warmup done ({n_warm} steps); timing {steps} steps", file=sys.stderr, flush=True)
    attn.profile_start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn.profile_stop()
    kern = {name: attn.profile_query(kind) for kind, name in attn.KERNEL_NAMES.items()}
    ms_step = (t1 - t0) * 1e3 / steps
    if flush is not None:
        # the flush between steps is not attention work
        ms_step = sum(kern[n][0] for n in ("fwd", "fwd_aux", "bwd_prep", "bwd_dkdv", "bwd_dq")) / steps
    return kern, ms_step, n_warm


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-min-s", type=float, default=0.5, metavar="S",
                    help="keep warming up past --warmup steps until S seconds of back-to-back steps have run "
                         "(the GPU clock needs that long to leave its idle level)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work (0 = skip)")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="write this many MiB before every step (evicts L2 and the Infinity Cache); the step time "
                         "is then the attention kernels' own event time, without the flush")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes) and exit")
    ap.add_argument("--standard", action="store_true",
                    help="time the tiled forward and the materialised standard forward (attn_fwd_standard) on the "
                         "workload and print the IO comparison line instead of the fwd+bwd step")
    ap.add_argument("--state-merge", type=int, default=0, metavar="N",
                    help="time the forward through N key-range states (attn_fwd_state) and their merge "
                         "(attn_merge_states) beside the one-shot attn_fwd, and print that line instead")
    ap.add_argument("--decode-splits", type=int, default=0,
                    help="decode workloads: key-range splits per sequence (0 = the library's choice)")
    ap.add_argument("--no-targets", dest="targets", action="store_false",
                    help="headline workload only: skip timing the L=4096 causal, d=64 and long-key workloads in "
                         "the same run")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); the "
              "attention kernels have no multi-GPU path", file=sys.stderr)
        return 2

    import torch

    from exact_tiled_softmax_amd import attn
    from exact_tiled_softmax_amd.inputs import WORKLOADS, kv_lens

    w = WORKLOADS[args.workload]
    # The CPU oracle runs first: its worker pool forks, which must happen
    # before this process initialises the GPU.
    cpu = None
    if (args.cpu_budget > 0 and not args.copy_calibration and not args.standard and not args.state_merge
            and w.dtype == "bf16"):
        print(f"[bench] timing the CPU oracle (~{args.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline_decode(w, kv_lens(w), args.cpu_budget) if w.decode else cpu_baseline(w, args.cpu_budget)

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))
        return 0
    attn.load()
    if w.dtype != "bf16":
        print("bench.py times the bf16 path", file=sys.stderr)
        return 2
    if w.decode:
        return bench_decode(args, w, cpu)
    if args.standard:
        return bench_standard(args, w)
    if args.state_merge > 0:
        return bench_states(args, w)
    dev = torch.device("cuda:0")
    kern, ms_step, n_warm = time_steps(attn, w, dev, args.steps, args.warmup, args.flush_mib, args.warmup_min_s)
    pairs, fwd_fl, bwd_fl, fwd_b, bwd_b = work(w)
    fwd_ms = (kern["fwd"][0] + kern["fwd_aux"][0]) / args.steps
    bwd_ms = (kern["bwd_prep"][0] + kern["bwd_dkdv"][0] + kern["bwd_dq"][0]) / args.steps
    total_tflops = (fwd_fl + bwd_fl) / (ms_step * 1e-3) / 1e12
    fwd_tflops = fwd_fl / (fwd_ms * 1e-3) / 1e12 if fwd_ms > 0 else None
    bwd_tflops = bwd_fl / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else None

    # dominant kernel: largest recorded time
    kfl = kernel_flops(w)
    kby = kernel_bytes(w)
    dom = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda n: kern[n][0])
    dom_avg_ms = kern[dom][0] / max(1, kern[dom][1])
    alg_fl, exe_fl = kfl[dom]
    achieved = alg_fl / (dom_avg_ms * 1e-3) / 1e12
    traffic = measured_traffic(dom, w.name)
    roofline = {
        "kernel": KERNEL_SYMBOL[dom],
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "avg_launch_ms": round(dom_avg_ms, 4),
        "launches": kern[dom][1],
        "algorithmic_flops_per_launch": alg_fl,
        "executed_flops_per_launch": exe_fl,
        "executed_tflops": round(exe_fl / (dom_avg_ms * 1e-3) / 1e12, 2),
        "algorithmic_bytes_per_launch": kby[dom],
        "traffic_over_algorithmic_bytes": round(traffic / kby[dom], 3) if traffic else None,
    }

    # the backward target workload and the side workloads, timed in the same
    # run with the same step counts (inputs of each freed before the next)
    targets = {w.name: {"fwd_frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4) if fwd_tflops else None,
                        "bwd_frac_of_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4) if bwd_tflops else None}}
    for tname in ((BWD_TARGET,) + SIDE_TARGETS if args.targets and w.name == HEADLINE else ()):
        wt = WORKLOADS[tname]
        kt, _, t_warm = time_steps(attn, wt, dev, args.steps, args.warmup, args.flush_mib, args.warmup_min_s)
        _, tf_fl, tb_fl, _, _ = work(wt)
        t_fwd_ms = (kt["fwd"][0] + kt["fwd_aux"][0]) / args.steps
        t_bwd_ms = (kt["bwd_prep"][0] + kt["bwd_dkdv"][0] + kt["bwd_dq"][0]) / args.steps
        targets[wt.name] = {
            "fwd_ms": round(t_fwd_ms, 4),
            "fwd_frac_of_peak": round(tf_fl / (t_fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_ms": round(t_bwd_ms, 4),
            "bwd_frac_of_peak": round(tb_fl / (t_bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "warmup_steps_run": t_warm,
            "kernel_ms_per_step": {n: round(kt[n][0] / args.steps, 4) for n in kt if kt[n][1]},
        }

    line = {
        "metric": METRIC,
        "value": round(total_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": args.warmup_min_s,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Tq": w.Tq, "Tk": w.Tk, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "step": "attn_fwd + attn_bwd",
                   **({"flush_mib_between_steps": args.flush_mib} if args.flush_mib > 0 else {})},
        "fwd_tflops": round(fwd_tflops, 2) if fwd_tflops else None,
        "fwd_frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4) if fwd_tflops else None,
        "bwd_tflops": round(bwd_tflops, 2) if bwd_tflops else None,
        "bwd_frac_of_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4) if bwd_tflops else None,
        "fwd_bwd_frac_of_peak": round(total_tflops / PEAK_BF16_TFLOPS, 4),
        "kernel_ms_per_step": {n: round(kern[n][0] / args.steps, 4) for n in kern},
        "targets": targets,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
