"""Float64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP kernels or their
binding and imports nothing from that package.

What it computes is the plain definition, written out in numpy float64 with the
full score rows materialised:

* Forward.  Standard attention, "The Hidden Recurrence in Softmax Attention:
  A Path to Flash Attention", section "Standard Attention / Forward Pass" (the
  masked exp, row-normalised, times V), with the 1/sqrt(head_dim) scale of
  "attention backprop", section "Forward Pass", made an explicit argument.  The
  softmax subtracts the row maximum before exponentiating (a textbook identity;
  plain exp overflows for the +-1000 scores that "Tiled attention with an online
  softmax", section "Constraints", requires).  The log-sum-exp is the natural
  log, as in "Tiled attention with an online softmax", section "Task"
  (the last paragraph: output a/l, log-sum-exp m + log l).
* Causal mask.  Key j is blocked for query i when j > i, on global indices
  ("Tiled attention with an online softmax", section "Task").  This is
  top-left alignment also when Tq != Tk.
* Backward.  "attention backprop", sections "Gradient of V and P" (dV = P^T dO,
  dP = dO V^T), "Gradient of S" (dS = dP o P - ROW_SUM(dO o O) o P) and
  "Gradient of Q and K" (dQ = dS K, dK = dS^T Q).  That page drops the scale;
  with S = scale * Q K^T the chain rule multiplies dQ and dK by scale.
* Online step and tiled forward.  The algorithm of "Tiled attention with an
  online softmax", section "Task", in the log-domain form of the rescale rule
  in "The Hidden Recurrence in Softmax Attention", section "Chunk-wise Mode with
  Online Softmax Re-scale" (new max = max of old max and block max; old l and
  accumulator multiplied by exp(old max - new max); block terms by
  exp(score - new max)).  The step's own formulas are missing from the page
  text; this reading is pinned by the page's third worked example.  It exists
  to pin the dense oracle (block-size invariance), never as the oracle itself.
* Partial state and merge.  The exact (m, l, a) of one key range (m its row
  maximum, l and a its exp-weighted sum and value sum), with global query and
  key offsets for the causal mask, and the rule that combines such states:
  "The Hidden Recurrence in Softmax Attention", section "Chunk-wise Mode with
  Online Softmax Re-scale" (each state rescaled by exp(m_s - max), summed;
  O = a / l, LSE = max + ln l).
* Decode.  The newest Tq queries of each sequence against the first L_b
  slots of a key cache, query i at position L_b - Tq + i ("The Hidden
  Recurrence in Softmax Attention", section "Recurrent mode": the query of
  step t sees the keys of steps up to t); the plain definition per row.
* Chunk-wise mode without the rescale.  "The Hidden Recurrence in Softmax
  Attention", section "Chunk-wise Mode": row sums and accumulators of
  exp(S) o M added chunk by chunk with no max subtracted.  Exact for modest
  scores, overflowing for large ones; kept as the negative control that shows
  why the rescale exists.
* Gradient of the log-sum-exp.  When a caller also differentiates LSE, its
  upstream gradient dLSE adds dLSE o P to dS, since d LSE_i / d S_ij = P_ij
  ("Flash Attention Backward Pass", which treats l as a smooth function of the
  scores that the gradient flows through).  Equivalently the row term
  ROW_SUM(dO o O) is replaced by ROW_SUM(dO o O) - dLSE.

Pins (tests/test_oracle_pins.py): the three worked examples of "Tiled
attention with an online softmax", section "Examples"; block-size invariance
to 1e-9 (section "Constraints"); closed forms and invariants; central finite
differences of the backward, also with a dLSE input; an independent library
routine (torch CPU autograd in float64, with and without dLSE); and merged
key-range states against the dense forward of the whole range.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def causal_blocked(tq: int, tk: int, row0: int = 0, col0: int = 0) -> np.ndarray:
    """Boolean [tq, tk] array, True where key (col0 + j) is blocked for query
    (row0 + i): blocked iff global key index > global query index."""
    rows = row0 + np.arange(tq)[:, None]
    cols = col0 + np.arange(tk)[None, :]
    return cols > rows


def _scores(q, k, scale, causal, row0=0):
    """Full score rows S = scale * Q K^T for the query rows row0.. of one head,
    with blocked keys set to -inf."""
    s = scale * (q @ k.T)
    if causal:
        s = np.where(causal_blocked(s.shape[0], s.shape[1], row0=row0), NEG_INF, s)
    return s


def _softmax_rows(s):
    """Row softmax and natural log-sum-exp of a score block whose rows are
    complete.  A row with every key blocked has P = 0 and LSE = -inf."""
    m = np.max(s, axis=1, keepdims=True)
    mu = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - mu)
    l = np.sum(e, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l > 0, mu + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return p, lse[:, 0]


def _head_forward(q, k, v, scale, causal, row_chunk):
    tq = q.shape[0]
    o = np.empty((tq, v.shape[1]), dtype=np.float64)
    lse = np.empty((tq,), dtype=np.float64)
    for r0 in range(0, tq, row_chunk):
        r1 = min(tq, r0 + row_chunk)
        p, lse[r0:r1] = _softmax_rows(_scores(q[r0:r1], k, scale, causal, row0=r0))
        o[r0:r1] = p @ v
    return o, lse


def dense_forward(q, k, v, scale, causal=False, row_chunk=2048):
    """Standard attention forward in float64.

    q: [..., Tq, d], k: [..., Tk, d], v: [..., Tk, dv] (leading batch/head
    dimensions are broadcast-free and must match).  Returns (o [..., Tq, dv],
    lse [..., Tq]).  Query rows are processed in chunks of `row_chunk` rows,
    each row complete, which only bounds memory."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    lead = q.shape[:-2]
    qf = q.reshape((-1,) + q.shape[-2:])
    kf = k.reshape((-1,) + k.shape[-2:])
    vf = v.reshape((-1,) + v.shape[-2:])
    o = np.empty(qf.shape[:-1] + (vf.shape[-1],), dtype=np.float64)
    lse = np.empty(qf.shape[:-1], dtype=np.float64)
    for n in range(qf.shape[0]):
        o[n], lse[n] = _head_forward(qf[n], kf[n], vf[n], scale, causal, row_chunk)
    return o.reshape(lead + o.shape[-2:]), lse.reshape(lead + lse.shape[-1:])


def _head_backward(q, k, v, dout, scale, causal, row_chunk, dlse=None):
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, q.shape[0], row_chunk):
        r1 = min(q.shape[0], r0 + row_chunk)
        p, _ = _softmax_rows(_scores(q[r0:r1], k, scale, causal, row0=r0))
        o = p @ v
        do = dout[r0:r1]
        # "attention backprop", "Gradient of V and P": dV = P^T dO, dP = dO V^T
        dv += p.T @ do
        dp = do @ v.T
        # "attention backprop", "Gradient of S": dS = dP o P - ROW_SUM(dO o O) o P
        rowsum = np.sum(do * o, axis=1, keepdims=True)
        ds = dp * p - rowsum * p
        if dlse is not None:
            # an upstream gradient on LSE_i = m_i + ln l_i flows through l
            # ("The Hidden Recurrence in Softmax Attention", "Flash Attention
            # Backward Pass"): d LSE_i / d S_ij = P_ij
            ds = ds + dlse[r0:r1, None] * p
        # "attention backprop", "Gradient of Q and K", times the chain-rule scale
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def dense_backward(q, k, v, dout, scale, causal=False, row_chunk=2048, dlse=None):
    """Gradients (dq, dk, dv) of L = sum(dout * O) (+ sum(dlse * LSE) when
    `dlse` [..., Tq] is given) for (O, LSE) = dense_forward(...).

    Recomputes P from the inputs in float64 (rows complete).  Shapes as in
    dense_forward; dout has O's shape."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    dlf = None if dlse is None else _as_f64(dlse).reshape((-1, q.shape[-2]))
    lead = q.shape[:-2]
    qf = q.reshape((-1,) + q.shape[-2:])
    kf = k.reshape((-1,) + k.shape[-2:])
    vf = v.reshape((-1,) + v.shape[-2:])
    df = dout.reshape((-1,) + dout.shape[-2:])
    dq = np.empty_like(qf)
    dk = np.empty_like(kf)
    dv = np.empty_like(vf)
    for n in range(qf.shape[0]):
        dq[n], dk[n], dv[n] = _head_backward(qf[n], kf[n], vf[n], df[n], scale, causal, row_chunk,
                                             None if dlf is None else dlf[n])
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


# --- Partial states of key ranges and their merge -----------------------------

def attention_state(q, k, v, scale, causal=False, q_offset=0, k_offset=0):
    """The state (m, l, acc) of each query row over one key range, in the
    sense of "Tiled attention with an online softmax", section "Task": m_i
    the largest allowed scaled score, l_i = sum_j exp(s_ij - m_i) and
    acc_i = sum_j exp(s_ij - m_i) v_j over the allowed keys j.  With
    `causal`, key j of this range is blocked for query i when
    k_offset + j > q_offset + i (global positions).  A row with no allowed
    key has m = -inf, l = 0, acc = 0.  Shapes as in dense_forward; returns
    (m [..., Tq], l [..., Tq], acc [..., Tq, dv])."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        s = np.where(causal_blocked(s.shape[-2], s.shape[-1], row0=q_offset, col0=k_offset), NEG_INF, s)
    m = np.max(s, axis=-1)
    mu = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - mu[..., None])
    return m, np.sum(e, axis=-1), e @ v


def merge_states(ms, ls, accs):
    """(O, LSE) of the union of key ranges from their states (sequences of
    m [..., Tq], l [..., Tq], acc [..., Tq, dv]): every state is rescaled to
    the common max M = max_s m_s ("The Hidden Recurrence in Softmax
    Attention", section "Chunk-wise Mode with Online Softmax Re-scale"),
    l = sum_s exp(m_s - M) l_s, acc = sum_s exp(m_s - M) acc_s, O = acc / l,
    LSE = M + ln l (O = 0 and LSE = -inf where l = 0)."""
    ms = [_as_f64(x) for x in ms]
    M = ms[0]
    for x in ms[1:]:
        M = np.maximum(M, x)
    mu = np.where(np.isneginf(M), 0.0, M)
    l = np.zeros_like(mu)
    acc = np.zeros_like(_as_f64(accs[0]))
    for m_s, l_s, a_s in zip(ms, ls, accs):
        w = np.exp(m_s - mu)
        l = l + w * _as_f64(l_s)
        acc = acc + w[..., None] * _as_f64(a_s)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[..., None] > 0, acc / np.where(l > 0, l, 1.0)[..., None], 0.0)
        lse = np.where(l > 0, mu + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o, lse


# --- Decode: a few newest queries against a cache of keys --------------------

def decode_forward(q, k, v, scale, kv_lens=None, causal=False):
    """Attention of the newest queries of each sequence over its cached keys
    (the recurrent mode of "The Hidden Recurrence in Softmax Attention",
    section "Recurrent mode": the query at step t sees the keys of steps up
    to t).

    q [B, H, Tq, d]; k [B, H, Tk, d], v [B, H, Tk, dv] hold Tk cache slots;
    sequence b uses the first L_b = clip(kv_lens[b], 0, Tk) of them (all Tk
    when kv_lens is None).  Query i of sequence b sits at position
    L_b - Tq + i.  With `causal`, key j is blocked for it when
    j > L_b - Tq + i; otherwise every cached key j < L_b is allowed.  A query
    with no allowed key gets O = 0 and LSE = -inf.  Returns (o [B, H, Tq, dv],
    lse [B, H, Tq]), each row from its complete score row."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, tq, _ = q.shape
    tk = k.shape[2]
    lens = np.full(B, tk) if kv_lens is None else np.clip(np.asarray(kv_lens, dtype=np.int64), 0, tk)
    o = np.zeros((B, H, tq, v.shape[3]))
    lse = np.full((B, H, tq), NEG_INF)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h, :n].T)
            if causal:
                s = np.where(causal_blocked(tq, n, row0=n - tq), NEG_INF, s)
            p, lse[b, h] = _softmax_rows(s)
            o[b, h] = p @ v[b, h, :n]
    return o, lse


# --- Chunk-wise mode without the rescale (negative control) -------------------

def chunkwise_unrescaled(q, k, v, block_size, scale, causal=False):
    """The chunk-wise mode of "The Hidden Recurrence in Softmax Attention",
    section "Chunk-wise Mode", before the rescale is introduced: over key
    chunks of `block_size` (starting at 0, the last possibly shorter) the row
    sums ll += (exp(S_chunk) o M) 1 and the accumulator A += (exp(S_chunk) o M)
    V_chunk are added up with no max subtracted; O = A / ll and LSE = ln ll.
    S = scale * Q K^T; M is the causal mask (key j blocked for query i when
    j > i) or no mask.  exp overflows to inf once a score passes about 709.78
    in float64; the result then holds inf or nan, which is the point of this
    function: it shows what the rescale prevents.  One head: q [Tq, d]."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if block_size < 1:
        raise ValueError("block_size must be >= 1")
    tq, tk = q.shape[0], k.shape[0]
    ll = np.zeros(tq)
    acc = np.zeros((tq, v.shape[1]))
    with np.errstate(over="ignore", invalid="ignore"):
        for start in range(0, tk, block_size):
            stop = min(start + block_size, tk)
            e = np.exp(scale * (q @ k[start:stop].T))
            if causal:
                e = np.where(causal_blocked(tq, stop - start, col0=start), 0.0, e)
            ll = ll + np.sum(e, axis=1)
            acc = acc + e @ v[start:stop]
        o = acc / ll[:, None]
        lse = np.log(ll)
    return o, lse


# --- Sampled outputs for large shapes ----------------------------------------

def forward_rows(q, k, v, rows, scale, causal=False):
    """O and LSE of selected query rows of one head (q [Tq,d], k [Tk,d],
    v [Tk,dv]); each row computed from its complete score row."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], NEG_INF, s)
    p, lse = _softmax_rows(s)
    return p @ v, lse


def backward_dq_rows(q, k, v, dout, rows, scale, causal=False):
    """dQ of selected query rows of one head.  Row i of dQ needs only row i of
    P, dP and the row sum D_i = sum(dO_i o O_i)."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], NEG_INF, s)
    p, _ = _softmax_rows(s)
    o = p @ v
    do = dout[rows]
    dp = do @ v.T
    ds = dp * p - np.sum(do * o, axis=1, keepdims=True) * p
    return scale * (ds @ k)


def backward_dkdv_cols(q, k, v, dout, cols, scale, causal=False, row_chunk=2048):
    """dK and dV of selected key rows of one head.  Column j of P needs every
    query row's normaliser, so full rows are formed chunk by chunk and only the
    selected columns are kept."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size, k.shape[1]))
    dv = np.zeros((cols.size, v.shape[1]))
    for r0 in range(0, q.shape[0], row_chunk):
        r1 = min(q.shape[0], r0 + row_chunk)
        p, _ = _softmax_rows(_scores(q[r0:r1], k, scale, causal, row0=r0))
        o = p @ v
        do = dout[r0:r1]
        dsum = np.sum(do * o, axis=1, keepdims=True)
        pc = p[:, cols]
        dpc = do @ v[cols].T
        dsc = dpc * pc - dsum * pc
        dv += pc.T @ do
        dk += scale * (dsc.T @ q[r0:r1])
    return dk, dv


# --- The pages' tiled algorithm (used only to pin the dense oracle) ----------

def online_softmax_step(m, l, acc, scores, v_block):
    """One key block added to the running state of each query row.

    m [N], l [N], acc [N, dv]; scores [N, b] (already scaled; -inf = blocked
    key); v_block [b, dv].  New max m' = max(m, max_j s_j).  Where m' is -inf
    the row has no allowed key yet, and 0 stands in for m' inside both
    exponentials ("Tiled attention with an online softmax", section "Task").
    Then c = exp(m - m'), p_j = exp(s_j - m'), l' = c l + sum_j p_j and
    acc' = c acc + sum_j p_j v_j.  Inputs are not modified."""
    m = _as_f64(m)
    l = _as_f64(l)
    acc = _as_f64(acc)
    scores = _as_f64(scores)
    v_block = _as_f64(v_block)
    m_new = np.maximum(m, np.max(scores, axis=1)) if scores.shape[1] else m.copy()
    shift = np.where(np.isneginf(m_new), 0.0, m_new)
    c = np.exp(m - shift)
    p = np.exp(scores - shift[:, None])
    l_new = c * l + np.sum(p, axis=1)
    acc_new = c[:, None] * acc + p @ v_block
    return m_new, l_new, acc_new


def tiled_forward(q, k, v, block_size, causal=False, scale=None):
    """The tiled forward of "Tiled attention with an online softmax", section
    "Task": key blocks start at 0, b, 2b, ...; the last may be shorter; the
    block's scores are Q K_b^T / sqrt(d) (d = last axis of Q) unless `scale` is
    given; causal blocks key j for query i when j > i (global indices).  The
    output row is a/l and the log-sum-exp m + log l.  One head: q [Tq,d]."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if block_size < 1:
        raise ValueError("block_size must be >= 1")
    tq, tk = q.shape[0], k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    m = np.full((tq,), NEG_INF)
    l = np.zeros((tq,))
    acc = np.zeros((tq, v.shape[1]))
    for start in range(0, tk, block_size):
        stop = min(tk, start + block_size)
        s = scale * (q @ k[start:stop].T)
        if causal:
            s = np.where(causal_blocked(tq, stop - start, col0=start), NEG_INF, s)
        m, l, acc = online_softmax_step(m, l, acc, s, v[start:stop])
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return out, lse
