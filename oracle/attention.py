"""Plain fp64 CPU definitions of exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Everything is float64 NumPy.  Inputs are upcast *exactly* from what the GPU
receives (fp32 as is, bf16 -> fp64 is exact), so the oracle sees the same
numbers the kernels see.  Library primitives used as single steps: ``@``
(matrix product), ``np.exp``, ``np.log``, ``max`` and ``sum`` reductions.
Nothing is blocked, fused or reordered beyond what each cited passage states.

Pages (cited by title and section):
  [P1] "FlashAttention 详解：从 Online Softmax 到单遍融合"
  [P2] "01 · IO-awareness、online softmax 与 tiling"
  [P3] "20. FlashAttention Sim | FlashAttention 模拟"
  [P4] "让注意力计算留在片上：分块 Softmax 的计算与访存分析"
  [P5] "FlashAttention 1～4 全解汇总"

Readings taken where the pages are silent or disagree:
  * the scale multiplies the logits, S = scale * Q K^T ([P2] §1 writes the
    scaled S; [P4] §01 likewise), and LSE is in scaled-logit units;
  * LSE = m + ln(l) uses the natural logarithm ([P2] §3, [P5] FA2 step 4);
  * causal masking is bottom-right aligned: key j is visible to query i iff
    j <= i + (Nk - Nq) (the pages never fix it; for Nq == Nk it is j <= i);
  * a local window (wl, wr) keeps key j for query i iff
    i + off - wl <= j <= i + off + wr with off = Nk - Nq, either side
    unbounded when None: the pages define no window; this is the plainest
    extension of the causal rule (causal is (None, 0), a sliding window of W
    keys is (W - 1, 0));
  * a query row with no visible key has O = 0 and LSE = -inf, and contributes
    nothing to the gradients;
  * a variable-length batch packs each head's sequences along the token axis,
    [H, T, d] with sequence b at rows cu[b] .. cu[b+1]-1; every sequence
    attends within itself under the causal or window rule taken over its own
    lengths: the pages name variable-length masks but fix no layout, and
    head-major packing keeps each head's rows contiguous as the fixed-length
    [B, H, N, d] layout does.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# masking
# ----------------------------------------------------------------------------
def window_bounds(causal: bool, window):
    """(wl, wr) of the mask: ``window`` itself when given (then ``causal``
    must be False), else (None, 0) for causal and (None, None) otherwise."""
    if window is None:
        return (None, 0) if causal else (None, None)
    if causal:
        raise ValueError("give either causal or a window, not both")
    wl, wr = window
    for w in (wl, wr):
        if w is not None and w < 0:
            raise ValueError("window sides are None (unbounded) or >= 0")
    return wl, wr


def visible_mask(Nq: int, Nk: int, causal: bool, rows=None, window=None) -> np.ndarray:
    """Boolean [len(rows), Nk]: True where key j is visible to query i.

    Non-causal: every key is visible.  Causal ([P2] §3 'apply_mask'): key j is
    visible to query i iff j <= i + (Nk - Nq) (bottom-right alignment, the
    reading taken here; it is j <= i when Nq == Nk).  Window (wl, wr): iff
    i + off - wl <= j <= i + off + wr, off = Nk - Nq, a None side unbounded.
    """
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    wl, wr = window_bounds(causal, window)
    j = np.arange(Nk)[None, :]
    diag = rows[:, None] + (Nk - Nq)
    ok = np.ones((rows.size, Nk), dtype=bool)
    if wr is not None:
        ok &= j <= diag + wr
    if wl is not None:
        ok &= j >= diag - wl
    return ok


# ----------------------------------------------------------------------------
# safe softmax over one vector
# ----------------------------------------------------------------------------
def softmax(x) -> np.ndarray:
    """Safe softmax of a vector, [P1] §4.3 eqs. (2)-(4): subtract the maximum,
    exponentiate, divide by the sum.  Subtracting the maximum leaves the result
    unchanged (shift invariance, [P1] appendix A.1)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


# ----------------------------------------------------------------------------
# the definition: materialise S and P (one head)
# ----------------------------------------------------------------------------
def _head_forward(q, k, v, scale, causal, rows, window=None):
    """One head.  q [r, d] holds the query rows ``rows`` of a sequence of
    length Nq; k [Nk, d]; v [Nk, dv].  Returns (O [r, dv], LSE [r], P [r, Nk]).

    [P2] §1: S = scale * Q K^T, P = row softmax(S), O = P V.
    [P2] §3 / [P5] FA2 step 4: LSE = m + log(l) with m the row max and
    l = sum_j exp(S_ij - m).
    """
    Nq, Nk = rows[1], k.shape[0]
    idx = rows[0]
    S = scale * (q @ k.T)
    S = np.where(visible_mask(Nq, Nk, causal, idx, window), S, NEG_INF)
    m = np.max(S, axis=1) if Nk > 0 else np.full(q.shape[0], NEG_INF)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])
    l = np.sum(E, axis=1)
    l_safe = np.where(empty, 1.0, l)
    P = E / l_safe[:, None]
    P[empty] = 0.0
    O = P @ v
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m_safe + np.log(l_safe))
    return O, lse, P


def _as_f64(*arrs):
    return [np.asarray(a, dtype=np.float64) for a in arrs]


def attention_forward(q, k, v, scale: float, causal: bool, window=None):
    """O and LSE for q [..., Nq, d], k [..., Nk, d], v [..., Nk, dv].

    Leading dimensions (batch, head) are independent ([P1] §4.1: attention is
    fully parallel over batch and head).  Returns (O [..., Nq, dv],
    LSE [..., Nq]) in float64.
    """
    q, k, v = _as_f64(q, k, v)
    lead = q.shape[:-2]
    Nq, dv = q.shape[-2], v.shape[-1]
    O = np.empty(lead + (Nq, dv))
    L = np.empty(lead + (Nq,))
    for ix in np.ndindex(*lead):
        O[ix], L[ix], _ = _head_forward(q[ix], k[ix], v[ix], scale, causal,
                                        (np.arange(Nq), Nq), window)
    return O, L


def attention_forward_rows(q, k, v, scale: float, causal: bool, rows, window=None):
    """Like ``attention_forward`` but only for the query indices ``rows``
    (the same rows for every head).  q is the full [..., Nq, d] tensor; the
    result holds O [..., len(rows), dv] and LSE [..., len(rows)].  Used where
    materialising all Nq rows would be too slow."""
    rows = np.asarray(rows, dtype=np.int64)
    lead = q.shape[:-2]
    Nq, dv = q.shape[-2], v.shape[-1]
    O = np.empty(lead + (rows.size, dv))
    L = np.empty(lead + (rows.size,))
    for ix in np.ndindex(*lead):
        qh, kh, vh = _as_f64(q[ix][rows], k[ix], v[ix])
        O[ix], L[ix], _ = _head_forward(qh, kh, vh, scale, causal, (rows, Nq), window)
    return O, L


def attention_backward(q, k, v, do, scale: float, causal: bool, window=None):
    """Gradients of sum(dO * O) w.r.t. Q, K, V, by [P2] §5:
        dV = P^T dO;  dP = dO V^T;  D = rowsum(dO * O);
        dS = P * (dP - D);  dQ = scale * dS K;  dK = scale * dS^T Q.
    P and O are the oracle's own fp64 values from the plain definition.
    Rows with no visible key have P = 0 and so contribute nothing.
    Returns (dq, dk, dv, O, LSE, D)."""
    q, k, v, do = _as_f64(q, k, v, do)
    lead = q.shape[:-2]
    Nq = q.shape[-2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dvv = np.empty_like(v)
    O = np.empty(lead + (Nq, v.shape[-1]))
    L = np.empty(lead + (Nq,))
    D = np.empty(lead + (Nq,))
    for ix in np.ndindex(*lead):
        Oh, Lh, P = _head_forward(q[ix], k[ix], v[ix], scale, causal,
                                  (np.arange(Nq), Nq), window)
        dOh = do[ix]
        dvv[ix] = P.T @ dOh
        dP = dOh @ v[ix].T
        Dh = np.sum(dOh * Oh, axis=1)
        dS = P * (dP - Dh[:, None])
        dq[ix] = scale * (dS @ k[ix])
        dk[ix] = scale * (dS.T @ q[ix])
        O[ix], L[ix], D[ix] = Oh, Lh, Dh
    return dq, dk, dvv, O, L, D


# ----------------------------------------------------------------------------
# variable-length batches (packed sequences)
# ----------------------------------------------------------------------------
def _sequence_bounds(cu, total: int, name: str) -> np.ndarray:
    """Validated offsets: cu[0] = 0, non-decreasing, cu[-1] <= total."""
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > total:
        raise ValueError(f"{name} must start at 0, never decrease and end at most at {total}")
    return cu


def varlen_forward(q, k, v, cu_q, cu_k, scale: float, causal: bool, window=None):
    """A batch of B sequences of different lengths, packed along the token
    axis ([P2] §3 lists variable-length batches among the masks of its tiled
    forward; the pages fix no layout).  q [H, Tq, d] holds sequence b's query
    rows at cu_q[b] .. cu_q[b+1]-1, k and v [H, Tk, d] its keys at
    cu_k[b] .. cu_k[b+1]-1.  Each sequence attends only within itself, with
    the causal or window rule of ``visible_mask`` taken over its own lengths
    (offset Lk_b - Lq_b).  Rows outside every sequence have no defined value
    and are returned as NaN.  Returns (O [H, Tq, dv], LSE [H, Tq])."""
    q, k, v = _as_f64(q, k, v)
    H, Tq = q.shape[0], q.shape[1]
    cu_q = _sequence_bounds(cu_q, Tq, "cu_q")
    cu_k = _sequence_bounds(cu_k, k.shape[1], "cu_k")
    if cu_q.size != cu_k.size:
        raise ValueError("cu_q and cu_k must describe the same number of sequences")
    O = np.full((H, Tq, v.shape[-1]), np.nan)
    L = np.full((H, Tq), np.nan)
    for b in range(cu_q.size - 1):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        O[:, qs], L[:, qs] = attention_forward(q[:, qs], k[:, ks], v[:, ks], scale, causal, window)
    return O, L


def varlen_backward(q, k, v, do, cu_q, cu_k, scale: float, causal: bool, window=None):
    """Gradients of sum(dO * O) for ``varlen_forward``: each sequence's
    gradients are those of ``attention_backward`` on its own rows; rows
    outside every sequence are NaN.  Returns (dq, dk, dv)."""
    q, k, v, do = _as_f64(q, k, v, do)
    cu_q = _sequence_bounds(cu_q, q.shape[1], "cu_q")
    cu_k = _sequence_bounds(cu_k, k.shape[1], "cu_k")
    if cu_q.size != cu_k.size:
        raise ValueError("cu_q and cu_k must describe the same number of sequences")
    dq, dk, dvv = np.full_like(q, np.nan), np.full_like(k, np.nan), np.full_like(v, np.nan)
    for b in range(cu_q.size - 1):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        dq[:, qs], dk[:, ks], dvv[:, ks], *_ = attention_backward(
            q[:, qs], k[:, ks], v[:, ks], do[:, qs], scale, causal, window)
    return dq, dk, dvv


# ----------------------------------------------------------------------------
# the online recurrence (second, independent formulation)
# ----------------------------------------------------------------------------
def online_rescale(m, l, block_max, block_sum_at_new_max=0.0):
    """One step of the online-softmax state update for a row, [P2] §2 and
    [P4] §02:  m' = max(m, block max);  alpha = exp(m - m');
    l' = alpha * l + (sum over the new block of exp(s - m')).
    Returns (m', alpha, l')."""
    m_new = max(m, block_max)
    alpha = np.exp(m - m_new)
    return m_new, alpha, alpha * l + block_sum_at_new_max


def tiled_forward(q, k, v, scale: float, causal: bool, block_q: int,
                  block_k: int, trace: bool = False, window=None):
    """FA2 forward recurrence with deferred normalisation ([P2] §3; [P5]
    FlashAttention-2 algorithm), for one head: q [Nq, d], k [Nk, d], v [Nk, dv].

    For each query block Q_i (m = -inf, l = 0, O~ = 0), for each key block j:
        S = scale * Q_i K_j^T, masked;  m_new = max(m, rowmax S);
        P~ = exp(S - m_new);  alpha = exp(m - m_new);
        l = alpha * l + rowsum P~;  O~ = alpha * O~ + P~ V_j;  m = m_new.
    Finally O_i = O~ / l and LSE_i = m + log(l).  A row whose keys seen so far
    are all masked keeps its initial state (m = -inf, nothing accumulated).
    With ``trace`` it also returns, per query block, the list of (m, l, O~)
    after every key block.
    """
    q, k, v = _as_f64(q, k, v)
    Nq, Nk = q.shape[0], k.shape[0]
    dv = v.shape[1]
    O = np.zeros((Nq, dv))
    L = np.full(Nq, NEG_INF)
    traces = []
    for i0 in range(0, Nq, block_q):
        rows = np.arange(i0, min(i0 + block_q, Nq))
        Qi = q[rows]
        m = np.full(rows.size, NEG_INF)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, dv))
        tr = []
        for j0 in range(0, Nk, block_k):
            cols = slice(j0, min(j0 + block_k, Nk))
            S = scale * (Qi @ k[cols].T)
            vis = visible_mask(Nq, Nk, causal, rows, window)[:, cols]
            S = np.where(vis, S, NEG_INF)
            m_new = np.maximum(m, np.max(S, axis=1))
            live = np.isfinite(m_new)
            base = np.where(live, m_new, 0.0)
            P = np.exp(S - base[:, None])
            alpha = np.where(live, np.exp(m - base), 1.0)
            l = alpha * l + np.sum(P, axis=1)
            acc = alpha[:, None] * acc + P @ v[cols]
            m = m_new
            if trace:
                tr.append((m.copy(), l.copy(), acc.copy()))
        live = l > 0
        O[rows] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            L[rows] = np.where(live, m + np.log(np.where(live, l, 1.0)), NEG_INF)
        traces.append(tr)
    if trace:
        return O, L, traces
    return O, L


def tiled_forward_renormalised(q, k, v, scale: float, causal: bool,
                               block_q: int, block_k: int, window=None):
    """Tiled forward that keeps the accumulator *normalised* after every key
    block ([P1] §4.6 with eq. (9); [P3] Step 1 update formulas):
        l_new = l * exp(m - m_new) + rowsum exp(S - m_new)
        o_new = o * (l * exp(m - m_new) / l_new) + exp(S - m_new) V / l_new
    One head; returns (O, LSE).  Equal to ``tiled_forward`` in exact
    arithmetic (the pages' "delay the rescale" remark, [P2] §2)."""
    q, k, v = _as_f64(q, k, v)
    Nq, Nk = q.shape[0], k.shape[0]
    O = np.zeros((Nq, v.shape[1]))
    L = np.full(Nq, NEG_INF)
    for i0 in range(0, Nq, block_q):
        rows = np.arange(i0, min(i0 + block_q, Nq))
        Qi = q[rows]
        m = np.full(rows.size, NEG_INF)
        l = np.zeros(rows.size)
        o = np.zeros((rows.size, v.shape[1]))
        for j0 in range(0, Nk, block_k):
            cols = slice(j0, min(j0 + block_k, Nk))
            S = scale * (Qi @ k[cols].T)
            S = np.where(visible_mask(Nq, Nk, causal, rows, window)[:, cols], S, NEG_INF)
            m_new = np.maximum(m, np.max(S, axis=1))
            live = np.isfinite(m_new)
            base = np.where(live, m_new, 0.0)
            E = np.exp(S - base[:, None])
            carried = np.where(live, l * np.exp(m - base), 0.0)
            l_new = carried + np.sum(E, axis=1)
            denom = np.where(l_new > 0, l_new, 1.0)
            o = o * (carried / denom)[:, None] + (E @ v[cols]) / denom[:, None]
            m, l = m_new, l_new
        O[rows] = o
        with np.errstate(divide="ignore"):
            L[rows] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return O, L


def attention_flops(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool,
                    window=None) -> int:
    """Forward FLOPs counted over visible (query, key) pairs only: two
    products of 2*d FLOPs per pair ([P2] §1: the work sits in the two
    matrix products).  Counts pairs with ``visible_mask``'s rule: query i
    sees the keys [i + off - wl, i + off + wr] clipped to [0, Nk)."""
    wl, wr = window_bounds(causal, window)
    off = Nk - Nq
    i = np.arange(Nq, dtype=np.int64)
    hi = np.full(Nq, Nk, dtype=np.int64) if wr is None else np.clip(i + off + wr + 1, 0, Nk)
    lo = np.zeros(Nq, dtype=np.int64) if wl is None else np.clip(i + off - wl, 0, Nk)
    pairs = int(np.sum(np.maximum(hi - lo, 0)))
    return 4 * d * pairs * B * H
