"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: values printed on the
pages (tests/golden/*.json, each citing its page and section), closed forms,
invariants, central finite differences and library routines (torch's fp64
softmax / scaled_dot_product_attention / autograd).  Each group is chosen so a
plausible slip in the oracle -- a dropped alpha, a wrong sign in dS, a
transposed operand, a wrong mask offset -- fails at least one test.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import (attention_backward, attention_forward, attention_forward_rows,
                    online_rescale, softmax, tiled_forward,
                    tiled_forward_renormalised, visible_mask)


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- page pins
def test_p4_worked_row_plain_and_tiled(golden):
    g = golden("p4_tiled_row.json")
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    # the row as attention: q = e1, k_j = (score_j, 0), scale 1
    q = np.array([[1.0, 0.0]])
    K = np.array([[s, 0.0] for s in g["scores"]])
    V = np.array(g["values"])
    O, L = attention_forward(q, K, V, 1.0, False)
    assert np.max(np.abs(O[0] - g["output"])) <= tol
    for tile in (1, 2, 3, 4):
        Ot, Lt = tiled_forward(q, K, V, 1.0, False, 1, tile)
        assert np.max(np.abs(Ot - O)) <= 1e-12
        assert abs(Lt[0] - L[0]) <= 1e-12
        Or, Lr = tiled_forward_renormalised(q, K, V, 1.0, False, 1, tile)
        assert np.max(np.abs(Or - O)) <= 1e-12
        assert abs(Lr[0] - L[0]) <= 1e-12
    # state after the first key block of size 2
    _, _, tr = tiled_forward(q, K, V, 1.0, False, 1, g["tile"], trace=True)
    m1, l1, acc1 = tr[0][0]
    st = g["after_first_block"]
    assert abs(m1[0] - st["m"]) <= tol
    assert abs(l1[0] - st["l"]) <= tol
    assert np.max(np.abs(acc1[0] - st["acc"])) <= tol
    # LSE from the definition: log sum exp of the scores
    assert abs(L[0] - math.log(sum(math.exp(s) for s in g["scores"]))) <= 1e-12


def test_p2_rescale_numbers(golden):
    g = golden("p2_rescale.json")
    tol = g["printed_abs_tol"]
    m_new, alpha, l_folded = online_rescale(g["m"], g["l"], g["block_max"], 0.0)
    assert m_new == g["m_new"]
    assert abs(alpha - g["alpha"]) <= tol["alpha"]
    assert abs(l_folded - g["l_folded"]) <= tol["l_folded"]
    assert abs(alpha - math.exp(-2.0)) <= 1e-15


def test_p2_rescale_inside_tiled_recurrence(golden):
    """Drive tiled_forward through the page's state: after a first block of
    ten scores equal to 3 the state is m=3, l=10; a second block whose max is
    5 must fold l to 10*alpha before adding its own sum."""
    g = golden("p2_rescale.json")
    scores = [3.0] * 10 + [5.0]
    q = np.array([[1.0]])
    K = np.array([[s] for s in scores])
    V = np.ones((11, 1))
    _, _, tr = tiled_forward(q, K, V, 1.0, False, 1, 10, trace=True)
    (m1, l1, _), (m2, l2, _) = tr[0]
    assert m1[0] == g["m"] and abs(l1[0] - g["l"]) <= 1e-12
    assert m2[0] == g["m_new"]
    folded = l2[0] - 1.0           # the new block contributes exp(5-5) = 1
    assert abs(folded - g["l_folded"]) <= g["printed_abs_tol"]["l_folded"]
    assert abs(folded - 10.0 * math.exp(-2.0)) <= 1e-12


def test_p1_softmax_printed_values(golden):
    g = golden("p1_softmax.json")
    for case in g["cases"]:
        x = np.array(case["x"])
        y = softmax(x)
        assert np.all(np.isfinite(y))
        assert np.max(np.abs(y - case["y"])) <= g["printed_abs_tol"]
        # the same numbers through attention: q = e1, K[:,0] = x, V = I
        n = x.size
        q = np.zeros((1, 2)); q[0, 0] = 1.0
        K = np.zeros((n, 2)); K[:, 0] = x
        O, L = attention_forward(q, K, np.eye(n), 1.0, False)
        assert np.max(np.abs(O[0] - case["y"])) <= g["printed_abs_tol"]
        Ot, _ = tiled_forward(q, K, np.eye(n), 1.0, False, 1, 2)
        assert np.max(np.abs(Ot[0] - case["y"])) <= g["printed_abs_tol"]


def test_p1_attention_row_printed_values(golden):
    g = golden("p1_attention_row.json")
    q = np.array([g["q"]])
    K = np.array(g["K"])
    V = np.array(g["V"])
    O, L = attention_forward(q, K, V, 1.0, False)
    assert np.max(np.abs(O[0] - g["output"])) <= g["printed_abs_tol"]
    # the per-key 1-pass recurrence is the block-size-1 case
    O1, L1 = tiled_forward(q, K, V, 1.0, False, 1, 1)
    assert np.max(np.abs(O1[0] - g["output"])) <= g["printed_abs_tol"]
    Or, _ = tiled_forward_renormalised(q, K, V, 1.0, False, 1, 1)
    assert np.max(np.abs(Or[0] - g["output"])) <= g["printed_abs_tol"]
    logits = K @ q[0]
    assert abs(L[0] - math.log(np.sum(np.exp(logits)))) <= 1e-12


def test_p3_seeded_cases_tiled_equals_plain(golden):
    g = golden("p3_seeded_cases.json")
    for c in g["cases"]:
        torch.manual_seed(c["seed"])
        q = torch.randn(c["seq"], c["dim"])
        k = torch.randn(c["seq"], c["dim"])
        v = torch.randn(c["seq"], c["dim"])
        scale = 1.0 / math.sqrt(c["dim"])
        qd, kd, vd = (t.double().numpy() for t in (q, k, v))
        O, L = attention_forward(qd, kd, vd, scale, False)
        Ot, Lt = tiled_forward(qd, kd, vd, scale, False, c["block"], c["block"])
        Or, _ = tiled_forward_renormalised(qd, kd, vd, scale, False, c["block"], c["block"])
        # library routine in fp64: softmax(q k^T scale) v
        ref = torch.softmax((q.double() @ k.double().T) * scale, dim=-1) @ v.double()
        assert np.max(np.abs(O - ref.numpy())) <= 1e-12
        assert np.max(np.abs(Ot - O)) <= 1e-12
        assert np.max(np.abs(Or - O)) <= 1e-12
        assert np.max(np.abs(Lt - L)) <= 1e-12
        assert np.max(np.abs(O - ref.numpy())) < g["page_threshold"]


# ---------------------------------------------------- library-routine checks
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 17, 17, 8), (1, 2, 64, 64, 16), (1, 1, 1, 1, 4)])
def test_forward_matches_torch_sdpa_fp64(shape, causal):
    B, H, Nq, Nk, d = shape
    r = rng(1)
    q, k, v = (r.standard_normal((B, H, n, d)) for n in (Nq, Nk, Nk))
    scale = 0.37
    O, L = attention_forward(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = (tq @ tk.transpose(-1, -2)) * scale
    if causal:  # Nq == Nk here, so top-left and bottom-right alignment agree
        s = s.masked_fill(torch.triu(torch.ones(Nq, Nk, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    assert np.max(np.abs(O - ref.numpy())) <= 1e-12
    assert np.max(np.abs(L - lse.numpy())) <= 1e-12


def test_bottom_right_alignment_when_nq_ne_nk():
    # Nq < Nk: the last query sees every key; query i sees Nk - Nq + i + 1 keys
    m = visible_mask(3, 7, True)
    assert m.sum(axis=1).tolist() == [5, 6, 7]
    # Nq > Nk: the first Nq - Nk queries see nothing
    m = visible_mask(6, 4, True)
    assert m.sum(axis=1).tolist() == [0, 0, 1, 2, 3, 4]
    assert visible_mask(5, 5, True).sum() == 15
    assert visible_mask(5, 9, False).all()


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    r = rng(2)
    N, d = 37, 8
    q, k = r.standard_normal((N, d)) * 3, r.standard_normal((N, d)) * 3
    P, _ = attention_forward(q, k, np.eye(N), 0.5, causal)   # V = I gives O = P
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14
    if causal:
        assert np.all(P[visible_mask(N, N, True) == False] == 0.0)  # noqa: E712


def test_masked_keys_get_zero_weight_bitwise():
    r = rng(3)
    N, d = 29, 8
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    O, L = attention_forward(q, k, v, 0.3, True)
    i0 = 11
    k2, v2 = k.copy(), v.copy()
    k2[i0 + 1:] = r.standard_normal((N - i0 - 1, d)) * 100
    v2[i0 + 1:] = 1e6
    O2, L2 = attention_forward(q, k2, v2, 0.3, True)
    assert np.array_equal(O[: i0 + 1], O2[: i0 + 1])
    assert np.array_equal(L[: i0 + 1], L2[: i0 + 1])


@pytest.mark.parametrize("causal", [False, True])
def test_shift_and_affine_invariance(causal):
    r = rng(4)
    Nq, Nk, d = 19, 23, 8
    scale = 0.25
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, 5))
    O, L = attention_forward(q, k, v, scale, causal)
    u = r.standard_normal(d)
    O2, L2 = attention_forward(q, k + u, v, scale, causal)
    live = np.isfinite(L)
    assert np.max(np.abs(O2 - O)) <= 1e-12
    assert np.max(np.abs((L2 - L)[live] - scale * (q @ u)[live])) <= 1e-12
    c = r.standard_normal(5)
    O3, _ = attention_forward(q, k, v + c, scale, causal)
    assert np.max(np.abs(O3 - (O + c))) <= 1e-12


def test_joint_key_value_permutation_noncausal():
    r = rng(5)
    q, k, v = r.standard_normal((9, 4)), r.standard_normal((13, 4)), r.standard_normal((13, 3))
    perm = r.permutation(13)
    O, L = attention_forward(q, k, v, 1.0, False)
    O2, L2 = attention_forward(q, k[perm], v[perm], 1.0, False)
    assert np.max(np.abs(O - O2)) <= 1e-13 and np.max(np.abs(L - L2)) <= 1e-13


# --------------------------------------------------------------- closed forms
def test_closed_forms():
    r = rng(6)
    d = 6
    q = r.standard_normal((5, d))
    k1, v1 = r.standard_normal((1, d)), r.standard_normal((1, 3))
    O, L = attention_forward(q, k1, v1, 0.7, False)
    assert np.max(np.abs(O - v1)) <= 1e-15
    assert np.max(np.abs(L - 0.7 * (q @ k1[0]))) <= 1e-15
    # K = 0: uniform weights over the visible keys
    N = 12
    q = r.standard_normal((N, d))
    v = r.standard_normal((N, 3))
    O, L = attention_forward(q, np.zeros((N, d)), v, 1.0, True)
    for i in range(N):
        assert np.max(np.abs(O[i] - v[: i + 1].mean(axis=0))) <= 1e-14
        assert abs(L[i] - math.log(i + 1)) <= 1e-14
    # causal row 0 sees only key 0
    O, _ = attention_forward(q, r.standard_normal((N, d)), v, 1.0, True)
    assert np.max(np.abs(O[0] - v[0])) <= 1e-15


def test_empty_rows_when_nq_exceeds_nk():
    r = rng(7)
    q, k, v = r.standard_normal((6, 4)), r.standard_normal((4, 4)), r.standard_normal((4, 4))
    O, L = attention_forward(q, k, v, 1.0, True)
    assert np.all(O[:2] == 0.0) and np.all(np.isneginf(L[:2]))
    assert np.all(np.isfinite(L[2:]))
    Ot, Lt = tiled_forward(q, k, v, 1.0, True, 4, 2)
    assert np.max(np.abs(Ot - O)) <= 1e-12
    assert np.all(np.isneginf(Lt[:2])) and np.max(np.abs(Lt[2:] - L[2:])) <= 1e-12


@pytest.mark.parametrize("bq,bk", [(64, 64), (7, 5), (128, 32), (1, 200)])
def test_tiled_equals_untiled_ragged(bq, bk):
    r = rng(8)
    Nq, Nk, d = 150, 170, 16
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    for causal in (False, True):
        O, L = attention_forward(q, k, v, 0.25, causal)
        Ot, Lt = tiled_forward(q, k, v, 0.25, causal, bq, bk)
        assert np.max(np.abs(Ot - O)) <= 1e-12
        assert np.max(np.abs(Lt - L)) <= 1e-12


def test_row_sampled_forward_agrees():
    r = rng(9)
    q, k, v = (r.standard_normal((2, 3, 40, 8)) for _ in range(3))
    rows = [0, 5, 17, 39]
    O, L = attention_forward(q, k, v, 0.4, True)
    Os, Ls = attention_forward_rows(q, k, v, 0.4, True, rows)
    assert np.array_equal(Os, O[:, :, rows]) and np.array_equal(Ls, L[:, :, rows])


def test_large_logits_do_not_overflow():
    q = np.zeros((1, 2)); q[0, 0] = 1.0
    K = np.zeros((3, 2)); K[:, 0] = [1000.0, 1001.0, 1002.0]
    O, L = attention_forward(q, K, np.eye(3), 1.0, False)
    assert np.all(np.isfinite(O)) and np.isfinite(L[0])
    assert abs(L[0] - (1002.0 + math.log(1 + math.exp(-1) + math.exp(-2)))) <= 1e-12


# ------------------------------------------------------------------ backward
def _loss(q, k, v, do, scale, causal):
    O, _ = attention_forward(q, k, v, scale, causal)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(5, 7, 3, 2), (6, 4, 4, 4), (8, 8, 2, 3)])
def test_backward_finite_differences(shape, causal):
    Nq, Nk, d, dv = shape
    r = rng(10)
    q, k = r.standard_normal((Nq, d)), r.standard_normal((Nk, d))
    v, do = r.standard_normal((Nk, dv)), r.standard_normal((Nq, dv))
    scale = 0.6
    dq, dk, dvv, *_ = attention_backward(q, k, v, do, scale, causal)
    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dvv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _loss(q, k, v, do, scale, causal)
            X[idx] = old - h
            fm = _loss(q, k, v, do, scale, causal)
            X[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - G)) <= 1e-7 * max(1.0, np.max(np.abs(G)))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    r = rng(11)
    B, H, N, d = 2, 2, 33, 8
    q, k, v, do = (r.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 1 / math.sqrt(d)
    dq, dk, dvv, O, L, D = attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    s = (tq @ tk.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    out.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dvv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-12
    assert np.max(np.abs(O - out.detach().numpy())) <= 1e-12
    assert np.max(np.abs(D - np.sum(do * O, axis=-1))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    r = rng(12)
    Nq, Nk, d = 21, 21, 6
    q, k, v, do = (r.standard_normal((n, d)) for n in (Nq, Nk, Nk, Nq))
    dq, dk, dvv, *_ = attention_backward(q, k, v, do, 0.5, causal)
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12          # rows of dS sum to 0
    assert np.max(np.abs(dvv.sum(axis=0) - do.sum(axis=0))) <= 1e-12
    u = r.standard_normal(d)
    dq2, *_ = attention_backward(q, k + u, v, do, 0.5, causal)
    assert np.max(np.abs(dq2 - dq)) <= 1e-12


def test_backward_empty_rows_contribute_nothing():
    r = rng(13)
    q, do = r.standard_normal((6, 4)), r.standard_normal((6, 4))
    k, v = r.standard_normal((4, 4)), r.standard_normal((4, 4))
    dq, dk, dvv, *_ = attention_backward(q, k, v, do, 1.0, True)
    assert np.all(dq[:2] == 0.0)
    do2 = do.copy(); do2[:2] = 123.0
    q2 = q.copy(); q2[:2] = -50.0
    _, dk2, dv2, *_ = attention_backward(q2, k, v, do2, 1.0, True)
    assert np.array_equal(dk, dk2) and np.array_equal(dvv, dv2)


def test_flop_count_matches_mask():
    for (Nq, Nk, causal) in [(64, 64, True), (30, 70, True), (70, 30, True), (33, 65, False)]:
        pairs = int(visible_mask(Nq, Nk, causal).sum())
        assert oracle.attention_flops(2, 3, Nq, Nk, 16, causal) == 4 * 16 * pairs * 6


# ------------------------------------------------------ local window (f4)
# Windows (wl, wr): key j visible to query i iff i+off-wl <= j <= i+off+wr,
# off = Nk - Nq, None = unbounded (the reading documented in oracle.attention).
WINDOWS = [(3, 0), (0, 0), (5, 2), (None, 1), (2, None), (40, 0), (0, 7)]


def _brute_window_row(qi, K, V, scale, lo, hi):
    """One row by explicit enumeration of the visible keys, math.exp only."""
    keys = [j for j in range(K.shape[0]) if lo <= j <= hi]
    if not keys:
        return np.zeros(V.shape[1]), -math.inf
    s = [scale * float(np.dot(qi, K[j])) for j in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    tot = sum(w)
    out = sum(wj * V[j] for wj, j in zip(w, keys)) / tot
    return out, m + math.log(tot)


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("Nq,Nk", [(9, 9), (5, 11), (11, 5)])
def test_window_forward_brute_force(window, Nq, Nk):
    r = rng(20)
    d = 3
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, 2))
    O, L = attention_forward(q, k, v, 0.8, False, window=window)
    wl, wr = window
    off = Nk - Nq
    for i in range(Nq):
        lo = -10**9 if wl is None else i + off - wl
        hi = 10**9 if wr is None else i + off + wr
        o_ref, l_ref = _brute_window_row(q[i], k, v, 0.8, lo, hi)
        assert np.max(np.abs(O[i] - o_ref)) <= 1e-12
        assert (L[i] == l_ref == -math.inf) or abs(L[i] - l_ref) <= 1e-12


@pytest.mark.parametrize("window", [(4, 0), (2, 3), (7, 1)])
def test_window_equals_unmasked_attention_on_the_slice(window):
    # each row's result is the plain (unmasked) definition over its key slice
    r = rng(21)
    Nq, Nk, d = 13, 17, 4
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    O, L = attention_forward(q, k, v, 0.5, False, window=window)
    wl, wr = window
    off = Nk - Nq
    for i in range(Nq):
        lo, hi = max(0, i + off - wl), min(Nk - 1, i + off + wr)
        Os, Ls = attention_forward(q[i:i + 1], k[lo:hi + 1], v[lo:hi + 1], 0.5, False)
        assert np.max(np.abs(O[i] - Os[0])) <= 1e-13
        assert abs(L[i] - Ls[0]) <= 1e-13


def test_window_closed_forms_and_limits():
    r = rng(22)
    Nq, Nk, d = 6, 9, 5
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    off = Nk - Nq
    # a window of one key: O_i = V_{i+off}, LSE_i = scale * q_i . k_{i+off}
    O, L = attention_forward(q, k, v, 0.7, False, window=(0, 0))
    for i in range(Nq):
        assert np.max(np.abs(O[i] - v[i + off])) <= 1e-14
        assert abs(L[i] - 0.7 * float(q[i] @ k[i + off])) <= 1e-14
    # unbounded left with right bound 0 is causal; bounds past the sequence change nothing
    Oc, Lc = attention_forward(q, k, v, 0.7, True)
    Ow, Lw = attention_forward(q, k, v, 0.7, False, window=(Nk + Nq, 0))
    assert np.array_equal(Oc, Ow) and np.array_equal(Lc, Lw)
    On, Ln = attention_forward(q, k, v, 0.7, False)
    Ow, Lw = attention_forward(q, k, v, 0.7, False, window=(Nk + Nq, Nk + Nq))
    assert np.array_equal(On, Ow) and np.array_equal(Ln, Lw)
    # rows whose window lies wholly outside the keys are empty
    O, L = attention_forward(q, k[:2], v[:2], 0.7, False, window=(1, 0))
    off2 = 2 - Nq
    for i in range(Nq):
        if i + off2 + 0 < 0 or i + off2 - 1 > 1:
            assert np.all(O[i] == 0.0) and L[i] == -math.inf
    with pytest.raises(ValueError):
        attention_forward(q, k, v, 0.7, True, window=(1, 0))
    with pytest.raises(ValueError):
        attention_forward(q, k, v, 0.7, False, window=(-1, 0))


def test_window_keys_outside_do_not_matter_bitwise():
    r = rng(23)
    Nq, Nk, d = 16, 16, 4
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    O, L = attention_forward(q, k, v, 0.9, False, window=(3, 1))
    k2, v2 = k.copy(), v.copy()
    i = 10            # row 10 sees keys 7..11
    for j in list(range(0, 7)) + list(range(12, Nk)):
        k2[j] += 100.0
        v2[j] -= 7.0
    O2, L2 = attention_forward(q, k2, v2, 0.9, False, window=(3, 1))
    assert np.array_equal(O[i], O2[i]) and L[i] == L2[i]


@pytest.mark.parametrize("window", [(2, 0), (1, 2), (None, 1)])
def test_window_backward_finite_differences(window):
    r = rng(24)
    Nq, Nk, d, dv = 6, 7, 3, 2
    q, k = r.standard_normal((Nq, d)), r.standard_normal((Nk, d))
    v, do = r.standard_normal((Nk, dv)), r.standard_normal((Nq, dv))
    scale = 0.6
    dq, dk, dvv, *_ = attention_backward(q, k, v, do, scale, False, window=window)

    def loss():
        O, _ = attention_forward(q, k, v, scale, False, window=window)
        return float(np.sum(O * do))

    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dvv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = loss()
            X[idx] = old - h
            fm = loss()
            X[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - G)) <= 1e-7 * max(1.0, np.max(np.abs(G)))


def test_window_backward_matches_torch_autograd_fp64():
    r = rng(25)
    N, d, wl, wr = 29, 6, 5, 2
    q, k, v, do = (r.standard_normal((1, 2, N, d)) for _ in range(4))
    scale = 1 / math.sqrt(d)
    dq, dk, dvv, O, L, D = attention_backward(q, k, v, do, scale, False, window=(wl, wr))
    hide = torch.ones(N, N, dtype=torch.bool)   # True = masked, built row by row
    for i in range(N):
        for j in range(max(0, i - wl), min(N, i + wr + 1)):
            hide[i, j] = False
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    s = ((tq @ tk.transpose(-1, -2)) * scale).masked_fill(hide, float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    out.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dvv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-12
    assert np.max(np.abs(L - torch.logsumexp(s, dim=-1).detach().numpy())) <= 1e-12


@pytest.mark.parametrize("bq,bk", [(4, 3), (64, 64), (5, 16)])
def test_window_tiled_equals_untiled(bq, bk):
    r = rng(26)
    Nq, Nk, d = 37, 45, 8
    q, k, v = r.standard_normal((Nq, d)), r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    for window in [(6, 0), (3, 4), (None, 2)]:
        O, L = attention_forward(q, k, v, 0.4, False, window=window)
        Ot, Lt = tiled_forward(q, k, v, 0.4, False, bq, bk, window=window)
        Or, Lr = tiled_forward_renormalised(q, k, v, 0.4, False, bq, bk, window=window)
        assert np.max(np.abs(Ot - O)) <= 1e-12 and np.max(np.abs(Or - O)) <= 1e-12
        fin = np.isfinite(L)
        assert np.array_equal(fin, np.isfinite(Lt)) and np.max(np.abs(Lt[fin] - L[fin])) <= 1e-12


def test_window_flop_count_matches_mask():
    for (Nq, Nk, window) in [(64, 64, (15, 0)), (30, 70, (3, 5)), (70, 30, (None, 2)), (33, 33, (4, None))]:
        pairs = int(visible_mask(Nq, Nk, False, window=window).sum())
        assert oracle.attention_flops(2, 3, Nq, Nk, 16, False, window=window) == 4 * 16 * pairs * 6


# ------------------------------------------------------- variable-length batches
def _packed(r, lens_q, lens_k, H=2, d=6, pad_q=0, pad_k=0):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    Tq, Tk = int(cu_q[-1]) + pad_q, int(cu_k[-1]) + pad_k
    q = r.standard_normal((H, Tq, d))
    k = r.standard_normal((H, Tk, d))
    v = r.standard_normal((H, Tk, d))
    do = r.standard_normal((H, Tq, d))
    return q, k, v, do, cu_q, cu_k


def _block_mask(cu_q, cu_k, causal, window):
    """True = visible, built key by key over the whole packed batch: the key
    must belong to the query's own sequence, and inside it pass the causal or
    window bound measured from that sequence's bottom-right diagonal."""
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    wl, wr = (None, 0) if causal else (window if window is not None else (None, None))
    vis = torch.zeros(Tq, Tk, dtype=torch.bool)
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            for j in range(lk):
                diag = i + lk - lq
                if (wr is None or j <= diag + wr) and (wl is None or j >= diag - wl):
                    vis[cu_q[b] + i, cu_k[b] + j] = True
    return vis


VARLEN = [
    # query lengths, key lengths, causal, window
    ([5, 1, 9], [5, 1, 9], True, None),
    ([4, 7, 3], [6, 2, 8], False, None),
    ([3, 8, 6], [9, 5, 6], True, None),          # Nq != Nk both ways: empty rows
    ([6, 6, 10], [6, 9, 4], False, (2, 1)),
    ([0, 5, 4], [3, 0, 4], False, (None, 0)),    # empty sequences on either side
]


@pytest.mark.parametrize("lens_q,lens_k,causal,window", VARLEN)
def test_varlen_forward_matches_block_masked_torch(lens_q, lens_k, causal, window):
    # one attention over the whole packed batch with a block-diagonal mask,
    # through torch's fp64 softmax and logsumexp (a library routine)
    r = rng(40 + sum(lens_q))
    q, k, v, _, cu_q, cu_k = _packed(r, lens_q, lens_k)
    O, L = oracle.varlen_forward(q, k, v, cu_q, cu_k, 0.45, causal, window)
    vis = _block_mask(cu_q, cu_k, causal, window)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    s = ((tq @ tk.transpose(-1, -2)) * 0.45).masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)   # rows with no key: P = 0
    ref = p @ tv
    assert np.max(np.abs(O - ref.numpy())) <= 1e-12
    fin = np.isfinite(lse.numpy())
    assert np.array_equal(np.isfinite(L), fin)
    assert np.max(np.abs(L[fin] - lse.numpy()[fin]), initial=0.0) <= 1e-12
    assert np.all(O[~np.broadcast_to(fin[..., None], O.shape)] == 0.0)


@pytest.mark.parametrize("lens_q,lens_k,causal,window", VARLEN[:4])
def test_varlen_backward_matches_block_masked_autograd(lens_q, lens_k, causal, window):
    r = rng(60 + sum(lens_k))
    q, k, v, do, cu_q, cu_k = _packed(r, lens_q, lens_k)
    dq, dk, dvv = oracle.varlen_backward(q, k, v, do, cu_q, cu_k, 0.3, causal, window)
    vis = _block_mask(cu_q, cu_k, causal, window)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    s = ((tq @ tk.transpose(-1, -2)) * 0.3).masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.where(vis.any(dim=-1, keepdim=True), p, torch.zeros_like(p))
    (p @ tv).backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dvv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-12


def test_varlen_equal_lengths_is_the_fixed_length_batch():
    r = rng(70)
    B, H, N, d = 3, 2, 11, 5
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    O, L = attention_forward(q, k, v, 0.5, True)
    pack = lambda x: x.transpose(1, 0, 2, 3).reshape(H, B * N, d)   # [B,H,N,d] -> [H, B*N, d]
    cu = np.arange(B + 1) * N
    Ov, Lv = oracle.varlen_forward(pack(q), pack(k), pack(v), cu, cu, 0.5, True)
    assert np.array_equal(Ov, pack(O))
    assert np.array_equal(Lv, L.transpose(1, 0, 2).reshape(H, B * N))


def test_varlen_sequence_order_and_padding():
    r = rng(71)
    lens = [4, 9, 2]
    q, k, v, _, cu, _ = _packed(r, lens, lens, pad_q=3, pad_k=2)
    O, L = oracle.varlen_forward(q, k, v, cu, cu, 0.6, True)
    # trailing rows outside every sequence have no value
    assert np.all(np.isnan(O[:, cu[-1]:])) and np.all(np.isnan(L[:, cu[-1]:]))
    # reversing the order of the sequences reverses the order of their outputs
    order = [2, 1, 0]
    seg = lambda x, b: x[:, cu[b]:cu[b + 1]]
    q2, k2, v2 = (np.concatenate([seg(x, b) for b in order], axis=1) for x in (q, k, v))
    cu2 = np.concatenate([[0], np.cumsum([lens[b] for b in order])])
    O2, L2 = oracle.varlen_forward(q2, k2, v2, cu2, cu2, 0.6, True)
    for pos, b in enumerate(order):
        assert np.array_equal(O2[:, cu2[pos]:cu2[pos + 1]], seg(O, b))
        assert np.array_equal(L2[:, cu2[pos]:cu2[pos + 1]], seg(L, b))
    with pytest.raises(ValueError):
        oracle.varlen_forward(q, k, v, [0, 5, 3], [0, 5, 3], 0.6, True)
    with pytest.raises(ValueError):
        oracle.varlen_forward(q, k, v, [1, 5], [1, 5], 0.6, True)
