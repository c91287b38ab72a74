"""GPU parity of the local-window entry points (fa_fwd_window, fa_bwd_window)
against the fp64 oracle (MI355X only).

Key j is visible to query i iff i + off - wl <= j <= i + off + wr with
off = Nk - Nq, a side None (-1 in the C ABI) unbounded.  The cases cover
windows narrower than one key tile, windows that straddle several tiles on
both sides, one-sided windows, windows wider than the sequence, Nq != Nk in
both directions (rows that see no key), ragged tails, both head dims and
both dtypes; the full-size sliding-window workload is checked on sampled
rows.  Windows (None, 0) and (None, None) must reproduce the causal and
unmasked calls bitwise, and so must a bounded window wide enough to hide
nothing (it runs the window kernels, which then skip no tile and mask no
extra key).
"""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_backward, attention_forward, attention_forward_rows
from parity import check_forward, check_grad, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_fwd(q, k, v, scale, window=None, causal=False):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.attention_forward(qd, kd, vd, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return o, lse


def gpu_fwd_bwd(q, k, v, do, scale, window=None, causal=False, deterministic=False):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention_forward(qd, kd, vd, scale=scale, causal=causal, window=window)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal,
                                       window=window, deterministic=deterministic)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


FWD = [
    # B, H, Nq, Nk, d, dtype, window
    (1, 2, 300, 300, 64, "bf16", (16, 0)),          # narrower than a key tile
    (1, 2, 300, 300, 128, "bf16", (0, 0)),          # the diagonal alone
    (2, 2, 333, 333, 128, "bf16", (100, 50)),       # two-sided, several tiles
    (1, 3, 257, 400, 64, "bf16", (None, 7)),        # Nk > Nq, right reach only
    (1, 2, 400, 257, 128, "bf16", (5, None)),       # Nq > Nk, left reach only
    (1, 2, 500, 200, 64, "bf16", (31, 0)),          # Nq > Nk: leading rows empty
    (1, 1, 130, 130, 64, "bf16", (1000, 1000)),     # wider than the sequence
    (1, 2, 700, 700, 128, "bf16", (255, 0)),        # window = 4 key tiles
    (1, 2, 77, 190, 64, "fp32", (20, 3)),
    (1, 1, 200, 200, 128, "fp32", (64, 0)),
    (1, 2, 150, 90, 128, "fp32", (None, 0)),        # = causal
    (1, 1, 1, 1, 64, "bf16", (0, 0)),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "-".join(map(str, c)))
def test_window_forward_small_and_ragged(case):
    B, H, Nq, Nk, d, dtype, window = case
    banner(f"window fwd {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, dtype, seed=1300 + Nq + 3 * Nk + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, window)
    o_ref, lse_ref = attention_forward(to64(q), to64(k), to64(v), scale, False, window=window)
    check_forward(to64(o), to64(lse), o_ref, lse_ref, dtype, str(case))


BWD = [
    # B, H, Nq, Nk, d, window
    (1, 2, 300, 300, 64, (16, 0)),
    (1, 2, 333, 333, 128, (100, 50)),
    (1, 2, 257, 400, 64, (None, 7)),
    (1, 2, 400, 257, 128, (5, None)),
    (1, 1, 500, 200, 64, (31, 0)),          # leading rows and some keys see nothing
    (1, 1, 260, 260, 128, (0, 0)),
    (2, 1, 390, 390, 64, (200, 130)),
]


@pytest.mark.parametrize("det", [False, True], ids=lambda x: "det" if x else "atomic")
@pytest.mark.parametrize("case", BWD, ids=lambda c: "-".join(map(str, c)))
def test_window_backward_small_and_ragged(case, det):
    B, H, Nq, Nk, d, window = case
    banner(f"window bwd {case} {'det' if det else 'atomic'}")
    q, k, v, do = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=1500 + Nq + Nk + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    _, _, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, window, deterministic=det)
    rq, rk, rv, *_ = attention_backward(to64(q), to64(k), to64(v), to64(do), scale, False,
                                        window=window)
    check_grad(to64(dq), rq, f"dq {case}")
    check_grad(to64(dk), rk, f"dk {case}")
    check_grad(to64(dv), rv, f"dv {case}")


@pytest.mark.parametrize("d", [64, 128])
def test_window_limits_reproduce_causal_and_unmasked_bitwise(d):
    banner(f"window limits d={d}")
    q, k, v, do = wl.make_inputs(1, 2, 390, 450, d, "bf16", seed=1700 + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    # bitwise comparisons: the deterministic backward
    c = gpu_fwd_bwd(q, k, v, do, scale, causal=True, deterministic=True)
    n = gpu_fwd_bwd(q, k, v, do, scale, causal=False, deterministic=True)
    # the causal and unmasked kernels through the window entry points
    wc = gpu_fwd_bwd(q, k, v, do, scale, window=(None, 0), deterministic=True)
    wn = gpu_fwd_bwd(q, k, v, do, scale, window=(None, None), deterministic=True)
    # the window kernels with bounds that hide nothing beyond the causal
    # diagonal (left reach past every key), and nothing at all
    bc = gpu_fwd_bwd(q, k, v, do, scale, window=(10**6, 0), deterministic=True)
    bn = gpu_fwd_bwd(q, k, v, do, scale, window=(10**6, 10**6), deterministic=True)
    names = ("o", "lse", "dq", "dk", "dv")
    for ref, got, what in ((c, wc, "(None,0)"), (n, wn, "(None,None)"),
                           (c, bc, "(1e6,0)"), (n, bn, "(1e6,1e6)")):
        for nm, a, b in zip(names, ref, got):
            assert torch.equal(a, b), f"{what}: {nm} differs"


def test_keys_outside_the_window_do_not_change_rows_bitwise():
    banner("window: keys outside do not matter")
    Nq = Nk = 400
    wl_, wr_ = 40, 10
    q, k, v = wl.make_inputs(1, 2, Nq, Nk, 128, "bf16", seed=1800)
    o1, l1 = gpu_fwd(q, k, v, 0.1, (wl_, wr_))
    # rows 200..239 see keys 160..249 at most: perturb everything else
    k2, v2 = k.clone(), v.clone()
    for sl in (slice(0, 160), slice(250, Nk)):
        k2[:, :, sl] = (torch.randn_like(k2[:, :, sl].float()) * 8).to(torch.bfloat16)
        v2[:, :, sl] = 100.0
    o2, l2 = gpu_fwd(q, k2, v2, 0.1, (wl_, wr_))
    assert torch.equal(o1[:, :, 200:240], o2[:, :, 200:240])
    assert torch.equal(l1[:, :, 200:240], l2[:, :, 200:240])


def test_window_is_deterministic():
    banner("window determinism")
    q, k, v, do = wl.make_inputs(2, 2, 500, 500, 64, "bf16", seed=1900, with_do=True)
    a = gpu_fwd_bwd(q, k, v, do, 0.125, window=(100, 0))
    b = gpu_fwd_bwd(q, k, v, do, 0.125, window=(100, 0))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_sliding_window_workload_sampled_rows():
    w = wl.SLIDING_WINDOW
    banner(w.describe())
    q, k, v = wl.workload_inputs(w)[:3]
    o, lse = gpu_fwd(q, k, v, w.scale, w.window)
    rows = wl.sample_rows(w.Nq, 128, 7007)
    o_ref, lse_ref = attention_forward_rows(q.double().numpy(), k.double().numpy(),
                                            v.double().numpy(), w.scale, False, rows,
                                            window=w.window)
    check_forward(to64(o[:, :, rows]), to64(lse[:, :, rows]), o_ref, lse_ref, w.dtype, w.name)


def test_sliding_window_training_shape_sampled_heads():
    # the training-step shape (B=4 H=16 N=4096 d=64) under a 1024-key window
    B, H, N, d, window = 4, 16, 4096, 64, (1023, 0)
    banner(f"window fwd+bwd B={B} H={H} N={N} d={d} {window}")
    q, k, v, do = wl.make_inputs(B, H, N, N, d, "bf16", seed=2100, with_do=True)
    scale = 1.0 / np.sqrt(d)
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, window)
    for bh in (0, B * H - 1):
        b, h = divmod(bh, H)
        banner(f"oracle head {bh}")
        rq, rk, rv, ro, rl, _ = attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                                   to64(do[b, h]), scale, False, window=window)
        check_forward(to64(o[b, h]), to64(lse[b, h]), ro, rl, "bf16", f"head {bh}")
        check_grad(to64(dq[b, h]), rq, f"dq head {bh}")
        check_grad(to64(dk[b, h]), rk, f"dk head {bh}")
        check_grad(to64(dv[b, h]), rv, f"dv head {bh}")
