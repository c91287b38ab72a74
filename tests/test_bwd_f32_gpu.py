"""GPU parity of fa_bwd and fa_bwd_window on fp32 inputs (true fp32 products
on the fp32 MFMA) against the fp64 oracle: the single-head fp32 workload,
small and ragged shapes of both head dims under every mask, rows and keys
that see nothing, and bitwise repeatability (fp32 has one algorithm, so both
values of ``deterministic`` give the same bits).

The GPU backward consumes the GPU forward's O and LSE, as a training step
does; the oracle computes everything from the same fp32 inputs in fp64.
"""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_backward
from parity import check_grad_f32, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_fwd_bwd(q, k, v, do, scale, causal=False, window=None, deterministic=True):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention_forward(qd, kd, vd, scale=scale, causal=causal, window=window)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal,
                                       window=window, deterministic=deterministic)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_all(got, q, k, v, do, scale, causal, window, what):
    rq, rk, rv, *_ = attention_backward(to64(q), to64(k), to64(v), to64(do), scale, causal,
                                        window=window)
    for g, r, n in zip(got, (rq, rk, rv), ("dq", "dk", "dv")):
        err = check_grad_f32(to64(g), r, f"{n} {what}")
        print(f"  {n}: max-abs err {err:.2e}, ||ref||_inf {np.max(np.abs(r)) if r.size else 0:.2e}", flush=True)


def test_single_head_fp32_workload_backward():
    w = wl.SINGLE_HEAD
    banner(w.describe() + " backward")
    q, k, v = wl.workload_inputs(w)
    do = wl.make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, "fp32", seed=w.seed + 1, with_do=True)[3]
    got = gpu_fwd_bwd(q, k, v, do, w.scale, w.causal)
    check_all(got, q, k, v, do, w.scale, w.causal, None, w.name)


SMALL = [
    # B, H, Nq, Nk, d, causal, window
    (1, 1, 1, 1, 64, False, None),
    (1, 2, 64, 64, 64, True, None),
    (2, 1, 100, 100, 64, False, None),
    (2, 1, 100, 100, 128, True, None),
    (1, 2, 130, 70, 128, True, None),       # leading query rows see no key
    (1, 1, 70, 130, 64, True, None),
    (1, 2, 200, 333, 128, False, None),
    (1, 1, 257, 257, 64, True, None),
    (1, 1, 1000, 1000, 128, True, None),    # many tiles each way
    (1, 4, 500, 500, 64, True, None),       # 8 tiles per head, 32 workgroups: XCD runs of mirrored pairs
    (1, 2, 300, 300, 64, False, (16, 0)),
    (1, 2, 333, 333, 128, False, (100, 50)),
    (1, 1, 500, 200, 64, False, (31, 0)),   # leading rows and some keys see nothing
    (1, 2, 257, 400, 128, False, (None, 7)),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_fp32_backward_small_and_ragged(case):
    B, H, Nq, Nk, d, causal, window = case
    banner(f"fp32 bwd {case}")
    q, k, v, do = wl.make_inputs(B, H, Nq, Nk, d, "fp32", seed=2500 + Nq + Nk + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    got = gpu_fwd_bwd(q, k, v, do, scale, causal, window)
    check_all(got, q, k, v, do, scale, causal, window, str(case))


def test_fp32_backward_empty_rows_and_keys_are_zero():
    # causal with Nq > Nk: the first Nq - Nk query rows see no key (dQ = 0);
    # a window (31, 0) over Nq < Nk: keys past the last query's reach get dK = dV = 0
    banner("fp32 bwd empty rows / keys")
    q, k, v, do = wl.make_inputs(1, 2, 190, 70, 64, "fp32", seed=2601, with_do=True)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, 0.125, causal=True)
    assert torch.count_nonzero(dq[:, :, : 190 - 70].cpu()) == 0
    q, k, v, do = wl.make_inputs(1, 2, 100, 300, 128, "fp32", seed=2602, with_do=True)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, 0.09, window=(31, 0))
    # query i sees keys i + 200 - 31 .. i + 200, so keys below 169 see nothing
    assert torch.count_nonzero(dk[:, :, :169].cpu()) == 0
    assert torch.count_nonzero(dv[:, :, :169].cpu()) == 0


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_backward_bitwise_repeatable_in_both_modes(d):
    banner(f"fp32 bwd repeatable d={d}")
    q, k, v, do = wl.make_inputs(1, 3, 333, 333, d, "fp32", seed=2700 + d, with_do=True)
    a = gpu_fwd_bwd(q, k, v, do, 0.1, causal=True, deterministic=True)
    b = gpu_fwd_bwd(q, k, v, do, 0.1, causal=True, deterministic=True)
    c = gpu_fwd_bwd(q, k, v, do, 0.1, causal=True, deterministic=False)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)
