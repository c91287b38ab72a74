"""GPU parity of fa_bwd (recomputation backward) against the fp64 oracle, in
both modes: the deterministic one (dQ from its own kernel, bitwise
repeatable) and the atomic one (one key-side kernel, dQ summed with fp32
atomics).

The GPU backward consumes the GPU forward's O and LSE, as a training step
does; the oracle computes everything from the same bf16 inputs in fp64.
"""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_backward
from parity import check_grad, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_fwd_bwd(q, k, v, do, scale, causal, deterministic):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention_forward(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal,
                                       deterministic=deterministic)
    torch.cuda.synchronize()
    return dq, dk, dv


MODES = [False, True]
mode_id = lambda det: "det" if det else "atomic"


SMALL = [
    # B, H, Nq, Nk, d, causal
    (1, 1, 1, 1, 64, False),
    (1, 2, 64, 64, 64, True),
    (2, 1, 100, 100, 64, False),
    (2, 1, 100, 100, 64, True),
    (1, 2, 130, 70, 128, True),      # leading query rows see no key
    (1, 1, 70, 130, 64, True),
    (1, 2, 200, 333, 128, False),
    (1, 1, 257, 257, 128, True),
]


@pytest.mark.parametrize("det", MODES, ids=mode_id)
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_backward_small_and_ragged(case, det):
    B, H, Nq, Nk, d, causal = case
    banner(f"bwd small {case} {mode_id(det)}")
    q, k, v, do = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=500 + Nq + Nk + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, causal, det)
    rq, rk, rv, *_ = attention_backward(to64(q), to64(k), to64(v), to64(do), scale, causal)
    check_grad(to64(dq), rq, f"dq {case}")
    check_grad(to64(dk), rk, f"dk {case}")
    check_grad(to64(dv), rv, f"dv {case}")


# Unpaired causal grids whose batch*head count is not a multiple of 16: both
# kernels' workgroup maps give each XCD an equal run of mirrored tile pairs
# (heavy tiles first, light ones in reverse).  Every head is checked.
XCD_RUNS = [
    # B, H, Nq, Nk, d
    (1, 4, 2000, 2000, 128),      # 16 key and query tiles, ragged tail
    (1, 6, 2048, 2048, 64),
    (1, 4, 1500, 2048, 128),      # Nk > Nq: 12 query tiles, 16 key tiles
]


@pytest.mark.parametrize("det", MODES, ids=mode_id)
@pytest.mark.parametrize("case", XCD_RUNS, ids=lambda c: "-".join(map(str, c)))
def test_backward_xcd_pair_runs(case, det):
    B, H, Nq, Nk, d = case
    for n in ((Nq + 127) // 128, (Nk + 127) // 128):
        assert n % 2 == 0 and (B * H * n) % 16 == 0 and (B * H * n // 8) % (2 * n) != 0   # the map's new branch
    banner(f"bwd xcd pair runs {case} {mode_id(det)}")
    q, k, v, do = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=590 + Nq + Nk + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, True, det)
    rq, rk, rv, *_ = attention_backward(to64(q), to64(k), to64(v), to64(do), scale, True)
    check_grad(to64(dq), rq, f"dq {case}")
    check_grad(to64(dk), rk, f"dk {case}")
    check_grad(to64(dv), rv, f"dv {case}")


# Large causal grids take the paired path in both backward kernels (a
# workgroup runs key tile j then n-1-j, query tile n-1-j then j): odd tile
# counts, ragged tails and Nq != Nk.
PAIRED = [
    # B, H, Nq, Nk, d
    (2, 70, 1900, 1900, 64),      # 15 key tiles and 15 query tiles of 128
    (1, 256, 1000, 1300, 64),     # Nk > Nq
    (1, 256, 1300, 1000, 128),    # Nq > Nk: leading rows see no key
]


@pytest.mark.parametrize("det", MODES, ids=mode_id)
@pytest.mark.parametrize("case", PAIRED, ids=lambda c: "-".join(map(str, c)))
def test_backward_paired_tiles_sampled_heads(case, det):
    B, H, Nq, Nk, d = case
    assert B * H * ((min(Nq, Nk) + 127) // 128) >= 2048   # both kernels pair
    banner(f"bwd paired {case} {mode_id(det)}")
    q, k, v, do = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=700 + Nq + Nk + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, scale, True, det)
    for bh in (0, B * H // 2, B * H - 1):
        b, h = divmod(bh, H)
        rq, rk, rv, *_ = attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                            to64(do[b, h]), scale, True)
        check_grad(to64(dq[b, h]), rq, f"dq {case} head {bh}")
        check_grad(to64(dk[b, h]), rk, f"dk {case} head {bh}")
        check_grad(to64(dv[b, h]), rv, f"dv {case} head {bh}")


def sampled_heads(w, seed, n=16):
    """The first and the last (batch, head) and n-2 others drawn with ``seed``."""
    g = torch.Generator().manual_seed(seed)
    others = [bh for bh in torch.randperm(w.B * w.H, generator=g).tolist() if bh not in (0, w.B * w.H - 1)]
    return [0, w.B * w.H - 1] + others[: n - 2]


@pytest.mark.parametrize("det", MODES, ids=mode_id)
def test_train_step_workload_sampled_heads(det):
    w = wl.TRAIN_STEP
    banner(w.describe() + " " + mode_id(det))
    q, k, v, do = wl.workload_inputs(w)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, w.scale, w.causal, det)
    heads = sampled_heads(w, 5050)
    for bh in heads:
        b, h = divmod(bh, w.H)
        banner(f"{w.name} oracle head {bh}")
        rq, rk, rv, *_ = attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                            to64(do[b, h]), w.scale, w.causal)
        check_grad(to64(dq[b, h]), rq, f"dq head {bh}")
        check_grad(to64(dk[b, h]), rk, f"dk head {bh}")
        check_grad(to64(dv[b, h]), rv, f"dv head {bh}")


@pytest.mark.parametrize("det", MODES, ids=mode_id)
def test_llama_causal_backward_sampled_heads(det):
    """The d = 128 backward at B=4 H=32 N=4096 causal, on the inputs bench.py
    times with --train-workload llama_causal_bf16 (the workload's seed, dO
    drawn after Q, K, V)."""
    w = wl.LLAMA_CAUSAL
    banner(w.describe() + " (backward) " + mode_id(det))
    q, k, v, do = wl.make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, with_do=True)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, w.scale, w.causal, det)
    heads = sampled_heads(w, 5151)
    for bh in heads:
        b, h = divmod(bh, w.H)
        banner(f"{w.name} backward oracle head {bh}")
        rq, rk, rv, *_ = attention_backward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                            to64(do[b, h]), w.scale, w.causal)
        check_grad(to64(dq[b, h]), rq, f"dq head {bh}")
        check_grad(to64(dk[b, h]), rk, f"dk head {bh}")
        check_grad(to64(dv[b, h]), rv, f"dv head {bh}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("det", MODES, ids=mode_id)
def test_backward_invariants_and_repeatability(det, d):
    banner(f"bwd invariants d={d} {mode_id(det)}")
    q, k, v, do = wl.make_inputs(1, 2, 256, 256, d, "bf16", seed=61, with_do=True)
    dq1, dk1, dv1 = gpu_fwd_bwd(q, k, v, do, 0.125, True, det)
    runs = [gpu_fwd_bwd(q, k, v, do, 0.125, True, det) for _ in range(3)]
    for dq2, dk2, dv2 in runs:
        # dK and dV are accumulated by one workgroup in both modes; dQ too in
        # the deterministic mode, while the atomic mode's fp32 adds may land
        # in any order (same tolerance, not bitwise)
        assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
        if det:
            assert torch.equal(dq1, dq2)
        else:
            err = (dq1.float() - dq2.float()).abs().max().item()
            assert err <= 2e-2 * max(1.0, dq1.float().abs().max().item())
    # rows of dS sum to zero, so the key gradients sum to ~0; sum_j dV_j = sum_i dO_i
    ksum = dk1.float().sum(dim=2).abs().max().item()
    kscale = dk1.float().abs().sum(dim=2).max().item()
    assert ksum <= 2e-2 * max(1.0, kscale)
    vs = dv1.float().sum(dim=2).cpu()
    ds = do.float().sum(dim=2)
    assert torch.max(torch.abs(vs - ds)).item() <= 2e-2 * max(1.0, ds.abs().max().item())


def test_binding_checks_devices_and_sizes_workspace_in_bytes():
    banner("binding: device checks, workspace in bytes")
    q, k, v, do = wl.make_inputs(1, 2, 100, 100, 64, "bf16", seed=71, with_do=True)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    with pytest.raises(ValueError):
        fa.attention_forward(qd, k, vd, causal=True)          # k left on the host
    o, lse = fa.attention_forward(qd, kd, vd, causal=True)
    need = fa.fa_bwd_workspace_bytes(1, 2, 100, 100, 64, fa.FA_BF16, 1)
    with pytest.raises(ValueError):
        fa.attention_backward(qd, kd, vd, o, lse, dod, causal=True,
                              workspace=torch.empty(need, dtype=torch.uint8), deterministic=True)
    # a float32 workspace: at least `need` bytes in fewer than `need` elements
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=True, workspace=ws,
                                       deterministic=True)
    dq0, dk0, dv0 = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=True, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0) and torch.equal(dk, dk0) and torch.equal(dv, dv0)
    # the atomic mode refuses the smaller, deterministic-sized workspace
    with pytest.raises(fa.FAError):
        fa.attention_backward(qd, kd, vd, o, lse, dod, causal=True, workspace=ws,
                              deterministic=False)
