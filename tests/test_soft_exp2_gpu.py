"""GPU parity of fa_fwd_soft_exp2 (the opt-in forward in which one softmax
exponential in 2, 4 or 8 is a polynomial on the FMA pipe) against the fp64
oracle, at the bf16 forward's tolerance: small and ragged shapes of both head
dims, causal and unmasked, Nq != Nk both ways (rows that see no key), and the
forward workloads on sampled heads or rows.  The same inputs through fa_fwd
must agree to within the polynomial's error, not bitwise."""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_forward, attention_forward_rows
from parity import check_forward, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_fwd(q, k, v, scale, causal, period):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.attention_forward(qd, kd, vd, scale=scale, causal=causal, soft_exp2=period)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # B, H, Nq, Nk, d, causal
    (1, 1, 1, 1, 64, False),
    (1, 2, 200, 200, 64, True),
    (2, 1, 333, 333, 64, False),
    (1, 2, 130, 70, 128, True),     # leading rows see no key
    (1, 1, 70, 250, 128, True),
    (1, 2, 257, 257, 128, False),
]


@pytest.mark.parametrize("period", [2, 4, 8])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_soft_exp2_small_and_ragged(case, period):
    B, H, Nq, Nk, d, causal = case
    banner(f"soft exp2 period {period} {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=3100 + Nq + Nk + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, causal, period)
    o_ref, lse_ref = attention_forward(to64(q), to64(k), to64(v), scale, causal)
    check_forward(to64(o), to64(lse), o_ref, lse_ref, "bf16", f"{case} period {period}")
    # against the hardware exponential: P differs by at most 7.5e-5 relative
    o_hw, lse_hw = gpu_fwd(q, k, v, scale, causal, 0)
    live = torch.isfinite(lse_hw)
    assert torch.equal(live, torch.isfinite(lse))
    assert (lse[live] - lse_hw[live]).abs().max().item() <= 1e-4 if live.any() else True
    assert (o.float() - o_hw.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("w,period,n", [(wl.GPT2_SMALL, 4, 8), (wl.TRAIN_STEP, 2, 32), (wl.LLAMA_CAUSAL, 8, 32)],
                         ids=["gpt2_small-4", "train_step-2", "llama_causal-8"])
def test_soft_exp2_workloads_sampled(w, period, n):
    banner(f"{w.describe()} soft exp2 period {period}")
    q, k, v = wl.workload_inputs(w)[:3]
    o, lse = gpu_fwd(q, k, v, w.scale, w.causal, period)
    g = torch.Generator().manual_seed(6000 + period)
    heads = [0, w.B * w.H - 1] + torch.randperm(w.B * w.H, generator=g)[:3].tolist()
    for bh in heads:
        b, h = divmod(bh, w.H)
        rows = wl.sample_rows(w.Nq, n, 6100 + bh)
        o_ref, lse_ref = attention_forward_rows(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), w.scale,
                                                w.causal, rows)
        check_forward(to64(o[b, h, rows]), to64(lse[b, h, rows]), o_ref, lse_ref, "bf16",
                      f"{w.name} head {bh} period {period}")


def test_soft_exp2_rejects_fp32_and_windows():
    q, k, v = (t.cuda() for t in wl.make_inputs(1, 1, 64, 64, 64, "fp32", seed=1))
    with pytest.raises(fa.FAError):
        fa.attention_forward(q, k, v, soft_exp2=4)
    qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
    with pytest.raises(ValueError):
        fa.attention_forward(qb, kb, vb, window=(8, 0), soft_exp2=4)
    with pytest.raises(fa.FAError):
        fa.attention_forward(qb, kb, vb, soft_exp2=3)
