"""GPU parity on tensors past 2^31 elements (MI355X only).

B = 40, H = 128, N = 4096, d = 128, bf16, causal: each of Q, K, V, O, dO,
dQ, dK and dV holds 40 * 128 * 4096 * 128 = 2.68e9 elements (5.4 GB), so
element offsets pass 2^31 at head 4096 and byte offsets pass 2^31 and 2^32
at heads 2048 and 4096.  Forward and backward run over the whole batch; the
fp64 oracle checks whole heads on both sides of each boundary, the first
head and the last.  About 43 GB of device memory.
"""

import math

import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_backward, attention_forward
from parity import check_forward, check_grad, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("det", [False, True], ids=lambda x: "det" if x else "atomic")
def test_forward_and_backward_past_2_31_elements(det):
    B, H, N, d = 40, 128, 4096, 128
    per_head = N * d
    assert B * H * per_head > 2 ** 31
    scale = 1.0 / math.sqrt(d)
    banner(f"large fwd+bwd B{B} H{H} N{N} d{d} causal ({B * H * per_head} elements per tensor)")
    q, k, v, do = wl.make_inputs_device(B, H, N, N, d, "bf16", seed=7007, device="cuda", with_do=True)
    o, lse = fa.attention_forward(q, k, v, scale=scale, causal=True)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, scale=scale, causal=True,
                                       deterministic=det)
    torch.cuda.synchronize()
    first_past = 2 ** 31 // per_head            # first head starting at element 2^31 (byte 2^32)
    heads = [0, first_past // 2 - 1, first_past // 2, first_past - 1, first_past, B * H - 1]
    for bh in heads:
        b, h = divmod(bh, H)
        banner(f"large: oracle head {bh} (elements from {bh * per_head})")
        qh, kh, vh, doh = (to64(t[b, h]) for t in (q, k, v, do))
        o_ref, lse_ref = attention_forward(qh, kh, vh, scale, True)
        check_forward(to64(o[b, h]), to64(lse[b, h]), o_ref, lse_ref, "bf16", f"head {bh}")
        rq, rk, rv, *_ = attention_backward(qh, kh, vh, doh, scale, True)
        check_grad(to64(dq[b, h]), rq, f"dq head {bh}")
        check_grad(to64(dk[b, h]), rk, f"dk head {bh}")
        check_grad(to64(dv[b, h]), rv, f"dv head {bh}")
