"""fa_bwd_noalloc (the backward with its workspace in a static device array)
against fa_bwd in its deterministic mode with a caller workspace, through the
C ABI.

Both run the same kernels on the same inputs, so the gradients must agree
bitwise; the first call is also checked against the fp64 oracle.  Calls run
back to back, each later one smaller than the one before, because the array
keeps the previous call's contents.
"""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_backward
from parity import check_grad, check_grad_f32, to64

pytestmark = pytest.mark.gpu

SCRATCH_ROWS = (8 << 20) // 8      # two fp32 row vectors fit in FA_NOALLOC_SCRATCH_BYTES


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def inputs(B, H, Nq, Nk, d, causal, seed, dtype="bf16"):
    q, k, v, do = wl.make_inputs_device(B, H, Nq, Nk, d, dtype, seed, "cuda", with_do=True)
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention_forward(q, k, v, scale=scale, causal=causal)
    return q, k, v, o, lse, do, scale


def noalloc(q, k, v, o, lse, do, scale, causal):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream().cuda_stream
    free0 = torch.cuda.mem_get_info()[0]
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           B, H, Nq, Nk, d, scale, int(causal),
                           fa.FA_F32 if q.dtype == torch.float32 else fa.FA_BF16, stream)
    torch.cuda.synchronize()
    assert st == 0, fa.fa_strerror(st)
    return (dq, dk, dv), free0 - torch.cuda.mem_get_info()[0]


# largest first: every later call runs on what the one before left behind
CALLS = [
    # B, H, Nq, Nk, d, causal, dtype
    (8, 32, 4096, 4096, 128, True, "bf16"),   # exactly the array's row limit
    (2, 3, 1000, 1000, 128, True, "bf16"),
    (1, 2, 300, 517, 64, False, "bf16"),
    (1, 2, 200, 150, 128, True, "fp32"),      # the fp32 kernels through the same array
]


def test_noalloc_matches_fa_bwd_on_calls_in_a_row():
    assert CALLS[0][0] * CALLS[0][1] * CALLS[0][2] == SCRATCH_ROWS
    grown = []
    for i, (B, H, Nq, Nk, d, causal, dtype) in enumerate(CALLS):
        banner(f"noalloc call {i}: {(B, H, Nq, Nk, d, causal, dtype)}")
        q, k, v, o, lse, do, scale = inputs(B, H, Nq, Nk, d, causal, seed=6100 + i, dtype=dtype)
        ref = fa.attention_backward(q, k, v, o, lse, do, scale=scale, causal=causal, deterministic=True)
        torch.cuda.synchronize()
        got, used = noalloc(q, k, v, o, lse, do, scale, causal)
        if i > 0:
            grown.append(used)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"call {i}: {name} differs from fa_bwd"
        if i >= len(CALLS) - 2:
            rq, rk, rv, *_ = attention_backward(to64(q), to64(k), to64(v), to64(do), scale, causal)
            chk = check_grad_f32 if dtype == "fp32" else check_grad
            chk(to64(got[0]), rq, f"dq call {i}")
            chk(to64(got[1]), rk, f"dk call {i}")
            chk(to64(got[2]), rv, f"dv call {i}")
    # after the first call has loaded the array, calls take no device memory
    assert grown == [0] * len(grown), grown

