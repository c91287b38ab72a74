"""GPU parity of the variable-length entry points (fa_fwd_varlen,
fa_bwd_varlen) against the fp64 oracle (MI355X only).

Sequences of different lengths are packed head-major, q [H, total_q, d] and
k, v [H, total_k, d], with int32 offsets cu_seqlens [B+1] on the device; each
sequence attends within itself under the causal, window or no mask taken over
its own lengths.  The cases mix lengths below, at and above the 128-row and
64-key tiles, empty sequences on either side, Nq != Nk per sequence, padding
rows past the last sequence (which must stay untouched), both head dims, and
the packed workload at its full size (sampled sequences and rows).  Equal
lengths must reproduce the fixed-length calls bitwise.
"""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_forward_rows, varlen_backward, varlen_forward
from parity import check_forward, check_grad, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def run_fwd(q, k, v, cu_q, cu_k, lens_q, lens_k, scale, causal=False, window=None,
            sentinel=None):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out = torch.full_like(qd, sentinel) if sentinel is not None else None
    lse = (torch.full((q.shape[0], q.shape[1]), sentinel, dtype=torch.float32, device="cuda")
           if sentinel is not None else None)
    o, l = fa.attention_forward_varlen(qd, kd, vd, cu_q.cuda(), cu_k.cuda(), max(lens_q, default=0),
                                       max(lens_k, default=0), scale=scale, causal=causal,
                                       window=window, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


def run_fwd_bwd(q, k, v, do, cu_q, cu_k, lens_q, lens_k, scale, causal=False, window=None,
                deterministic=False):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    cq, ck = cu_q.cuda(), cu_k.cuda()
    mq, mk = max(lens_q, default=0), max(lens_k, default=0)
    o, lse = fa.attention_forward_varlen(qd, kd, vd, cq, ck, mq, mk, scale=scale, causal=causal,
                                         window=window)
    dq, dk, dv = fa.attention_backward_varlen(qd, kd, vd, o, lse, dod, cq, ck, mq, mk, scale=scale,
                                              causal=causal, window=window,
                                              deterministic=deterministic)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def inside(cu):
    """Row indices covered by the sequences."""
    return np.arange(int(cu[-1]))


FWD = [
    # query lengths, key lengths, d, causal, window
    ([1, 127, 128, 129, 300], None, 64, True, None),
    ([200, 17, 450], None, 128, False, None),
    ([100, 260, 64], [300, 60, 64], 128, True, None),    # Nq != Nk both ways: empty rows
    ([0, 190, 0, 70], [40, 190, 0, 0], 64, True, None),  # empty sequences on either side
    ([333, 90, 512], None, 128, False, (40, 7)),
    ([257, 31], [129, 400], 64, False, (None, 20)),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "-".join(map(str, c)).replace(" ", ""))
def test_varlen_forward_small_and_ragged(case):
    lens_q, lens_k, d, causal, window = case
    lens_k = lens_q if lens_k is None else lens_k
    banner(f"varlen fwd {case}")
    q, k, v, cu_q, cu_k = wl.make_varlen_inputs(lens_q, lens_k, 2, d, "bf16",
                                                seed=3000 + sum(lens_q) + d, pad_q=5, pad_k=3)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_fwd(q, k, v, cu_q, cu_k, lens_q, lens_k, scale, causal, window, sentinel=7.0)
    O, L = varlen_forward(to64(q), to64(k), to64(v), cu_q.numpy(), cu_k.numpy(), scale, causal,
                          window)
    rows = inside(cu_q)
    check_forward(to64(o)[:, rows], to64(lse)[:, rows], O[:, rows], L[:, rows], "bf16", str(case))
    # padding rows past the last sequence are not written
    assert torch.all(o[:, int(cu_q[-1]):] == 7.0) and torch.all(lse[:, int(cu_q[-1]):] == 7.0)


BWD = [
    ([1, 127, 129, 300], None, 64, True, None),
    ([200, 17, 450], None, 128, False, None),
    ([100, 260, 64], [300, 60, 64], 128, True, None),
    ([0, 190, 70], [40, 190, 0], 64, True, None),
    ([333, 90], None, 64, False, (40, 7)),
]


@pytest.mark.parametrize("det", [False, True], ids=lambda x: "det" if x else "atomic")
@pytest.mark.parametrize("case", BWD, ids=lambda c: "-".join(map(str, c)).replace(" ", ""))
def test_varlen_backward_small_and_ragged(case, det):
    lens_q, lens_k, d, causal, window = case
    lens_k = lens_q if lens_k is None else lens_k
    banner(f"varlen bwd {case} {'det' if det else 'atomic'}")
    q, k, v, do, cu_q, cu_k = wl.make_varlen_inputs(lens_q, lens_k, 2, d, "bf16",
                                                    seed=3300 + sum(lens_k) + d, with_do=True)
    scale = 1.0 / np.sqrt(d)
    _, _, dq, dk, dv = run_fwd_bwd(q, k, v, do, cu_q, cu_k, lens_q, lens_k, scale, causal, window,
                                   deterministic=det)
    rq, rk, rv = varlen_backward(to64(q), to64(k), to64(v), to64(do), cu_q.numpy(), cu_k.numpy(),
                                 scale, causal, window)
    check_grad(to64(dq), rq, f"dq {case}")
    check_grad(to64(dk), rk, f"dk {case}")
    check_grad(to64(dv), rv, f"dv {case}")


@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_varlen_equal_lengths_reproduce_fixed_length_bitwise(d, causal):
    B, H, N = 3, 2, 300
    banner(f"varlen = fixed length, d={d} causal={causal}")
    q, k, v, do = wl.make_inputs(B, H, N, N, d, "bf16", seed=3600 + d, with_do=True)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.attention_forward(qd, kd, vd, causal=causal)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, deterministic=True)
    pack = lambda x: x.transpose(0, 1).reshape(H, B * N, d).contiguous()   # [B,H,N,d] -> [H,B*N,d]
    cu = torch.arange(B + 1, dtype=torch.int32) * N
    got = run_fwd_bwd(pack(q), pack(k), pack(v), pack(do), cu, cu, [N] * B, [N] * B,
                      1.0 / np.sqrt(d), causal, deterministic=True)
    ref = (pack(o), lse.transpose(0, 1).reshape(H, B * N), pack(dq), pack(dk), pack(dv))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), name


def test_varlen_is_deterministic():
    banner("varlen determinism")
    lens = [300, 77, 512, 129]
    q, k, v, do, cu, _ = wl.make_varlen_inputs(lens, lens, 2, 64, "bf16", seed=3700, with_do=True)
    a = run_fwd_bwd(q, k, v, do, cu, cu, lens, lens, 0.125, True, deterministic=True)
    b = run_fwd_bwd(q, k, v, do, cu, cu, lens, lens, 0.125, True, deterministic=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_varlen_workload_sampled_sequences_and_rows():
    w = wl.VARLEN_CAUSAL
    banner(w.describe())
    q, k, v, cu_q, cu_k = wl.varlen_workload_inputs(w)
    L = w.lengths()
    o, lse = run_fwd(q, k, v, cu_q, cu_k, L, L, w.scale, w.causal)
    # the longest, the shortest and two seeded sequences; 48 rows of each
    g = torch.Generator().manual_seed(8008)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L))} |
                  set(torch.randperm(len(L), generator=g)[:2].tolist()))
    for b in seqs:
        s, e = int(cu_q[b]), int(cu_q[b + 1])
        rows = wl.sample_rows(e - s, 48, 9000 + b)
        banner(f"oracle sequence {b} ({e - s} tokens)")
        O, Lr = attention_forward_rows(q[:, s:e].double().numpy(), k[:, s:e].double().numpy(),
                                       v[:, s:e].double().numpy(), w.scale, w.causal, rows)
        idx = [s + r for r in rows]
        check_forward(to64(o[:, idx]), to64(lse[:, idx]), O, Lr, w.dtype, f"sequence {b}")
