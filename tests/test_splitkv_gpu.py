"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the fp64 oracle.

The split changes only how the key range is scheduled: each run of key tiles
produces a normalised partial O and LSE, and the combine step merges them by
rescaling, so the result must match the plain definition to the same bf16
tolerance as fa_fwd.  Cases cover decoding shapes (one or a few query rows,
long key ranges), several query tiles with causal runs that see no key,
rows with no visible key at all, one run (no split), automatic run counts,
ragged key tails and both head dimensions.
"""

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_forward
from parity import check_forward, to64

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


CASES = [
    # B, H, Nq, Nk, d, causal, n_splits (0 = automatic)
    (1, 2, 1, 1000, 128, True, 4),
    (2, 3, 1, 4097, 64, False, 0),
    (1, 4, 5, 3000, 128, True, 7),
    (1, 2, 300, 700, 64, True, 3),      # 3 query tiles; early tiles' later runs see no key
    (1, 2, 257, 100, 128, True, 2),     # 157 leading rows see no key
    (1, 1, 1, 1, 64, False, 1),
    (1, 1, 16, 64, 64, False, 1),       # one run: no split
    (2, 2, 1, 33000, 128, False, 0),    # long decode, ragged last tile
    (1, 3, 130, 2000, 64, False, 1000), # more runs asked for than tiles exist
    (1, 2, 1, 70, 128, True, 5),        # one query row: more runs than key tiles
    (3, 2, 1, 2500, 64, True, 0),       # one query row, d = 64, automatic runs
    (1, 1, 1, 200, 128, False, 1),      # one query row, one run
    (1, 2, 1, 0, 128, True, 0),         # one query row, no keys: O = 0, LSE = -inf
    (2, 1, 1, 0, 64, False, 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_splitkv_matches_oracle(case):
    B, H, Nq, Nk, d, causal, ns = case
    banner(f"splitkv {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=3100 + Nq + Nk + d + ns)
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.attention_forward_splitkv(qd, kd, vd, scale=scale, causal=causal, n_splits=ns)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(to64(q), to64(k), to64(v), scale, causal)
    check_forward(to64(o), to64(lse), o_ref, lse_ref, "bf16", str(case))


def test_splitkv_agrees_with_unsplit_and_is_deterministic():
    banner("splitkv vs fa_fwd")
    q, k, v = wl.make_inputs(2, 4, 64, 5000, 128, "bf16", seed=3333)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o1, l1 = fa.attention_forward_splitkv(qd, kd, vd, causal=True, n_splits=9)
    o2, l2 = fa.attention_forward_splitkv(qd, kd, vd, causal=True, n_splits=9)
    o0, l0 = fa.attention_forward(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert (o1.float() - o0.float()).abs().max().item() <= 2e-2
    assert (l1 - l0).abs().max().item() <= 1e-3


def test_decode_workload_sampled_heads():
    w = wl.DECODE
    banner(w.describe())
    q, k, v = wl.workload_inputs(w)[:3]
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.attention_forward_splitkv(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(6006)
    for bh in [0, w.B * w.H - 1] + torch.randperm(w.B * w.H, generator=g)[:4].tolist():
        b, h = divmod(bh, w.H)
        o_ref, lse_ref = attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), w.scale, w.causal)
        check_forward(to64(o[b, h]), to64(lse[b, h]), o_ref, lse_ref, "bf16", f"{w.name} head {bh}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_large_logit_jump_and_agreement(d):
    """Single query row: keys whose logits exceed the earlier ones by ~200
    log2 units (each run's scaling base and the combine's rescale must
    follow them), checked against the oracle; plus run-to-run determinism
    and agreement with fa_fwd."""
    banner(f"decode jump d={d}")
    B, H, Nk = 1, 3, 3000
    q, k, v = wl.make_inputs(B, H, 1, Nk, d, "bf16", seed=3500 + d)
    A = 40.0 if d == 128 else 34.0
    for h, j in ((0, 2999), (1, 1500), (2, 7)):
        q[0, h, 0, :] = 0
        q[0, h, 0, 0] = A
        k[0, h, j, 0] = A
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o1, l1 = fa.attention_forward_splitkv(qd, kd, vd, scale=scale, causal=True, n_splits=6)
    o2, l2 = fa.attention_forward_splitkv(qd, kd, vd, scale=scale, causal=True, n_splits=6)
    o0, l0 = fa.attention_forward(qd, kd, vd, scale=scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = attention_forward(to64(q), to64(k), to64(v), scale, True)
    check_forward(to64(o1), to64(l1), o_ref, lse_ref, "bf16", f"decode jump d={d}")
    assert (o1.float() - o0.float()).abs().max().item() <= 2e-2
    assert (l1 - l0).abs().max().item() <= 1e-3
