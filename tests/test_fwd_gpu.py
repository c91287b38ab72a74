"""GPU parity of fa_fwd against the fp64 oracle (MI355X only).

Every case calls the HIP path through the C ABI (exact_attention_20_amd ->
libfa.so) and compares with the oracle on the same seeded inputs.  Full-size
workloads run on the GPU at their real shape and launch configuration; the
oracle then checks sampled heads or rows it can compute one by one.
"""

import json
import os

import numpy as np
import pytest
import torch

import exact_attention_20_amd as fa
import workloads as wl
from oracle import attention_forward, attention_forward_rows
from parity import check_forward, to64

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_fwd(q, k, v, scale, causal):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.attention_forward(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------ small / ragged
SMALL = [
    # B, H, Nq, Nk, d, dtype, causal
    (1, 1, 1, 1, 64, "bf16", False),
    (1, 1, 1, 1, 128, "fp32", True),
    (2, 3, 17, 17, 64, "bf16", True),
    (1, 2, 100, 257, 128, "bf16", False),
    (1, 2, 100, 257, 128, "bf16", True),
    (1, 2, 257, 100, 128, "bf16", True),      # 157 leading rows see no key
    (1, 1, 300, 300, 64, "bf16", True),
    (2, 2, 128, 128, 128, "bf16", True),
    (1, 1, 129, 64, 64, "bf16", False),
    (1, 1, 64, 129, 64, "bf16", True),
    (1, 3, 383, 383, 64, "bf16", False),
    (1, 2, 77, 130, 64, "fp32", False),
    (1, 2, 77, 130, 64, "fp32", True),
    (1, 1, 200, 200, 128, "fp32", True),
    (1, 1, 200, 71, 128, "fp32", True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_and_ragged(case):
    B, H, Nq, Nk, d, dtype, causal = case
    banner(f"fwd small {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, dtype, seed=77 + Nq + 3 * Nk + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = attention_forward(to64(q), to64(k), to64(v), scale, causal)
    check_forward(to64(o), to64(lse), o_ref, lse_ref, dtype, str(case))


def test_single_head_fp32_workload():
    w = wl.SINGLE_HEAD
    banner(w.describe())
    q, k, v = wl.workload_inputs(w)
    o, lse = gpu_fwd(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = attention_forward(to64(q), to64(k), to64(v), w.scale, w.causal)
    check_forward(to64(o), to64(lse), o_ref, lse_ref, "fp32", w.name)


def _sampled_heads_check(w, n_heads, seed):
    q, k, v = wl.workload_inputs(w)[:3]
    o, lse = gpu_fwd(q, k, v, w.scale, w.causal)
    g = torch.Generator().manual_seed(seed)
    heads = torch.randperm(w.B * w.H, generator=g)[:n_heads].tolist()
    for bh in heads:
        b, h = divmod(bh, w.H)
        o_ref, lse_ref = attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), w.scale, w.causal)
        check_forward(to64(o[b, h]), to64(lse[b, h]), o_ref, lse_ref, w.dtype, f"{w.name} head {bh}")


def _sampled_rows_check(w, n_rows, seed):
    """Every (batch, head) with its own seeded draw of n_rows query rows (seed
    + b*H + h; rows 0 and Nq-1 always in)."""
    q, k, v = wl.workload_inputs(w)[:3]
    o, lse = gpu_fwd(q, k, v, w.scale, w.causal)
    for b in range(w.B):
        for h in range(w.H):
            rows = wl.sample_rows(w.Nq, n_rows, seed + b * w.H + h)
            o_ref, lse_ref = attention_forward_rows(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]),
                                                    w.scale, w.causal, rows)
            check_forward(to64(o[b, h, rows]), to64(lse[b, h, rows]), o_ref, lse_ref, w.dtype,
                          f"{w.name} head {(b, h)}")


def test_gpt2_small_workload_sampled_heads():
    banner(wl.GPT2_SMALL.describe())
    _sampled_heads_check(wl.GPT2_SMALL, 8, 2002)


def test_llama_causal_workload_sampled_rows():
    banner(wl.LLAMA_CAUSAL.describe())
    _sampled_rows_check(wl.LLAMA_CAUSAL, 64, 3000)


def test_long_context_workload_256_rows_per_head():
    # head h: 256 rows drawn with seed 4000 + h, rows 0 and N-1 forced
    banner(wl.LONG_CONTEXT.describe())
    _sampled_rows_check(wl.LONG_CONTEXT, 256, 4000)


def test_train_step_forward_sampled_rows():
    banner(wl.TRAIN_STEP.describe() + " (forward)")
    _sampled_rows_check(wl.TRAIN_STEP, 96, 5000)


# ------------------------------------------ paired query tiles (large causal grids)
# With causal masking, d = 64, at most 64 query tiles per head and at least
# 2048 (batch*head, 128-row query tile) units, a bf16 workgroup runs query tile
# n-1-j and then its mirror j, prefetching the second one's Q and first key
# tile while the first finishes.  These shapes take that path with an even and
# an odd tile count, ragged tails and Nq != Nk; the last one is the same kind
# of grid at d = 128, which does not pair.
PAIRED = [
    # B, H, Nq, Nk, d
    (2, 64, 2000, 2000, 64),      # 16 query tiles, ragged 80-row tail
    (2, 70, 1900, 1900, 64),      # 15 query tiles: the middle one runs alone
    (1, 256, 1000, 1300, 64),     # Nk > Nq (bottom-right causal alignment)
    (1, 256, 1100, 900, 64),      # Nq > Nk: leading rows see no key
    (2, 64, 2000, 2000, 128),     # unpaired at d = 128
]


@pytest.mark.parametrize("case", PAIRED, ids=lambda c: "-".join(map(str, c)))
def test_paired_query_tiles_sampled_heads(case):
    B, H, Nq, Nk, d = case
    assert B * H * ((Nq + 127) // 128) >= 2048   # the paired path
    banner(f"fwd paired {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=900 + Nq + Nk + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, True)
    g = torch.Generator().manual_seed(Nq * 7 + Nk)
    heads = [0, B * H - 1] + torch.randperm(B * H, generator=g)[:3].tolist()
    for bh in heads:
        b, h = divmod(bh, H)
        o_ref, lse_ref = attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), scale, True)
        check_forward(to64(o[b, h]), to64(lse[b, h]), o_ref, lse_ref, "bf16", f"{case} head {bh}")


# ------------------------- XCD runs of mirrored pairs (unpaired causal grids)
# When the batch*head count is not a multiple of 16, the workgroup map gives
# each XCD an equal run of mirrored query-tile pairs (its heavy tiles first,
# then the light ones in reverse) instead of cutting two-head groups between
# XCDs.  These shapes take that map (an even tile count, a multiple of 16
# workgroups, runs that are not whole two-head groups); every head is checked.
XCD_RUNS = [
    # B, H, Nq, Nk, d
    (1, 4, 2000, 2000, 128),      # 16 query tiles, 80-row tail: runs of 4 pairs
    (1, 6, 2048, 2048, 64),       # 96 workgroups, runs of 6 pairs
    (1, 12, 1024, 1024, 128),     # 8 query tiles per head
    (1, 4, 1500, 2048, 128),      # Nk > Nq (bottom-right causal alignment)
]


@pytest.mark.parametrize("case", XCD_RUNS, ids=lambda c: "-".join(map(str, c)))
def test_xcd_pair_runs_whole_heads(case):
    B, H, Nq, Nk, d = case
    n_qt = (Nq + 127) // 128
    total = B * H * n_qt
    assert n_qt % 2 == 0 and total % 16 == 0 and (total // 8) % (2 * n_qt) != 0   # the map's new branch
    banner(f"fwd xcd pair runs {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=990 + Nq + Nk + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, True)
    for b in range(B):
        for h in range(H):
            o_ref, lse_ref = attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), scale, True)
            check_forward(to64(o[b, h]), to64(lse[b, h]), o_ref, lse_ref, "bf16", f"{case} head {(b, h)}")


# ------------------------------------- persistent grid (causal d = 128, large)
# With causal masking, d = 128, an even query-tile count and at least 1024
# mirrored pairs of 128-row query tiles, the forward runs 512 persistent
# workgroups.  The pairs, head-major, are cut into eight equal runs, one per
# XCD (workgroup w is on XCD w mod 8); each workgroup takes pairs of its run
# and prefetches its next item across heads.  These shapes take that path
# with a ragged tail and a head count that leaves the shares unequal, and with
# Nq != Nk both ways.  Each sampled head is also run alone (one workgroup per
# query tile, every key walk upwards): the query tiles of the upper half, the
# first item of each pair, walk their keys upwards there too and must be
# bitwise equal; the lower half walk theirs downwards under the persistent
# schedule, so they agree to within rounding (the same sums in another order).
PERSIST = [
    # B, H, Nq, Nk
    (1, 200, 1700, 1700),     # 14 query tiles, 36-row tail; 1400 pairs: runs of 175 cut heads
    (4, 64, 1024, 1500),      # Nk > Nq (bottom-right causal alignment)
    (4, 64, 1280, 700),       # Nq > Nk: the first 580 rows see no key
]


def takes_persistent_grid(BH, n_qt):
    """The library's choice: causal d = 128 bf16, an even tile count, at
    least 1024 pairs and a last round that most workgroups share."""
    T = BH * (n_qt // 2)
    return n_qt % 2 == 0 and T >= 1024 and 10 * T >= 8 * 512 * -(-T // 512)


@pytest.mark.parametrize("case", PERSIST, ids=lambda c: "-".join(map(str, c)))
def test_persistent_grid_sampled_heads_and_bitwise(case):
    B, H, Nq, Nk = case
    d = 128
    n_qt = (Nq + 127) // 128
    assert takes_persistent_grid(B * H, n_qt)
    banner(f"fwd persistent {case}")
    q, k, v = wl.make_inputs(B, H, Nq, Nk, d, "bf16", seed=950 + Nq + Nk)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, True)
    g = torch.Generator().manual_seed(Nq * 5 + Nk)
    heads = [0, 1, 7, B * H - 1] + torch.randperm(B * H, generator=g)[:3].tolist()
    for bh in heads:
        b, h = divmod(bh, H)
        o_ref, lse_ref = attention_forward(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), scale, True)
        check_forward(to64(o[b, h]), to64(lse[b, h]), o_ref, lse_ref, "bf16", f"{case} head {bh}")
        o1, lse1 = gpu_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale, True)
        o1, lse1, oh, lseh = o1[0, 0].cpu(), lse1[0, 0].cpu(), o[b, h].cpu(), lse[b, h].cpu()
        up = (n_qt // 2) * 128   # first row of the upper half's query tiles
        assert torch.equal(o1[up:], oh[up:]), f"{case} head {bh}: O (upper tiles) differs from the lone head"
        assert torch.equal(lse1[up:], lseh[up:]), f"{case} head {bh}: LSE (upper tiles) differs"
        fin = torch.isfinite(lse1[:up])
        assert torch.equal(fin, torch.isfinite(lseh[:up])), f"{case} head {bh}: empty rows differ"
        assert (lse1[:up][fin] - lseh[:up][fin]).abs().max().item() <= 1e-5 if fin.any() else True
        assert (o1[:up].float() - oh[:up].float()).abs().max().item() <= 2e-2


# Fewer heads than XCDs, or a count that is not a multiple of eight: every
# XCD still gets an eighth of the pairs, so runs start and end inside heads
# and one head's pairs are served by several XCDs.  Rows are sampled per head
# (the heads are too long for the whole-head oracle), and each head is also
# run alone (fewer than 1024 pairs: one workgroup per query tile), whose
# upper-half query tiles must be bitwise equal.
PERSIST_FEW_HEADS = [
    # B, H, N
    (1, 3, 131000),    # 1024 query tiles (56-row tail), 1536 pairs: runs of 192 cut heads
    (1, 2, 131000),    # 1024 pairs: each head spans four runs
]


@pytest.mark.parametrize("case", PERSIST_FEW_HEADS, ids=lambda c: "-".join(map(str, c)))
def test_persistent_grid_few_heads_sampled_rows_and_bitwise(case):
    B, H, N = case
    d = 128
    n_qt = (N + 127) // 128
    assert takes_persistent_grid(B * H, n_qt) and not takes_persistent_grid(1, n_qt)   # a lone head is not
    banner(f"fwd persistent few heads {case}")
    q, k, v = wl.make_inputs(B, H, N, N, d, "bf16", seed=970 + H)
    scale = 1.0 / np.sqrt(d)
    o, lse = gpu_fwd(q, k, v, scale, True)
    up = (n_qt // 2) * 128   # first row of the upper half's query tiles
    for bh in range(B * H):
        b, h = divmod(bh, H)
        rows = wl.sample_rows(N, 128, 9700 + bh)
        o_ref, lse_ref = attention_forward_rows(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), scale, True, rows)
        check_forward(to64(o[b, h, rows]), to64(lse[b, h, rows]), o_ref, lse_ref, "bf16", f"{case} head {bh}")
        o1, lse1 = gpu_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale, True)
        assert torch.equal(o1[0, 0, up:].cpu(), o[b, h, up:].cpu()), f"{case} head {bh}: O (upper tiles) differs from the lone head"
        assert torch.equal(lse1[0, 0, up:].cpu(), lse[b, h, up:].cpu()), f"{case} head {bh}: LSE (upper tiles) differs"


# ------------------------------------------------------------------ page pins
def _pad_fp32(x, width):
    out = torch.zeros(x.shape[0], width, dtype=torch.float32)
    out[:, : x.shape[1]] = torch.as_tensor(x, dtype=torch.float32)
    return out


def _pin_run(q, K, V):
    """One query row through the GPU in fp32 with d zero-padded to 64 (the
    padding changes neither the logits nor the output columns kept)."""
    qp = _pad_fp32(np.atleast_2d(q), 64)[None, None]
    kp = _pad_fp32(K, 64)[None, None]
    vp = _pad_fp32(V, 64)[None, None]
    o, lse = gpu_fwd(qp, kp, vp, 1.0, False)
    return o[0, 0, 0].cpu().double().numpy(), float(lse[0, 0, 0])


def test_page_pin_worked_tiled_row():
    g = json.load(open(os.path.join(GOLDEN, "p4_tiled_row.json")))
    banner("pin: worked tiled row")
    K = np.array([[s, 0.0] for s in g["scores"]])
    o, lse = _pin_run([1.0, 0.0], K, np.array(g["values"]))
    assert np.max(np.abs(o[:2] - g["output"])) <= 0.5e-6 + 1e-6
    assert np.all(o[2:] == 0.0)
    assert abs(lse - np.log(np.sum(np.exp(g["scores"])))) <= 1e-5 * 4


def test_page_pin_one_row_attention():
    g = json.load(open(os.path.join(GOLDEN, "p1_attention_row.json")))
    banner("pin: one-row attention")
    o, _ = _pin_run(g["q"], np.array(g["K"]), np.array(g["V"]))
    assert np.max(np.abs(o[:2] - g["output"])) <= 1e-5 * 2


def test_page_pin_softmax_values_including_large_logits():
    g = json.load(open(os.path.join(GOLDEN, "p1_softmax.json")))
    for case in g["cases"]:
        banner(f"pin: softmax {case['x']}")
        x = np.array(case["x"])
        n = x.size
        K = np.zeros((n, 2)); K[:, 0] = x
        o, lse = _pin_run([1.0, 0.0], K, np.eye(n))
        assert np.all(np.isfinite(o)) and np.isfinite(lse)
        assert np.max(np.abs(o[:n] - case["y"])) <= 1e-6


# ------------------------------------------------------------ invariants/edges
def test_no_keys_gives_zero_rows():
    banner("Nk = 0")
    q = torch.randn(1, 2, 40, 64).to(torch.bfloat16).cuda()
    k = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = fa.attention_forward(q, k, k.clone(), causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_masked_keys_do_not_change_rows_bitwise():
    banner("masked keys perturbation")
    q, k, v = wl.make_inputs(1, 2, 300, 300, 128, "bf16", seed=99)
    o1, l1 = gpu_fwd(q, k, v, 0.1, True)
    i0 = 150
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i0 + 1:] = torch.randn_like(k2[:, :, i0 + 1:].float()).to(torch.bfloat16) * 8
    v2[:, :, i0 + 1:] = 100.0
    o2, l2 = gpu_fwd(q, k2, v2, 0.1, True)
    assert torch.equal(o1[:, :, : i0 + 1], o2[:, :, : i0 + 1])
    assert torch.equal(l1[:, :, : i0 + 1], l2[:, :, : i0 + 1])


def test_forward_is_deterministic():
    banner("determinism")
    q, k, v = wl.make_inputs(2, 4, 500, 500, 128, "bf16", seed=5)
    o1, l1 = gpu_fwd(q, k, v, 0.088, True)
    o2, l2 = gpu_fwd(q, k, v, 0.088, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_pointer_may_be_null():
    banner("lse = NULL")
    q, k, v = (t.cuda() for t in wl.make_inputs(1, 2, 130, 130, 64, "bf16", seed=6))
    o_ref, _ = fa.attention_forward(q, k, v, causal=True)
    o = torch.empty_like(q)
    st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, 1, 2, 130, 130, 64,
                   0.125, 1, fa.FA_BF16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(o, o_ref)


def test_shift_and_value_offset_invariance_fp32():
    banner("shift invariance fp32")
    q, k, v = wl.make_inputs(1, 2, 90, 90, 64, "fp32", seed=8)
    u = torch.randn(64)
    o1, l1 = gpu_fwd(q, k, v, 0.2, True)
    o2, l2 = gpu_fwd(q, k + u, v, 0.2, True)
    o3, _ = gpu_fwd(q, k, v + 3.0, 0.2, True)
    assert torch.max(torch.abs(o2 - o1)).item() <= 1e-5
    shift = 0.2 * (q @ u)
    assert torch.max(torch.abs((l2 - l1).cpu() - shift)).item() <= 1e-4
    assert torch.max(torch.abs(o3 - (o1 + 3.0))).item() <= 1e-5
