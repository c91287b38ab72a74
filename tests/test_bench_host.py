"""Host-side logic of bench.py (CPU only): the visible-pair count behind
every TFLOP/s figure, the algorithmic FLOP and byte counts of the workloads,
the HBM-counter summary, and the refusal of more than one GPU."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402
from oracle.attention import visible_mask  # noqa: E402


@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (7, 7, False, None), (7, 7, True, None), (5, 9, True, None), (9, 5, True, None),
    (20, 20, False, (3, 0)), (20, 33, False, (4, 2)), (33, 20, False, (None, 1)),
    (12, 12, False, (0, None)), (1, 64, True, None),
])
def test_visible_pairs_counts_the_oracle_mask(Nq, Nk, causal, window):
    mask = visible_mask(Nq, Nk, causal, window=window)
    assert bench.visible_pairs(Nq, Nk, causal, window) == int(mask.sum())


def test_flops_and_bytes_of_the_bench_workload():
    w = wl.LLAMA_CAUSAL
    # causal N(N+1)/2 pairs per head, 4*d FLOPs each (two products of 2*d)
    assert bench.fwd_flops(w) == 4 * 128 * (4096 * 4097 // 2) * 4 * 32 == 549890031616
    # read Q, K, V once, write O (bf16) and the fp32 LSE
    assert bench.algorithmic_bytes(w) == 4 * 32 * (4 * 4096 * 128 * 2 + 4096 * 4) == 538968064
    g = wl.GPT2_SMALL
    assert bench.fwd_flops(g) == 4 * 64 * 1024 * 1024 * 8 * 12


def _write_counters(d, kernel_values):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for kern, counter, vals in kernel_values:
            for v in vals:
                wr.writerow({"Kernel_Name": kern, "Counter_Name": counter, "Counter_Value": v})


def test_summarize_counters_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    mib = 64
    # the copy reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _write_counters(tmp_path / "cF", [("void copy_kernel<...>", "FETCH_SIZE", [mib * 512] * 3)])
    _write_counters(tmp_path / "cW", [("void copy_kernel<...>", "WRITE_SIZE", [mib * 1024] * 3)])
    # the kernel: per-dispatch KiB, averaged over dispatches
    _write_counters(tmp_path / "F", [("fwd_bf16_kernel", "FETCH_SIZE", [1000, 3000]),
                                     ("other", "FETCH_SIZE", [7])])
    _write_counters(tmp_path / "W", [("fwd_bf16_kernel", "WRITE_SIZE", [500, 500])])
    out = bench.summarize_counters("llama_causal_bf16", "fwd_bf16_kernel", str(tmp_path / "F"),
                                   str(tmp_path / "W"), str(tmp_path / "cF"), str(tmp_path / "cW"), mib)
    assert out["copy_calibration"]["fetch_scale"] == 2.0
    assert out["copy_calibration"]["write_scale"] == 1.0
    assert out["fetch_bytes"] == 2000 * 1024 * 2
    assert out["write_bytes"] == 500 * 1024
    assert out["hbm_bytes_per_launch"] == out["fetch_bytes"] + out["write_bytes"]
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_host_description_states_cores_and_model():
    h = bench.host_description()
    assert h["nproc"] == os.cpu_count() and h["nproc"] >= 1
    assert 1 <= h["affinity_cores"] <= h["nproc"]
    assert isinstance(h["cpu_model"], str) and h["cpu_model"]


def test_cpu_baseline_parity_leg_flags_a_wrong_output():
    """The parity check that precedes the timing: the oracle's own output
    passes, the same output with one element moved by 0.05 (beyond the bf16
    bar of 2e-2 on O) fails, and so does an LSE moved by 2e-3 (bar 1e-3)."""
    import torch
    from oracle import attention_forward
    w = wl.Workload("tiny", 1, 2, 40, 40, 64, "bf16", True, seed=77)
    q, k, v = wl.make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed)
    o = torch.zeros(w.B, w.H, w.Nq, w.d, dtype=torch.float64)
    lse = torch.zeros(w.B, w.H, w.Nq, dtype=torch.float64)
    for h in range(w.H):
        oh, lh = attention_forward(q[0, h].double().numpy(), k[0, h].double().numpy(),
                                   v[0, h].double().numpy(), w.scale, w.causal)
        o[0, h], lse[0, h] = torch.from_numpy(oh), torch.from_numpy(lh)
    res, par = bench.cpu_baseline(w, q, k, v, target_s=30.0, o_gpu=o, lse_gpu=lse)
    assert par["ok"] and par["heads_checked"] == 2 and par["o_max_abs_err"] == 0.0
    assert res["cores"] >= 1 and res["nproc"] == os.cpu_count() and "cpu_model" in res
    bad = o.clone()
    bad[0, 1, 17, 5] += 0.05
    assert not bench.cpu_baseline(w, q, k, v, target_s=30.0, o_gpu=bad, lse_gpu=lse)[1]["ok"]
    badl = lse.clone()
    badl[0, 0, 3] += 2e-3
    assert not bench.cpu_baseline(w, q, k, v, target_s=30.0, o_gpu=o, lse_gpu=badl)[1]["ok"]
