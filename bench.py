"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-train-step] [--cold]

A step is one fa_fwd launch over the whole workload (default: B=4 H=32
N=4096 d=128 bf16 causal, LSE saved), with Q, K, V already resident in device
memory.  W untimed warm-up steps, then K steps timed with HIP events recorded
on the stream the kernel is launched on, bracketed by device synchronisation.
Throughput is causal-adjusted: 4*d FLOPs per visible (query, key) pair.

Prints ONE JSON line.  ``roofline`` compares the kernel against MI355X's
published dense bf16 MFMA peak (2.5 PFLOP/s); ``traffic`` is taken from the
committed rocprofv3 counter summary when it was measured on the current kernel
source, else null.  ``hbm`` gives the algorithmic bytes (read Q, K, V once,
write O and LSE) per launch and the rate they are moved at; ``cold`` (with
--cold, and always for the short-sequence GPT-2-shaped workload) repeats the
timing one launch at a time after flushing L2 and the Infinity Cache.
``train_step`` times fa_fwd and fa_bwd (both modes) on the training-step
workload.  ``mfma_ceiling`` times an 8192^3 bf16 torch.matmul (hipBLASLt) on
the same GPU: the MFMA rate the vendor library sustains, as context for
``roofline.frac``; it runs before the warm-up, which takes the chip through
its clock transient (boost, then power limit) before the timed launches.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on the host cores (core count and CPU model stated); that leg runs
before the timing and also compares the sampled heads of the GPU's own output
with the oracle (``parity``; a failure exits non-zero).  ``samples`` gives the
per-launch median, min and interquartile range of the K timed launches;
``device`` the GPU and software stack; ``mfma_ceiling.probe`` the bf16 MFMA rate
and core clock this GPU sustains under a pure MFMA load (libfa_probe.so).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, causal-adjusted) and % of MFMA peak, 1×MI355X"
PEAK = {"bf16": 2500.0, "fp32": 157.3}          # TFLOP/s, MI355X published dense figures
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["exact_attention_20_amd/csrc/fa_fwd.hip", "exact_attention_20_amd/csrc/fa_device.h"]


def visible_pairs(Nq: int, Nk: int, causal: bool, window=None) -> int:
    """Number of (query, key) pairs the mask leaves visible (bottom-right
    aligned causal mask: key j visible to query i iff j <= i + Nk - Nq; a
    local window (wl, wr): iff i + off - wl <= j <= i + off + wr, off = Nk - Nq,
    a None side unbounded)."""
    if window is None and not causal:
        return Nq * Nk
    wl, wr = window if window is not None else (None, 0)
    off = Nk - Nq
    total = 0
    for i in range(Nq):
        lo = 0 if wl is None else max(0, i + off - wl)
        hi = Nk - 1 if wr is None else min(Nk - 1, i + off + wr)
        total += max(0, hi - lo + 1)
    return total


def atomic_adds(Nq: int, Nk: int, causal: bool, window, d: int) -> int:
    """float32 atomic adds of one head in the backward's atomic mode: its
    key-side kernel walks, for each 128-key tile, the 64-query steps that
    can see it (as the kernel bounds them) and adds d values per query row
    below Nq in every step."""
    wl, wr = window if window is not None else ((None, 0) if causal else (None, None))
    off = Nk - Nq
    offr = None if wr is None else off + wr
    offl = None if wl is None else off - wl
    total = 0
    for k0 in range(0, Nk, 128):
        qstart = 0 if offr is None else max(0, k0 - offr)
        qend = Nq if offl is None else max(0, min(Nq, k0 + 128 - offl))
        for q0 in range(qstart // 64 * 64, qend, 64):
            total += min(64, Nq - q0) * d
    return total


def fwd_flops(w) -> int:
    return 4 * w.d * visible_pairs(w.Nq, w.Nk, w.causal, w.window) * w.B * w.H


def algorithmic_bytes(w) -> int:
    """Compulsory HBM bytes of one forward launch: read Q, K, V once, write O
    and the fp32 LSE."""
    esz = 2 if w.dtype == "bf16" else 4
    return w.B * w.H * ((2 * w.Nq + 2 * w.Nk) * w.d * esz + 4 * w.Nq)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload_name: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source and this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload_name)
    if not entry or t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def blas_threads() -> int:
    """Threads of the BLAS the oracle's NumPy products run on."""
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(blas) if blas else 1
    except Exception:
        return 1


def host_description() -> dict:
    """The host cores the oracle runs on: logical CPUs, the ones this process
    may use, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return {"nproc": os.cpu_count(), "affinity_cores": affinity, "cpu_model": model}


def cpu_baseline(w, q, k, v, target_s: float = 15.0, o_gpu=None, lse_gpu=None):
    """Time the fp64 oracle (as it stands) on whole heads of the workload until
    about ``target_s`` seconds of CPU work; report its causal-adjusted rate.
    With the GPU's outputs of the same workload (host tensors), every head the
    oracle computes is also compared with them at the parity tolerances (the
    check that precedes the GPU timing)."""
    import numpy as np
    from oracle import attention_forward
    threads = blas_threads()
    per_head_flops = fwd_flops(w) / (w.B * w.H)
    done, t_total = 0, 0.0
    heads = w.B * w.H
    err_o, err_l, ref_o, ref_l = 0.0, 0.0, 0.0, 1.0
    while done < heads and t_total < target_s:
        b, h = divmod(done, w.H)
        qh, kh, vh = (t[b, h].double().numpy() for t in (q, k, v))
        t0 = time.perf_counter()
        o_ref, lse_ref = attention_forward(qh, kh, vh, w.scale, w.causal, window=w.window)
        t_total += time.perf_counter() - t0
        if o_gpu is not None:
            live = ~np.isneginf(lse_ref)
            err_o = max(err_o, float(np.max(np.abs(o_gpu[b, h].double().numpy() - o_ref))))
            ref_o = max(ref_o, float(np.max(np.abs(o_ref))))
            if live.any():
                err_l = max(err_l, float(np.max(np.abs(lse_gpu[b, h].double().numpy()[live] - lse_ref[live]))))
                ref_l = max(ref_l, float(np.max(np.abs(lse_ref[live]))))
        done += 1
    rate = per_head_flops * done / t_total / 1e12
    res = {"value": round(rate, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} of {heads} (batch, head) pairs of {w.describe()}, fp64 NumPy, "
                     f"{t_total:.1f} s; numpy exp single-threaded, BLAS {threads} threads",
           "blas_threads": threads, **host_description()}
    parity = None
    if o_gpu is not None:
        if w.dtype == "bf16":
            tol = {"o_abs": 2e-2, "lse_abs": 1e-3}
            ok = err_o <= tol["o_abs"] and err_l <= tol["lse_abs"]
        else:   # fp32: relative to the largest reference magnitude
            tol = {"o_rel": 1e-5, "lse_rel": 1e-5}
            ok = err_o <= tol["o_rel"] * ref_o and err_l <= tol["lse_rel"] * ref_l
        parity = {"heads_checked": done, "heads": heads, "o_max_abs_err": err_o, "lse_max_abs_err": err_l,
                  "tolerance": tol, "ok": bool(ok),
                  "note": "whole heads of the timed workload's own output against the fp64 oracle, "
                          "before the timed launches"}
    return res, parity


def timed_launches(fn, stream, steps: int):
    """K back-to-back launches of ``fn`` with a HIP event recorded on
    ``stream`` before each and after the last, bracketed by device
    synchronisation.  Returns the mean ms per launch over the whole region
    (the step time) and the per-launch samples' median, min and
    interquartile range."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i].record(stream)
        fn()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    total = ev[0].elapsed_time(ev[steps])

    def q(f):
        x = f * (len(per) - 1)
        lo = int(math.floor(x))
        hi = min(lo + 1, len(per) - 1)
        return per[lo] + (per[hi] - per[lo]) * (x - lo)

    return total / steps, {"n": steps, "median_ms": round(q(0.5), 5), "min_ms": round(per[0], 5),
                           "iqr_ms": round(q(0.75) - q(0.25), 5), "p25_ms": round(q(0.25), 5),
                           "p75_ms": round(q(0.75), 5)}


def device_description() -> dict:
    """The GPU, its architecture and compute units, and the software stack."""
    import torch
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm, "hip": torch.version.hip,
            "torch": torch.__version__}


def mfma_probe(grid: int = 1024, iters: int = 4000, repeats: int = 3) -> dict:
    """The bf16 MFMA rate this GPU sustains under a pure MFMA load
    (libfa_probe.so: four waves per SIMD, 16 independent 32x32x16 MFMAs per
    round, no memory traffic) and the core clock meanwhile (s_memtime against
    the 100 MHz s_memrealtime), median of ``repeats`` launches."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_20_amd", "libfa_probe.so"))
    lib.fa_probe_mfma_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    lib.fa_probe_mfma_flops.restype = ctypes.c_double
    lib.fa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda:0")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream()
    flops = lib.fa_probe_mfma_flops(grid, iters)
    res = []
    for _ in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.fa_probe_mfma_launch(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                                      grid, iters, ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"fa_probe_mfma_launch failed with {st}")
        cyc, ticks = (int(x) for x in clocks.cpu().tolist())
        res.append((flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, cyc / (ticks / 100e6) / 1e9))
    res = sorted(res[1:])
    tf, ghz = res[len(res) // 2]
    return {"op": "libfa_probe: 32x32x16 bf16 MFMA chains, 4 waves/SIMD, no memory traffic",
            "tflops": round(tf, 1), "sclk_ghz": round(ghz, 3), "frac_of_published": round(tf / PEAK["bf16"], 4)}


def atomic_probe(grid: int = 8192, repeats: int = 5) -> dict:
    """Chip-wide rate of float32 buffer atomic adds to distinct addresses
    (libfa_probe.so), the bound of the backward's atomic-dQ mode; median of
    ``repeats`` launches."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_20_amd", "libfa_probe.so"))
    lib.fa_probe_atomic_elems.restype = ctypes.c_long
    lib.fa_probe_atomic_elems.argtypes = [ctypes.c_int]
    lib.fa_probe_atomic_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    n = lib.fa_probe_atomic_elems(grid)
    buf = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.fa_probe_atomic_launch(ctypes.c_void_p(buf.data_ptr()), grid, ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"fa_probe_atomic_launch failed with {st}")
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts[1:])[repeats // 2]
    return {"op": "libfa_probe: fp32 buffer atomic add, distinct addresses, 256 B per wave instruction",
            "adds_per_s": round(n / (ms * 1e-3), -8), "ms": round(ms, 4), "adds": n}


def valu_probe(sclk_ghz: float, repeats: int = 5) -> dict:
    """Cycles a wave's v_exp_f32 and v_fma_f32 hold a SIMD (libfa_probe.so,
    8 waves per SIMD, 8 independent chains per lane), at the core clock
    ``sclk_ghz``: an exponential (with its add), two FMAs, and both mixed --
    mixed near the sum of the two means the exponential shares the FMA pipe."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_20_amd", "libfa_probe.so"))
    lib.fa_probe_valu_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_long), ctypes.POINTER(ctypes.c_long)]
    grid = 256 * 32
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for variant, name in ((0, "exp+add"), (1, "fma x2"), (2, "exp+add, fma x2")):
        ne, no = ctypes.c_long(), ctypes.c_long()
        ts = []
        for _ in range(repeats + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = lib.fa_probe_valu_launch(ctypes.c_void_p(out.data_ptr()), grid, variant,
                                          ctypes.c_void_p(stream.cuda_stream), ctypes.byref(ne), ctypes.byref(no))
            e1.record(stream)
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"fa_probe_valu_launch failed with {st}")
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts[1:])[repeats // 2]
        waves_per_simd = grid * 4 / 1024
        cyc_per_step = ms * 1e-3 * sclk_ghz * 1e9 / waves_per_simd / (ne.value or no.value // (2 if variant == 1 else 3))
        res[name] = {"ms": round(ms, 4), "cycles_per_step": round(cyc_per_step, 2)}
    res["note"] = ("cycles one wave's step holds its SIMD (8 waves per SIMD); a step is one chain's "
                   "exp+add, two FMAs, or both")
    return res


def soft_exp2_ab(fa, w, argv, stream, steps: int, rounds: int) -> dict:
    """fa_fwd (period 0) against fa_fwd_soft_exp2 with periods 8, 4 and 2 on
    one workload: after the hardware ceilings (which settle the clock) and a
    warm-up of each, ``rounds`` rounds that time ``steps`` launches of every
    variant in turn; the median over rounds of each variant's ms per launch.
    (Its parity is the GPU tests'.)"""
    fns = {}
    for period in (0, 8, 4, 2):
        if period == 0:
            fns[period] = lambda: fa.fa_fwd(*argv)
        else:
            fns[period] = (lambda per: lambda: fa.fa_fwd_soft_exp2(*argv[:13], per, argv[13]))(period)
    gemm_ceiling()
    mfma_probe()
    res = {p_: [] for p_ in fns}
    for p_, fn in fns.items():
        time_launches(fn, stream, 3, 3)
    for _ in range(rounds):
        for p_, fn in fns.items():
            res[p_].append(time_launches(fn, stream, steps, 1))
    med = {p_: sorted(v)[len(v) // 2] for p_, v in res.items()}
    flops = fwd_flops(w)
    return {"soft_exp2_ab": {"workload": w.name, "rounds": rounds, "steps": steps,
                             "median_ms": {str(p_): round(m, 5) for p_, m in med.items()},
                             "tflops": {str(p_): round(flops / (m * 1e-3) / 1e12, 1) for p_, m in med.items()},
                             "vs_hardware_exp": {str(p_): round(med[0] / m - 1.0, 4) for p_, m in med.items() if p_},
                             "note": "period 0 = fa_fwd (v_exp_f32 throughout); period p = one exponential "
                                     "in p by the degree-3 polynomial on the FMA pipe"}}


def settle_clock(fn, min_ms: float = 150.0, min_launches: int = 50) -> dict:
    """Launch the timed workload untimed until at least ``min_ms`` of wall
    clock and ``min_launches`` launches have passed, so that the warm-up and
    the timed launches see the chip's sustained clock.  After an idle host
    phase the chip runs a launch at boost clock, then up to 25% slower while
    it meets its power limit, and only after about 50 launches (≈ 27 ms) of
    the Llama-shaped forward settles to the rate it then holds for at least
    2,000 launches (517-522 µs per launch, one box)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= min_ms and n >= min_launches:
            return {"launches": n, "ms": round(el, 1),
                    "note": "untimed launches of the timed workload before the warm-up: the sustained clock"}


def time_launches(fn, stream, steps: int, warmup: int) -> float:
    """Average ms per call of ``fn`` with HIP events on ``stream``."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def train_step_timing(fa, wl, steps: int, warmup: int, window=None, w=None):
    """fa_fwd then fa_bwd on the training-step workload (B=4 H=16 N=4096
    d=64 bf16 causal; or the bf16 workload ``w``, with dO drawn after its
    inputs), each timed on its own with HIP events; inputs, outputs and the
    backward workspace are resident before timing starts.  With a local
    ``window`` (wl, wr) the same shape runs fa_fwd_window and fa_bwd_window
    instead of the causal calls."""
    import torch
    w = wl.TRAIN_STEP if w is None else w
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in wl.make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed,
                                                     with_do=True))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    fwd_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), fa.FA_BF16, sh)
    f_fwd, f_bwd = fa.fa_fwd, fa.fa_bwd
    wa = None
    if window is not None:
        wa = tuple(-1 if x is None else x for x in window)
        fwd_args = fwd_args[:11] + wa + fwd_args[12:]
        f_fwd, f_bwd = fa.fa_fwd_window, fa.fa_bwd_window

    def fwd():
        st = f_fwd(*fwd_args)
        if st != 0:
            raise fa.FAError(st, f_fwd.__name__)

    def bwd_fn(det):
        need = fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, fa.FA_BF16, det)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        mask = (int(w.causal),) if wa is None else wa
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                w.B, w.H, w.Nq, w.Nk, w.d, w.scale) + mask + (fa.FA_BF16, det, ws.data_ptr(), need, sh)

        def bwd():
            st = f_bwd(*args)
            if st != 0:
                raise fa.FAError(st, f_bwd.__name__)
        bwd.ws = ws
        return bwd

    # the inputs were just made on the host, so each call settles the clock
    # first (settle_clock) as the timed workload does
    fwd()
    settle_clock(fwd, min_ms=100.0)
    ms_f = time_launches(fwd, stream, steps, warmup)
    bwd_det, bwd_atomic = bwd_fn(1), bwd_fn(0)
    settle_clock(bwd_det, min_ms=100.0)
    ms_b = time_launches(bwd_det, stream, steps, warmup)
    settle_clock(bwd_atomic, min_ms=100.0)
    ms_a = time_launches(bwd_atomic, stream, steps, warmup)
    causal = w.causal if window is None else False
    pairs = visible_pairs(w.Nq, w.Nk, causal, window) * w.B * w.H
    shape = w.describe() if window is None else w.describe().replace("causal", f"window {window}")
    # the atomic mode's float32 adds: 64 x d per (64-query, 128-key) tile pair
    atomics = atomic_adds(w.Nq, w.Nk, causal, window, w.d) * w.B * w.H
    return {"workload": w.name, "shape": shape,
            "fwd_ms": round(ms_f, 5), "fwd_tflops": round(4 * w.d * pairs / ms_f / 1e9, 3),
            "bwd_ms": round(ms_b, 5), "bwd_tflops": round(10 * w.d * pairs / ms_b / 1e9, 3),
            "bwd_atomic_ms": round(ms_a, 5),
            "bwd_atomic_tflops": round(10 * w.d * pairs / ms_a / 1e9, 3),
            "bwd_atomic_adds": atomics,
            "bwd_flops": 10 * w.d * pairs,
            "note": "bwd = deterministic mode (dQ kernel + key-side kernel(s), the default); "
                    "bwd_atomic = pre-pass, one key-side kernel adding dQ with fp32 atomics, dQ "
                    "conversion; both counted at 10*d FLOPs per visible pair"}


def gemm_ceiling(n: int = 8192, iters: int = 20) -> dict:
    """Context for the roofline: the bf16 MFMA rate the vendor library itself
    sustains on this GPU, one n x n x n torch.matmul (hipBLASLt) timed with HIP
    events.  The published 2.5 PFLOP/s assumes the 2.4 GHz peak clock, which
    a chip running MFMAs flat out does not hold."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to(dev)
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to(dev)
    c = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    ms = time_launches(lambda: torch.matmul(a, b, out=c), stream, iters, 3)
    del a, b, c
    return {"op": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)", "ms": round(ms, 4),
            "tflops": round(2 * n ** 3 / ms / 1e9, 1)}


def bench_varlen(fa, wl, w, args) -> dict:
    """One fa_fwd_varlen launch over the packed variable-length workload per
    step, timed like the fixed-length line; FLOPs are 4*d per visible pair
    summed over the sequences."""
    import torch
    dev = torch.device("cuda:0")
    L = w.lengths()
    q, k, v, cu_q, cu_k = wl.varlen_workload_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    cq, ck = cu_q.to(dev), cu_k.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.H, qd.shape[1]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    T = qd.shape[1]
    mask = (-1, 0) if w.causal else (-1, -1)
    argv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
            cq.data_ptr(), ck.data_ptr(), len(L), w.H, T, T, max(L), max(L), w.d, w.scale,
            mask[0], mask[1], fa.FA_BF16, stream.cuda_stream)

    def step():
        st = fa.fa_fwd_varlen(*argv)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_varlen")

    # the ceilings first, as in the fixed-length line (they take the chip
    # through its clock transient before the warm-up)
    gc = None
    if not args.no_gemm_ceiling:
        gc = gemm_ceiling()
        gc["probe"] = mfma_probe()
    settle = settle_clock(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, samples = timed_launches(step, stream, args.steps)
    pairs = sum(visible_pairs(n, n, w.causal) for n in L)
    flops = 4 * w.d * pairs * w.H
    tflops = flops / (ms * 1e-3) / 1e12
    nbytes = w.H * (4 * T * w.d * 2 + 4 * T)
    result = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle": settle, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) inputs; seeded log-uniform sequence lengths)",
        "config": {"workload": w.name, "sequences": len(L), "min_len": min(L), "max_len": max(L),
                   "total_tokens": T, "H": w.H, "d": w.d, "causal": w.causal, "lse_saved": True,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK[w.dtype],
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK[w.dtype], 4),
                     "traffic": traffic_for(w.name)},
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "peak_GBps": 8000.0, "note": "algorithmic bytes / launch time, warm caches"},
        "samples": {**samples, "note": "per-launch HIP events inside the timed region"},
        "device": device_description(),
    }
    if gc is not None:
        gc["value_over_gemm"] = round(tflops / gc["tflops"], 4)
        gc["probe"]["value_over_probe"] = round(tflops / gc["probe"]["tflops"], 4)
        result["mfma_ceiling"] = gc
    if not args.no_train_step:
        # fa_bwd_varlen on the same packed batch (dO drawn after the inputs),
        # deterministic mode then atomic mode
        g = torch.Generator(device="cpu").manual_seed(w.seed + 1)
        do = torch.randn(qd.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        step()
        bwd_ms = {}
        for det in (1, 0):
            need = fa.fa_bwd_varlen_workspace_bytes(w.H, T, w.d, fa.FA_BF16, det)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            bargv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()) + argv[5:17] + \
                    (fa.FA_BF16, det, ws.data_ptr(), need, stream.cuda_stream)

            def bwd():
                st = fa.fa_bwd_varlen(*bargv)
                if st != 0:
                    raise fa.FAError(st, "fa_bwd_varlen")

            settle_clock(bwd, min_ms=100.0)
            bwd_ms[det] = time_launches(bwd, stream, 20, 5)
            del ws
        result["backward"] = {"bwd_ms": round(bwd_ms[1], 5),
                              "bwd_tflops": round(10 * w.d * pairs * w.H / bwd_ms[1] / 1e9, 3),
                              "bwd_atomic_ms": round(bwd_ms[0], 5),
                              "bwd_atomic_tflops": round(10 * w.d * pairs * w.H / bwd_ms[0] / 1e9, 3),
                              "note": "fa_bwd_varlen: deterministic mode (dQ kernel + key-side kernel), "
                                      "then the atomic mode; 10*d FLOPs per visible pair"}
    if not args.no_cpu_baseline:
        from oracle import attention_forward
        # whole (head, sequence) pairs, head by head, until ~15 s of CPU work
        done, t_total, done_pairs = 0, 0.0, 0
        while done < w.H * len(L) and t_total < 15.0:
            h, b = divmod(done, len(L))
            s, e = int(cu_q[b]), int(cu_q[b + 1])
            t0 = time.perf_counter()
            attention_forward(q[h, s:e].double().numpy(), k[h, s:e].double().numpy(),
                              v[h, s:e].double().numpy(), w.scale, w.causal)
            t_total += time.perf_counter() - t0
            done_pairs += visible_pairs(L[b], L[b], w.causal)
            done += 1
        result["cpu_baseline"] = {
            "value": round(4 * w.d * done_pairs / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {w.H * len(L)} (head, sequence) pairs, fp64 NumPy, "
                      f"{t_total:.1f} s; numpy exp single-threaded",
            "blas_threads": blas_threads(), **host_description()}
    return result


def _counter_means(csv_dir: str, counter: str):
    """Per-kernel mean of one rocprofv3 --pmc counter (KiB per dispatch for
    FETCH_SIZE / WRITE_SIZE) from the counter_collection CSVs in csv_dir."""
    import csv
    import glob
    sums = {}
    for path in glob.glob(os.path.join(csv_dir, "*counter_collection.csv")):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                acc = sums.setdefault(row["Kernel_Name"], [0.0, 0])
                acc[0] += float(row["Counter_Value"])
                acc[1] += 1
    return {k: v[0] / v[1] for k, v in sums.items()}


def summarize_sq(csv_dirs, sclk_ghz: float) -> str:
    """Markdown table of per-dispatch means of every counter in the
    rocprofv3 --pmc CSVs of ``csv_dirs``, one row per kernel variant (name,
    grid, VGPRs, LDS bytes), with the dispatch duration and, where the SQ
    counters are there, other VALU instructions and LDS instructions per MFMA
    and the MFMA pipes' busy share: SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs
    x duration x ``sclk_ghz``."""
    import csv
    import glob
    rows = {}
    for d in csv_dirs:
        for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
            with open(path) as f:
                for r in csv.DictReader(f):
                    key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["VGPR_Count"]) + int(r["Accum_VGPR_Count"]),
                           int(r["LDS_Block_Size"]))
                    disp = rows.setdefault(key, {})
                    c = disp.setdefault((path, r["Dispatch_Id"]), {})
                    c[r["Counter_Name"]] = float(r["Counter_Value"])
                    c["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    names = sorted({n for disp in rows.values() for c in disp.values() for n in c if not n.startswith("_")})
    out = ["| kernel (grid, VGPRs, LDS B) | dispatches | us | " + " | ".join(names) +
           " | other VALU / MFMA | LDS / MFMA | MFMA busy |",
           "|---" * (len(names) + 6) + "|"]
    for key, disp in sorted(rows.items(), key=lambda kv: -len(kv[1])):
        n = len(disp)
        mean = {nm: sum(c.get(nm, 0.0) for c in disp.values()) / n for nm in names}
        us = sum(c["_ns"] for c in disp.values()) / n / 1e3
        mf = mean.get("SQ_INSTS_MFMA", 0.0)
        valu = f"{(mean['SQ_INSTS_VALU'] - mf) / mf:.2f}" if mf and "SQ_INSTS_VALU" in mean else ""
        lds = f"{mean['SQ_INSTS_LDS'] / mf:.2f}" if mf and "SQ_INSTS_LDS" in mean else ""
        busy = (f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * us * 1e3 * sclk_ghz):.3f}"
                if "SQ_VALU_MFMA_BUSY_CYCLES" in mean else "")
        out.append(f"| {key[0]} ({key[1] // 256 if key[1] % 256 == 0 else key[1]}, {key[2]}, {key[3]}) | {n} | "
                   f"{us:.1f} | " + " | ".join(f"{mean[nm]:,.0f}" for nm in names) + f" | {valu} | {lds} | {busy} |")
    return "\n".join(out)


def summarize_counters(workload: str, kernel: str, fetch_dir: str, write_dir: str,
                       copy_fetch_dir: str, copy_write_dir: str, copy_mib: int) -> dict:
    """HBM bytes per launch of ``kernel`` from two --pmc runs (FETCH_SIZE,
    WRITE_SIZE), each scaled by what the same counter reads for a plain
    device copy of ``copy_mib`` MiB; written to profiles/traffic.json."""
    copy_bytes = copy_mib << 20
    cf = max(v for k, v in _counter_means(copy_fetch_dir, "FETCH_SIZE").items() if "copy" in k.lower())
    cw = max(v for k, v in _counter_means(copy_write_dir, "WRITE_SIZE").items() if "copy" in k.lower())
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fk = _counter_means(fetch_dir, "FETCH_SIZE")[kernel] * 1024.0 * f_scale
    wk = _counter_means(write_dir, "WRITE_SIZE")[kernel] * 1024.0 * w_scale
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    if t.get("kernel_source_hash") != kernel_source_hash():
        t = {"kernel_source_hash": kernel_source_hash(), "workloads": {}}
    t["workloads"][workload] = {
        "kernel": kernel, "hbm_bytes_per_launch": int(fk + wk),
        "fetch_bytes": int(fk), "write_bytes": int(wk),
        "copy_calibration": {"bytes": copy_bytes, "fetch_scale": round(f_scale, 4),
                             "write_scale": round(w_scale, 4)},
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    return t["workloads"][workload]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama_causal_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--train-workload", default="train_step_bf16",
                    help="bf16 workload of the fwd+bwd leg (default: the training step)")
    ap.add_argument("--no-train-step", action="store_true",
                    help="skip the forward+backward timing on the training-step workload")
    ap.add_argument("--no-gemm-ceiling", action="store_true",
                    help="skip the vendor-GEMM reference rate reported beside the roofline")
    ap.add_argument("--cold", action="store_true",
                    help="also time launches one by one after flushing L2 and the Infinity Cache "
                         "(a 512 MiB write before each); on by default for the short-sequence "
                         "GPT-2-shaped workload, whose inputs fit in the Infinity Cache")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device copies of MIB MiB "
                         "(reference kernel for scaling the HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=5,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "COPY_MIB"),
                    help="write profiles/traffic.json for --workload from rocprofv3 --pmc output "
                         "directories (no GPU needed)")
    ap.add_argument("--probes", action="store_true",
                    help="print the MFMA, float32 atomic and VALU (exp vs FMA) probes of "
                         "libfa_probe.so as one JSON line and exit")
    ap.add_argument("--summarize-sq", nargs="+", metavar="PMC_DIR",
                    help="print per-kernel means of the counters in rocprofv3 --pmc output "
                         "directories as a markdown table (no GPU needed)")
    ap.add_argument("--soft-exp2-ab", type=int, default=0, metavar="ROUNDS",
                    help="instead of the benchmark line, time fa_fwd against fa_fwd_soft_exp2 "
                         "(one exponential in 8, 4, 2 by the FMA-pipe polynomial) on --workload "
                         "in ROUNDS interleaved rounds of --steps launches; one JSON line")
    ap.add_argument("--sclk-ghz", type=float, default=2.1,
                    help="core clock for --summarize-sq's MFMA busy share")
    args = ap.parse_args()
    if args.probes:
        import torch
        if not torch.cuda.is_available():
            print("bench.py --probes needs a GPU", file=sys.stderr)
            sys.exit(1)
        mp = mfma_probe()
        print(json.dumps({"mfma": mp, "atomic": atomic_probe(), "valu": valu_probe(mp["sclk_ghz"]),
                          "device": device_description()}), flush=True)
        return
    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq, args.sclk_ghz))
        return
    if args.summarize_counters:
        fd, wd, cfd, cwd, mib = args.summarize_counters
        kern = "fwd_bf16_kernel" if "bf16" in args.workload else "fwd_f32_kernel"
        print(json.dumps(summarize_counters(args.workload, kern, fd, wd, cfd, cwd, int(mib))))
        return
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(across GPUs the forward would shard over batch*head with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_20_amd as fa
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == wl.VARLEN_CAUSAL.name:
        print(json.dumps(bench_varlen(fa, wl, wl.VARLEN_CAUSAL, args)), flush=True)
        return
    w = {x.name: x for x in wl.ALL}[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = wl.workload_inputs(w)[:3]
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    dtype_code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F32
    argv = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), dtype_code, sh)

    def step():
        st = fa.fa_fwd(*argv)
        if st != 0:
            raise fa.FAError(st, "fa_fwd")

    if w.window is not None:
        # local window: fa_fwd_window, (wl, wr) in place of the causal flag
        wargv = argv[:11] + tuple(-1 if x is None else x for x in w.window) + argv[12:]

        def step():  # noqa: F811
            st = fa.fa_fwd_window(*wargv)
            if st != 0:
                raise fa.FAError(st, "fa_fwd_window")

    # Decoding (a few query rows against a long key range) runs the split-KV
    # path: it is HBM-bound, so its roofline is the 8 TB/s HBM peak.
    decode = w.name == "decode_bf16"
    unsplit_ms = None
    if decode:
        unsplit_ms = time_launches(step, stream, max(5, args.steps // 5), 3)
        need = fa.fa_fwd_splitkv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, dtype_code, 0)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        sargv = argv[:13] + (0, ws.data_ptr(), need, sh)

        def step():  # noqa: F811
            st = fa.fa_fwd_splitkv(*sargv)
            if st != 0:
                raise fa.FAError(st, "fa_fwd_splitkv")

    if args.soft_exp2_ab:
        print(json.dumps(soft_exp2_ab(fa, w, argv, stream, args.steps, args.soft_exp2_ab)), flush=True)
        return

    # Parity first (the cpu_baseline leg): one launch, its output against the
    # fp64 oracle on every head the bounded CPU sample reaches.
    cpu_res, parity = None, None
    if not args.no_cpu_baseline:
        step()
        torch.cuda.synchronize()
        cpu_res, parity = cpu_baseline(w, q, k, v, o_gpu=o.cpu(), lse_gpu=lse.cpu())
        if parity is not None and not parity["ok"]:
            print(json.dumps({"error": "parity check failed before timing", "parity": parity}), flush=True)
            sys.exit(1)

    # The hardware ceilings (one hipBLASLt GEMM, the MFMA probe) run before the
    # warm-up.  A kernel launched after an idle host phase (the oracle above)
    # runs its first 2 ms at boost clock, then up to 25% slower while the chip
    # meets its power limit, and settles after about 10 ms of MFMA load; the
    # ceilings' 30 ms of full-rate MFMA work take it through that transient,
    # so the warm-up and the timed launches see the settled clock.
    gc = None
    if w.dtype == "bf16" and not args.no_gemm_ceiling:
        gc = gemm_ceiling()
        gc["probe"] = mfma_probe()
    # then the timed workload itself until the clock has settled
    settle = settle_clock(step)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, samples = timed_launches(step, stream, args.steps)
    flops = fwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK[w.dtype]

    traffic = traffic_for(w.name)
    nbytes = algorithmic_bytes(w)
    if w.window is not None:
        wl_, wr_ = w.window
        result_window = {"window": [wl_, wr_]}
    else:
        result_window = {}
    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, **result_window, "lse_saved": True,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic},
        "samples": {**samples, "median_tflops": round(flops / (samples["median_ms"] * 1e-3) / 1e12, 3),
                    "note": "per-launch HIP events inside the timed region; value and ms_per_step are "
                            "the mean over the whole region"},
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "peak_GBps": 8000.0, "note": "algorithmic bytes / launch time, warm caches"},
        "device": device_description(),
        "parity": parity if parity is not None else {"ok": None, "note": "skipped with --no-cpu-baseline"},
    }
    if decode:
        gbps = nbytes / (ms * 1e-3) / 1e9
        result["metric"] = "attention decode (split-KV) HBM GB/s, 1xMI355X"
        result["value"] = round(gbps, 1)
        result["unit"] = "GB/s"
        result["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
                              "frac": round(gbps / 8000.0, 4), "traffic": traffic}
        result["decode"] = {"path": "fa_fwd_splitkv, automatic run count", "unsplit_fa_fwd_ms": round(unsplit_ms, 5),
                            "unsplit_GBps": round(nbytes / (unsplit_ms * 1e-3) / 1e9, 1),
                            "tflops": round(tflops, 3)}
    if args.cold or w.name == "gpt2_small_bf16":
        # L2 (4 MiB per XCD) and the 256 MiB Infinity Cache are flushed by a
        # 512 MiB write before every launch; each launch is timed on its own.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        times = []
        for _ in range(max(10, args.steps // 2)):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        cms = times[len(times) // 2]
        result["cold"] = {"ms_median": round(cms, 5), "tflops": round(flops / (cms * 1e-3) / 1e12, 3),
                          "achieved_GBps": round(nbytes / (cms * 1e-3) / 1e9, 1), "launches": len(times),
                          "note": "L2 and Infinity Cache flushed before each launch"}
    if gc is not None:
        gc["value_over_gemm"] = round(tflops / gc["tflops"], 4) if not decode else None
        gc["probe"]["value_over_probe"] = round(tflops / gc["probe"]["tflops"], 4) if not decode else None
        result["mfma_ceiling"] = gc
    if not args.no_train_step:
        tw = {x.name: x for x in wl.ALL}[args.train_workload]
        ts = train_step_timing(fa, wl, steps=20, warmup=5, w=tw)
        ap = atomic_probe()
        ap["bwd_atomic_bound_ms"] = round(ts["bwd_atomic_adds"] / ap["adds_per_s"] * 1e3, 4)
        ts["atomic_probe"] = ap
        result["train_step"] = ts
        if w.window is not None:
            result["train_step_window"] = train_step_timing(fa, wl, steps=20, warmup=5,
                                                            window=(1023, 0))
    if cpu_res is not None:
        result["cpu_baseline"] = cpu_res
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
