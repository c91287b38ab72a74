"""Seeded synthetic inputs shared by the tests, ``bench.py`` and ``smoke()``.

This module holds only shapes and random draws -- none of the attention
arithmetic -- so that both the HIP path and the fp64 oracle can be fed the
identical tensors without sharing any method code.

Recipe: a CPU ``torch.Generator`` seeded per case draws Q, K, V (then dO for
backward) in that order with ``randn`` in float32, iid N(0, 1).  For bf16
cases the float32 draw is cast with round-to-nearest-even (torch's cast).
Layout is [B, H, N, d], contiguous, d innermost.  The scale is 1/sqrt(d).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str          # "fp32" | "bf16"
    causal: bool
    backward: bool = False
    seed: int = 0
    window: tuple | None = None   # local window (wl, wr), None sides unbounded; replaces causal

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def describe(self) -> str:
        mode = "causal" if self.causal else "non-causal"
        if self.window is not None:
            mode = f"window {self.window}"
        bwd = ", fwd+bwd" if self.backward else ""
        return (f"B={self.B} H={self.H} Nq={self.Nq} Nk={self.Nk} d={self.d} "
                f"{self.dtype} {mode}{bwd}")


# The five workloads the method is measured on (sizes and modes as stated for
# the headline measurement).  Seeds are 1000 + index.
SINGLE_HEAD = Workload("single_head_fp32", 1, 1, 256, 256, 64, "fp32", False, seed=1001)
GPT2_SMALL = Workload("gpt2_small_bf16", 8, 12, 1024, 1024, 64, "bf16", False, seed=1002)
LLAMA_CAUSAL = Workload("llama_causal_bf16", 4, 32, 4096, 4096, 128, "bf16", True, seed=1003)
LONG_CONTEXT = Workload("long_context_bf16", 1, 32, 32768, 32768, 128, "bf16", True, seed=1004)
TRAIN_STEP = Workload("train_step_bf16", 4, 16, 4096, 4096, 64, "bf16", True, backward=True, seed=1005)

# Decoding one new token of a single sequence against the long-context key
# length (split-KV path; unsplit, its 32 query tiles would leave the GPU idle):
# Nq = 1 with bottom-right causal alignment sees every key.
DECODE = Workload("decode_bf16", 1, 32, 1, 32768, 128, "bf16", True, seed=1006)

# Local attention over the long-context shape: every query sees itself and
# the 4095 keys before it (a sliding window of 4096 keys ending at the
# diagonal), so the work is 1/8 of the causal case's.
SLIDING_WINDOW = Workload("sliding_window_bf16", 1, 32, 32768, 32768, 128, "bf16", False,
                          seed=1007, window=(4095, 0))

ALL = [SINGLE_HEAD, GPT2_SMALL, LLAMA_CAUSAL, LONG_CONTEXT, TRAIN_STEP, DECODE, SLIDING_WINDOW]


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int,
                with_do: bool = False, dv: int | None = None):
    """Seeded CPU tensors (q, k, v[, do]) in the requested dtype."""
    dv = d if dv is None else dv
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, Nk, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, Nk, dv, generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_do:
        out.append(torch.randn(B, H, Nq, dv, generator=g, dtype=torch.float32))
    td = torch_dtype(dtype)
    return [t.to(td).contiguous() for t in out]


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, with_do=w.backward)


def sample_rows(N: int, count: int, seed: int):
    """``count`` distinct query indices in [0, N), seeded, always including
    the first and the last row; sorted."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    count = min(count, N)
    perm = torch.randperm(N, generator=g)[: count].tolist()
    rows = set(perm)
    rows.update({0, N - 1})
    rows = sorted(rows)
    while len(rows) > count:
        # drop interior rows until the budget holds (0 and N-1 stay)
        rows.pop(len(rows) // 2)
    return rows
