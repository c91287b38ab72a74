"""Seeded synthetic inputs shared by the tests, ``bench.py`` and ``smoke()``.

This module holds only shapes and random draws -- none of the attention
arithmetic -- so that both the HIP path and the fp64 oracle can be fed the
identical tensors without sharing any method code.

Recipe: a CPU ``torch.Generator`` seeded per case draws Q, K, V (then dO for
backward) in that order with ``randn`` in float32, iid N(0, 1).  For bf16
cases the float32 draw is cast with round-to-nearest-even (torch's cast).
Layout is [B, H, N, d], contiguous, d innermost.  The scale is 1/sqrt(d).
Inputs too large to draw on the host (``make_inputs_device``) follow the same
recipe with a seeded generator on the device instead, a different stream of
numbers from the same distribution; the oracle then reads back the heads it
checks.
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


@dataclass(frozen=True)
class VarlenWorkload:
    """A packed variable-length batch: ``n_seq`` sequences whose lengths are
    drawn log-uniformly in [lo, hi] (seeded), every head's tokens packed
    head-major [H, total, d]; queries and keys have the same lengths."""
    name: str
    n_seq: int
    lo: int
    hi: int
    H: int
    d: int
    dtype: str
    causal: bool
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def lengths(self):
        return varlen_lengths(self.n_seq, self.lo, self.hi, self.seed)

    def describe(self) -> str:
        L = self.lengths()
        mode = "causal" if self.causal else "non-causal"
        return (f"{self.n_seq} sequences of {min(L)}..{max(L)} tokens (total {sum(L)}) H={self.H} "
                f"d={self.d} {self.dtype} {mode}, packed")


# A packed batch of 32 sequences of 64..8192 tokens (log-uniform mix, as in
# a batch of documents of very different lengths), causal, at the
# Llama-shaped head count and head dimension.
VARLEN_CAUSAL = VarlenWorkload("varlen_causal_bf16", 32, 64, 8192, 32, 128, "bf16", True, seed=1008)


def varlen_lengths(n: int, lo: int, hi: int, seed: int):
    """``n`` sequence lengths in [lo, hi], log-uniform, from a seeded CPU
    generator (the same draw on every machine)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    u = torch.rand(n, generator=g, dtype=torch.float64)
    L = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return [int(x) for x in torch.clamp(torch.round(L), lo, hi).tolist()]


def make_varlen_inputs(lens_q, lens_k, H: int, d: int, dtype: str, seed: int,
                       with_do: bool = False, pad_q: int = 0, pad_k: int = 0):
    """Seeded packed tensors q [H, Tq, d], k, v [H, Tk, d] (and do [H, Tq, d])
    plus int32 CPU offsets cu_q, cu_k; ``pad_q``/``pad_k`` rows past the last
    sequence are drawn too.  Same recipe as ``make_inputs``."""
    cu_q = torch.tensor([0] + list(torch.cumsum(torch.tensor(lens_q, dtype=torch.int64), 0).tolist()),
                        dtype=torch.int32)
    cu_k = torch.tensor([0] + list(torch.cumsum(torch.tensor(lens_k, dtype=torch.int64), 0).tolist()),
                        dtype=torch.int32)
    Tq, Tk = int(cu_q[-1]) + pad_q, int(cu_k[-1]) + pad_k
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(H, Tq, d, generator=g, dtype=torch.float32)
    k = torch.randn(H, Tk, d, generator=g, dtype=torch.float32)
    v = torch.randn(H, Tk, d, generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_do:
        out.append(torch.randn(H, Tq, d, generator=g, dtype=torch.float32))
    td = torch_dtype(dtype)
    return [t.to(td).contiguous() for t in out] + [cu_q, cu_k]


def varlen_workload_inputs(w: VarlenWorkload):
    L = w.lengths()
    return make_varlen_inputs(L, L, w.H, w.d, w.dtype, w.seed)


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


def make_inputs_device(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int,
                       device, with_do: bool = False, chunk_heads: int = 256):
    """Seeded device tensors (q, k, v[, do]): a device generator draws
    float32 N(0, 1) values a few heads at a time, cast to ``dtype`` (RNE), so
    no full-size float32 copy is ever held."""
    g = torch.Generator(device=device).manual_seed(seed)
    td = torch_dtype(dtype)
    shapes = [(Nq, d), (Nk, d), (Nk, d)] + ([(Nq, d)] if with_do else [])
    out = []
    for (n, dd) in shapes:
        t = torch.empty(B * H, n, dd, dtype=td, device=device)
        for h0 in range(0, B * H, chunk_heads):
            h1 = min(B * H, h0 + chunk_heads)
            t[h0:h1] = torch.randn(h1 - h0, n, dd, generator=g, dtype=torch.float32, device=device).to(td)
        out.append(t.view(B, H, n, dd))
    return out


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
