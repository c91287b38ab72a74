"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every symbol ``include/fa.h`` declares, and
reject bad arguments with the documented status codes before making any HIP
call.  Every call below is built so validation fails (or the call is an empty
no-op), so no kernel is ever launched here.
"""

import os
import re

import pytest

import exact_attention_20_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = 0x100000        # a 16-byte-aligned, never-dereferenced address
FAKE_MIS = 0x100008    # 8-byte aligned only


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == {"fa_fwd", "fa_fwd_soft_exp2", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "fa_bwd",
                         "fa_bwd_workspace_bytes", "fa_bwd_noalloc", "fa_fwd_window", "fa_bwd_window",
                         "fa_fwd_varlen", "fa_bwd_varlen", "fa_bwd_varlen_workspace_bytes",
                         "fa_strerror"}
    for s in syms:
        assert hasattr(lib, s), s


def test_strerror_covers_codes():
    for code in range(0, -12, -1):
        msg = fa.fa_strerror(code)
        assert msg and msg != "unknown status", code
    assert fa.fa_strerror(-99) == "unknown status"


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=16, Nk=16, d=64,
             scale=0.125, causal=0, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd(**a)


def test_fwd_validation_codes():
    assert fwd(B=-1) == -2
    assert fwd(Nq=-3) == -2
    assert fwd(Nk=(1 << 23) + 1) == -2
    assert fwd(d=96) == -3
    assert fwd(d=256) == -3
    assert fwd(dtype=7) == -4
    assert fwd(scale=0.0) == -8
    assert fwd(scale=float("nan")) == -8
    assert fwd(scale=-1.0) == -8
    assert fwd(scale=float("inf")) == -8
    assert fwd(q=0) == -1
    assert fwd(o=0) == -1
    assert fwd(v=0) == -1
    assert fwd(q=FAKE_MIS) == -5
    assert fwd(k=FAKE_MIS) == -5
    assert fwd(lse=FAKE + 2) == -5


def test_fwd_empty_is_a_noop():
    # nothing to compute: returns before any HIP call, pointers may be NULL
    assert fwd(B=0, q=0, k=0, v=0, o=0, lse=0) == 0
    assert fwd(H=0, q=0, k=0, v=0, o=0, lse=0) == 0
    assert fwd(Nq=0, q=0, k=0, v=0, o=0, lse=0) == 0


def test_workspace_bytes():
    rows = 4 * 16 * 4096
    n = fa.fa_bwd_workspace_bytes(4, 16, 4096, 4096, 64, fa.FA_BF16, 1)
    assert n == 2 * rows * 4                   # two float32 row vectors, already 256-aligned
    assert n % 256 == 0
    # the atomic mode adds the float32 dQ buffer
    assert fa.fa_bwd_workspace_bytes(4, 16, 4096, 4096, 64, fa.FA_BF16, 0) == n + rows * 64 * 4
    assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 64, fa.FA_BF16, 1) == 2 * 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 64, fa.FA_BF16, 0) == 2 * 256 + 768
    assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 128, fa.FA_BF16, 7) == 2 * 256
    for det in (0, 1):
        assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 96, fa.FA_BF16, det) == 0
        # fp32 runs the deterministic kernels in either mode: the two row vectors only
        assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 64, fa.FA_F32, det) == 2 * 256
        assert fa.fa_bwd_workspace_bytes(2, 3, 300, 5, 128, fa.FA_F32, det) == 2 * 1800 * 4 + 2 * 224
        assert fa.fa_bwd_workspace_bytes(1, 1, 3, 5, 64, 7, det) == 0
        assert fa.fa_bwd_workspace_bytes(-1, 1, 3, 5, 64, fa.FA_BF16, det) == 0
        assert fa.fa_bwd_workspace_bytes(1, 1, 0, 5, 64, fa.FA_BF16, det) == 0


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=1, H=2, Nq=32, Nk=32, d=64, scale=0.125, causal=1, dtype=fa.FA_BF16,
             deterministic=0, workspace=FAKE, workspace_bytes=1 << 20, stream=0)
    a.update(kw)
    return fa.fa_bwd(**a)


def test_bwd_validation_codes():
    for det in (0, 1):
        assert bwd(deterministic=det, dtype=7) == -4
        assert bwd(deterministic=det, d=32) == -3
        assert bwd(deterministic=det, Nk=-1) == -2
        assert bwd(deterministic=det, scale=0.0) == -8
        assert bwd(deterministic=det, dO=0) == -1
        assert bwd(deterministic=det, dk=0) == -1
        assert bwd(deterministic=det, lse=0) == -1
        assert bwd(deterministic=det, dq=FAKE_MIS) == -5
        assert bwd(deterministic=det, workspace=0) == -6
        need = fa.fa_bwd_workspace_bytes(1, 2, 32, 32, 64, fa.FA_BF16, det)
        assert bwd(deterministic=det, workspace_bytes=need - 1) == -6
        assert bwd(deterministic=det, B=0) == 0
    # the atomic mode's workspace does not fit a deterministic-sized buffer
    small = fa.fa_bwd_workspace_bytes(1, 2, 32, 32, 64, fa.FA_BF16, 1)
    assert bwd(deterministic=0, workspace_bytes=small) == -6
    # fp32 takes the same checks (every call here stops before a launch)
    for det in (0, 1):
        f32 = dict(deterministic=det, dtype=fa.FA_F32)
        need = fa.fa_bwd_workspace_bytes(1, 2, 32, 32, 64, fa.FA_F32, det)
        assert need == small
        assert bwd(workspace_bytes=need - 1, **f32) == -6
        assert bwd(workspace=0, **f32) == -6
        assert bwd(d=96, **f32) == -3
        assert bwd(dv=0, **f32) == -1
        assert bwd(q=FAKE_MIS, **f32) == -5
        assert bwd(scale=float("inf"), **f32) == -8
        assert bwd(B=0, **f32) == 0
    # the key-side grid (64-key tiles) must fit in 32 bits, whatever Nq is
    assert bwd(B=1 << 14, H=1 << 14, Nq=32, Nk=1000) == -2
    assert bwd(B=1 << 14, H=1 << 14, Nq=32, Nk=1000, dtype=fa.FA_F32) == -2


def bwd_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=1, H=2, Nq=32, Nk=32, d=64, scale=0.125, causal=1, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_bwd_noalloc(**a)


def test_bwd_noalloc_validation_codes():
    # fa_bwd's own checks, before any HIP call
    assert bwd_noalloc(dtype=7) == -4
    assert bwd_noalloc(d=32) == -3
    assert bwd_noalloc(Nk=-1) == -2
    assert bwd_noalloc(scale=float("nan")) == -8
    assert bwd_noalloc(B=0, q=0, k=0, v=0, o=0, lse=0, dO=0, dq=0, dk=0, dv=0) == 0
    # the static array holds two fp32 vectors of up to 2^20 query rows
    limit = (8 << 20) // 8
    assert fa.fa_bwd_workspace_bytes(8, 32, 4096, 4096, 128, fa.FA_BF16, 1) == 8 << 20
    assert 8 * 32 * 4096 == limit
    assert bwd_noalloc(B=1, H=1, Nq=limit + 1, Nk=64) == -10
    assert bwd_noalloc(B=3, H=32, Nq=limit // 96 + 64, Nk=64) == -10
    assert "static buffer" in fa.fa_strerror(-10)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "_PKG", str(tmp_path))
    with pytest.raises(RuntimeError, match="no fallback"):
        fa.load_library()


def split(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Nq=1, Nk=1000, d=128,
             scale=0.088, causal=1, dtype=fa.FA_BF16, n_splits=4, workspace=FAKE,
             workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return fa.fa_fwd_splitkv(**a)


def test_splitkv_workspace_plan():
    # 1000 keys = 16 tiles of 64; 4 runs of 4 tiles; 2 heads x 1 row
    n = fa.fa_fwd_splitkv_workspace_bytes(1, 2, 1, 1000, 128, fa.FA_BF16, 4)
    assert n == 4096 + 256            # O parts 4*2*1*128*4 B, LSE parts 32 B -> 256
    # 5 requested runs of 16 tiles -> 4 tiles per run -> 4 effective runs
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 1, 1000, 128, fa.FA_BF16, 5) == n
    # more runs than tiles clamp to one tile per run
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 1, 1, 100, 64, fa.FA_BF16, 50) == 512 + 256
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 1, 1, 100, 64, fa.FA_F32, 2) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 1, 1, 100, 64, fa.FA_BF16, -1) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 1, 0, 100, 64, fa.FA_BF16, 2) == 0
    # automatic choice: 8 heads x 1 row, 8192 keys = 128 tiles -> capped at 32 runs of 4
    auto = fa.fa_fwd_splitkv_workspace_bytes(1, 8, 1, 8192, 64, fa.FA_BF16, 0)
    assert auto == 32 * 8 * 64 * 4 + 1024


def test_splitkv_validation_codes():
    assert split(dtype=fa.FA_F32) == -4
    assert split(n_splits=-1) == -2
    assert split(n_splits=1025) == -2
    assert split(d=96) == -3
    assert split(scale=float("nan")) == -8
    assert split(q=0) == -1
    assert split(o=FAKE_MIS) == -5
    assert split(workspace=0) == -6
    need = fa.fa_fwd_splitkv_workspace_bytes(1, 2, 1, 1000, 128, fa.FA_BF16, 4)
    assert split(workspace_bytes=need - 1) == -6
    assert split(workspace=FAKE_MIS) == -5
    assert split(B=0) == 0
    assert split(Nq=0) == 0


def fwdw(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=16, Nk=16, d=64,
             scale=0.125, window_left=8, window_right=0, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_window(**a)


def bwdw(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=1, H=2, Nq=32, Nk=32, d=64, scale=0.125, window_left=8, window_right=4,
             dtype=fa.FA_BF16, deterministic=0, workspace=FAKE, workspace_bytes=1 << 20, stream=0)
    a.update(kw)
    return fa.fa_bwd_window(**a)


def test_window_validation_codes():
    # a reach below -1 is rejected before anything else is looked at
    assert fwdw(window_left=-2) == -9
    assert fwdw(window_right=-5, q=0) == -9
    assert bwdw(window_left=-2) == -9
    assert bwdw(window_right=-2, dtype=fa.FA_F32) == -9
    # the shared checks still apply to every window, bounded or not
    for wl, wr in ((8, 0), (-1, 0), (-1, -1), (0, 0), (3, -1), (1 << 30, 1 << 30)):
        assert fwdw(window_left=wl, window_right=wr, d=96) == -3
        assert fwdw(window_left=wl, window_right=wr, q=0) == -1
        assert fwdw(window_left=wl, window_right=wr, k=FAKE_MIS) == -5
        assert fwdw(window_left=wl, window_right=wr, scale=0.0) == -8
        assert fwdw(window_left=wl, window_right=wr, B=0, q=0, k=0, v=0, o=0, lse=0) == 0
        assert bwdw(window_left=wl, window_right=wr, dtype=7) == -4
        assert bwdw(window_left=wl, window_right=wr, dtype=fa.FA_F32, workspace=0) == -6
        assert bwdw(window_left=wl, window_right=wr, workspace=0) == -6
        assert bwdw(window_left=wl, window_right=wr, dk=0) == -1
        assert bwdw(window_left=wl, window_right=wr, B=0) == 0


def fwdv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu_seqlens_q=FAKE, cu_seqlens_k=FAKE,
             B=3, H=2, total_q=100, total_k=120, max_seqlen_q=50, max_seqlen_k=60, d=64,
             scale=0.125, window_left=-1, window_right=0, dtype=fa.FA_BF16, stream=0)
    a.update(kw)
    return fa.fa_fwd_varlen(**a)


def bwdv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, B=3, H=2, total_q=100, total_k=120,
             max_seqlen_q=50, max_seqlen_k=60, d=128, scale=0.125, window_left=-1,
             window_right=-1, dtype=fa.FA_BF16, deterministic=1, workspace=FAKE,
             workspace_bytes=1 << 20, stream=0)
    a.update(kw)
    return fa.fa_bwd_varlen(**a)


def test_varlen_validation_codes():
    for call in (fwdv, bwdv):
        assert call(window_left=-2) == -9
        assert call(B=-1) == -2
        assert call(total_q=-1) == -2
        assert call(max_seqlen_k=-1) == -2
        assert call(max_seqlen_q=(1 << 23) + 1) == -2
        assert call(d=96) == -3
        assert call(dtype=fa.FA_F32) == -4
        assert call(dtype=5) == -4
        assert call(scale=0.0) == -8
        assert call(cu_seqlens_q=0) == -1
        assert call(cu_seqlens_k=0) == -1
        assert call(cu_seqlens_k=FAKE + 2) == -5
        assert call(q=0) == -1
        assert call(v=FAKE_MIS) == -5
        # nothing to compute: no pointer is looked at
        assert call(B=0, q=0, k=0, v=0, o=0, lse=0, cu_seqlens_q=0, cu_seqlens_k=0) == 0
        assert call(H=0, q=0, cu_seqlens_q=0) == 0
    assert fwdv(total_q=0, q=0, o=0) == 0
    assert fwdv(lse=FAKE + 2) == -5
    assert bwdv(lse=0) == -1
    assert bwdv(dk=FAKE_MIS) == -5
    assert bwdv(workspace=0) == -6
    need = fa.fa_bwd_varlen_workspace_bytes(2, 100, 128, fa.FA_BF16, 1)
    assert need == 2 * 1024                 # 2 heads x 100 rows x 4 B -> 800 -> 1024, twice
    assert bwdv(workspace_bytes=need - 1) == -6
    atomic = fa.fa_bwd_varlen_workspace_bytes(2, 100, 128, fa.FA_BF16, 0)
    assert atomic == need + 200 * 128 * 4
    assert bwdv(deterministic=0, workspace_bytes=atomic - 1) == -6
    assert bwdv(total_q=0, total_k=0, q=0, k=0) == 0


def test_varlen_workspace_bytes():
    ws = fa.fa_bwd_varlen_workspace_bytes
    assert ws(16, 4096 * 4, 64, fa.FA_BF16, 1) == 2 * 16 * 4096 * 4 * 4
    assert ws(16, 4096 * 4, 64, fa.FA_BF16, 0) == 2 * 16 * 4096 * 4 * 4 + 16 * 4096 * 4 * 64 * 4
    assert ws(1, 3, 64, fa.FA_BF16, 1) == 512
    assert ws(1, 3, 64, fa.FA_BF16, 0) == 512 + 768
    for det in (0, 1):
        assert ws(1, 3, 64, fa.FA_F32, det) == 0
        assert ws(1, 3, 80, fa.FA_BF16, det) == 0
        assert ws(-1, 3, 64, fa.FA_BF16, det) == 0
    # more rows per head than FA_MAX_SEQ are fine when packed
    assert ws(2, 1 << 24, 64, fa.FA_BF16, 1) == 2 * 2 * (1 << 24) * 4


_REMARKS = """\
src.hip:87:1: remark: Function Name: _ZN2fa15fwd_bf16_kernelILi64ELi1ELb0ELb0EEEvNS_9FwdParamsE [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     TotalSGPRs: 106 [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
src.hip:87:1: remark:     LDS Size [bytes/block]: 32784 [-Rpass-analysis=kernel-resource-usage]
some unrelated warning line
src.hip:624:1: remark: Function Name: _ZN2fa13bwd_dq_kernelILi128ELi1ELb0EEEvNS_9BwdParamsE [-Rpass-analysis=kernel-resource-usage]
src.hip:624:1: remark:     VGPRs: 252 [-Rpass-analysis=kernel-resource-usage]
src.hip:624:1: remark:     VGPRs Spill: 4 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_usage_remark_parser():
    """The compiler's per-kernel resource remarks become one row per kernel."""
    from exact_attention_20_amd import build

    rows = build.parse_remarks(_REMARKS)
    assert [r["_name"] for r in rows] == [
        "_ZN2fa15fwd_bf16_kernelILi64ELi1ELb0ELb0EEEvNS_9FwdParamsE",
        "_ZN2fa13bwd_dq_kernelILi128ELi1ELb0EEEvNS_9BwdParamsE",
    ]
    assert rows[0]["VGPRs"] == "128" and rows[0]["LDS Size [bytes/block]"] == "32784"
    assert rows[0]["Occupancy [waves/SIMD]"] == "4" and rows[0]["ScratchSize [bytes/lane]"] == "0"
    assert rows[1]["VGPRs Spill"] == "4" and "AGPRs" not in rows[1]
    table = build.resource_table([("a.hip", "void fa::k<64, 1>(fa::FwdParams)", rows[0])])
    assert "| a.hip | `k<64, 1>` | 128 | 0 | 0 |" in table


def fwd_soft(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=16, Nk=16, d=64,
             scale=0.125, causal=0, dtype=fa.FA_BF16, period=4, stream=0)
    a.update(kw)
    return fa.fa_fwd_soft_exp2(**a)


def test_soft_exp2_validation_codes():
    # every call here stops before a launch
    for period in (0, 1, 3, 5, 16, -2):
        assert fwd_soft(period=period) == -11
    assert fwd_soft(dtype=fa.FA_F32) == -4
    assert fwd_soft(dtype=7) == -4
    assert fwd_soft(d=96) == -3
    assert fwd_soft(Nq=-1) == -2
    assert fwd_soft(scale=0.0) == -8
    assert fwd_soft(q=0) == -1
    assert fwd_soft(k=FAKE_MIS) == -5
    assert fwd_soft(B=0, q=0, k=0, v=0, o=0, lse=0) == 0
    assert "2, 4 or 8" in fa.fa_strerror(-11)
