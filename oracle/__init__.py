"""fp64 CPU oracle for exact (softmax) attention -- TEST INFRASTRUCTURE ONLY.

This package is the independent reference that the HIP kernels are checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path (the C-ABI library and its
Python binding in ``exact_attention_20_amd``) never imports, calls or links
anything here, and nothing here imports the product path.  The two share no
code; only the seeded input generators in ``workloads`` feed both.

Sources (pages, cited by title and section; see ``attention.py``):
  [P1] "FlashAttention 详解：从 Online Softmax 到单遍融合"
  [P2] "01 · IO-awareness、online softmax 与 tiling"
  [P3] "20. FlashAttention Sim | FlashAttention 模拟"
  [P4] "让注意力计算留在片上：分块 Softmax 的计算与访存分析"
  [P5] "FlashAttention 1～4 全解汇总"

Every function is pinned by a ``-m "not gpu"`` test (tests/test_oracle.py)
against values the pages print, closed forms, invariants, finite differences
or a library routine.  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    visible_mask,
    window_bounds,
    attention_forward,
    attention_forward_rows,
    attention_backward,
    varlen_forward,
    varlen_backward,
    online_rescale,
    tiled_forward,
    tiled_forward_renormalised,
    softmax,
    attention_flops,
)
