"""CPU float64 oracle for Split-KV block-sparse draft attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product path (the HIP library and its Python binding) never
imports it and shares no code, headers, tables or helpers with it.

Sources followed (pages as published, cited by title and section):
  [P1] "Split-KV: Breaking the Context Parallelism Bottleneck in Diffusion
       Drafter Training" (kongchang.com, English article) — lede, "The
       Query-Context Asymmetry", "Split-KV's Core Mechanism", "LPT Scheduling".
  [P3] arXiv:2611.05926 listing "Split-KV: Efficient Context Parallelism for
       Training Diffusion Drafters" — Abstract.

Readings of points the pages leave open are stated in each function's
docstring.

Parity status: every function here is pinned by tests under ``tests/`` marked
``not gpu`` (brute force, closed forms, library special cases, finite
differences, the Graham bound); none is "parity unpinned".
"""
from .attention import (  # noqa: F401
    block_ends, visible_mask, attention, chunk_partials, lse_merge, attention_bwd,
    attention_workload, partials_workload, bwd_workload,
)
from .own_block import (  # noqa: F401
    context_ends, attention_own, own_partial, attention_own_bwd, attention_own_workload, bwd_own_workload,
)
from .plan import (  # noqa: F401
    item_table, lpt, static_assign, csr_from_assign, loads_from_assign, imbalance,
    brute_force_makespan, graham_bound, coarsen_runs,
)
