"""Split-KV block-sparse draft attention for AMD Instinct MI355X (gfx950).

The compute path lives in libsplitkv.so (HIP kernels behind the C ABI of
include/splitkv.h); ``binding`` marshals arguments to it and ``path`` drives
the plan -> partial forward -> merge -> backward sequence on one GPU.
Importing the package fails if the library has not been built.
"""
from . import binding  # noqa: F401  (raises ImportError when libsplitkv.so is missing)
from .binding import (  # noqa: F401
    Problem, SkvError, lpt_plan, lse_merge, lse_merge_all, skv_coarsen_fwd_items, skv_drop_zero_cost,
    skv_gather_items, skv_plan_fwd_runs, skv_static_plan, sparse_attn_bwd, sparse_attn_own_fwd, sparse_attn_partial_fwd,
)
from .path import SplitKVAttention, unmasked_pairs  # noqa: F401
