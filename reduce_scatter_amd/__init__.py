"""reduce_scatter_amd -- n-rank all-reduce / reduce-scatter / all-gather on one
MI355X, with the n rank buffers resident in its HBM.

This package is a thin ctypes binding over ``libar.so`` (HIP kernels for
gfx950 plus the C ABI declared in ``include/ar.h`` and, for the M-to-N layout
reshard, ``include/ar_reshard.h``).  The functions keep the C
names and only marshal arguments: every step of the collective runs in the
library's kernels.  There is no CPU fallback; importing the package fails
loudly when the library has not been built (``python
reduce_scatter_amd/build.py``).
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    AR_MAX_RANKS,
    COLLS,
    DTYPES,
    OPS,
    SCHEDS,
    ArError,
    Plan,
    PointerTable,
    ar_all_gather,
    ar_allreduce,
    ar_allreduce_ex,
    ar_plan,
    ar_reduce_scatter,
    ar_reduce_scatter_ex,
    ar_status_string,
    ar_tree_parent,
    ar_dtree_parent,
    library_path,
    pointers,
    REPLICATE,
    ROUTES,
    Layout,
    ReshardPlan,
    ar_layout_shard,
    ar_reshard,
    ar_reshard_plan,
    local_shape,
)

__all__ = [
    "ar_allreduce",
    "ar_allreduce_ex",
    "ar_reduce_scatter_ex",
    "ar_reduce_scatter",
    "ar_all_gather",
    "ar_plan",
    "ar_tree_parent",
    "ar_dtree_parent",
    "ar_status_string",
    "ArError",
    "Plan",
    "DTYPES",
    "OPS",
    "SCHEDS",
    "COLLS",
    "AR_MAX_RANKS",
    "library_path",
    "pointers",
    "PointerTable",
    "REPLICATE",
    "ROUTES",
    "Layout",
    "ReshardPlan",
    "ar_layout_shard",
    "ar_reshard",
    "ar_reshard_plan",
    "local_shape",
]
