"""Tree-verification attention for speculative decoding on MI355X (gfx950).

LongSpec's Hybrid Tree Attention: every draft-tree node attends without a mask to the committed
KV prefix and, under an ancestor-only mask, to the other tree nodes; the two partial results are
merged exactly through their log-sum-exps. The computation lives in hand-written HIP kernels
behind the C ABI of ``include/treeattn.h``; this package is the thin Python binding (torch is
used for device memory and streams only) plus the seeded synthetic-input generators.
"""
from ._lib import (  # noqa: F401
    TA_BF16, TA_DEV_BAD_COMMIT, TA_DEV_BAD_LEN, TA_DEV_BAD_PAGE, TA_DEV_BAD_PARENT,
    TA_DEV_BAD_TOKEN, TA_F32, TA_MAX_TREE, TreeAttnError, combine, forward, gdn_commit,
    gdn_verify, greedy_accept,
    greedy_accept_workspace_size, kv_commit, load, make_problem, mask_build, merge, num_splits,
    partials, prefix, spec_sample, spec_sample_workspace_size, status_string, tree,
    workspace_lse_offset, workspace_size,
)

__all__ = ["forward", "partials", "combine", "prefix", "tree", "merge", "mask_build",
           "make_problem", "workspace_size", "workspace_lse_offset", "num_splits", "load",
           "status_string", "TreeAttnError", "greedy_accept", "greedy_accept_workspace_size",
           "kv_commit", "spec_sample", "spec_sample_workspace_size", "gdn_verify",
           "gdn_commit"]
