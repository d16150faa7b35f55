"""fp64 CPU oracle for tree-verification attention.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg to check and time against. The GPU library and
its binding never import it.
"""

from .hta_oracle import (  # noqa: F401
    BadTree,
    attend_rows,
    check_parent,
    default_scale,
    lse_merge,
    tree_mask_bits,
    tree_visible_nodes,
    verify_attn,
)
from .accept_oracle import accept, accept_path, commit, target_tokens  # noqa: F401,E402
from .draft_oracle import cross_attn, window_append, window_attn, window_visible  # noqa: F401,E402
from .tree_oracle import build_tree, build_trees, most_recent_match, ranked_tokens  # noqa: F401,E402
