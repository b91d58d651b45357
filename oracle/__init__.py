"""Plain float64 CPU oracle for draft-tree verification.

TEST INFRASTRUCTURE ONLY. The oracle states, slowly and directly, what the
verification step computes, so that the HIP library can be checked against
it. Only ``tests/``, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it; the library never calls it and
never falls back to it. It shares no code with the HIP path.

Every function is pinned by tests that do not reuse its own formulas (worked
examples from the pages, closed forms, library routines, brute force); nothing
here is "parity unpinned".
"""
from .tv_oracle import (  # noqa: F401
    ERR_BAD_TREE,
    ERR_CAPACITY,
    ERR_OK,
    accept,
    ancestor_words,
    ancestors_or_self,
    attention_row,
    build_tree,
    PAGE,
    commit,
    eagle2_tree,
    gather_pages,
    scatter_pages,
    next_token_distribution,
    inverse_cdf,
    rope,
    softmax64,
    speculative_sample,
    tree_attention,
    tree_depth,
    tree_is_valid,
    tree_mask,
    typical_accept,
    verify_step,
)
