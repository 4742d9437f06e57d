"""CPU oracle (test infrastructure only; see zha_oracle's header)."""

from .zha_oracle import (  # noqa: F401
    N_REF,
    NEAR_TIE_REL,
    sigma,
    pool,
    build_tree_unit,
    build_tree,
    node_scores,
    select_top_p,
    expand,
    search,
    attention_over,
    attend_head,
    attend,
    HeadResult,
    LevelDecision,
)
