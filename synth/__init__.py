"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench."""

from .workloads import (  # noqa: F401
    Workload,
    tiny_tree,
    grpo_group,
    agentic_trie,
    independent,
    long_history,
    standard,
    round_bf16,
    feature_tables,
    from_sequences,
    curriculum_batch,
    shared_history,
    sequence_packing_forest,
    gdn_tables,
)
