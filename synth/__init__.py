"""Seeded synthetic inputs for paged KV attention workloads.

This package is the only code that both the CPU oracle side and the HIP side
consume.  It produces *inputs* only:

* workload shapes (head counts, head dim, block size, layers, pool size),
* op programs: which pool calls happen in which order (allocate, fork,
  append, free, decode, tree-verify, prefill), referring to sequences by
  handle,
* bf16 sample tensors (fp32 N(0,1) draws rounded to nearest-even), keyed by
  the op that consumes them, never by a physical block,
* the block free-list order (identity or a seeded permutation),
* draft-tree parent pointers.

It holds none of the method's arithmetic: no refcount / copy-on-write rules,
no block-table logic, no softmax.  Each side runs a program with its own
implementation.
"""

from .bf16 import f32_to_bf16_bits
from .workloads import (
    Shape,
    Workload,
    STREAM_K,
    STREAM_V,
    STREAM_Q,
    STREAM_PERM,
    STREAM_TREE,
    named,
    NAMES,
    fork_workload,
    shared_prompt_workload,
    mcts_workload,
    verify_workload,
    prefill_workload,
    verify_commit_workload,
    draw_tree,
)

__all__ = [
    "f32_to_bf16_bits",
    "Shape",
    "Workload",
    "STREAM_K",
    "STREAM_V",
    "STREAM_Q",
    "STREAM_PERM",
    "STREAM_TREE",
    "named",
    "NAMES",
    "fork_workload",
    "shared_prompt_workload",
    "mcts_workload",
    "verify_workload",
    "prefill_workload",
    "verify_commit_workload",
    "draw_tree",
]
