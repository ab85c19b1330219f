"""Batched verify step of speculative decoding on AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (include/specdec.h);
this package holds the thin ctypes binding over it, the in-tree build and the
seeded synthetic workloads used by the tests and the benchmark.
"""
from ._lib import (SpecdecError, Workspace, acceptance_counts, choose_k, load,  # noqa: F401
                   ngram_propose, sampling_floors, softmax_stats, tree_mask, tree_verify_greedy, verify,
                   verify_greedy, version, workspace_errors)

__all__ = ["SpecdecError", "Workspace", "acceptance_counts", "choose_k", "load", "ngram_propose",
           "sampling_floors", "softmax_stats", "tree_mask", "tree_verify_greedy", "verify", "verify_greedy",
           "version", "workspace_errors"]
