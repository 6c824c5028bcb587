"""Seeded synthetic inputs for the verify step (shared by tests and benchmark).

Holds no verification arithmetic: only the recipe that fabricates logits and
drafted tokens of the shapes and distributions of the five named workloads.
"""
from .gen import (WORKLOADS, Workload, make_inputs, make_tree_inputs, ragged_lengths,  # noqa: F401
                  ragged_rows, to_numpy_inputs, tree_parents)
