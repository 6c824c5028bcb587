"""Seeded synthetic inputs for the verify step (shared by tests and benchmark).

Holds no verification arithmetic: only the recipe that fabricates logits and
drafted tokens of the shapes and distributions of the five named workloads.
"""
from .gen import (WORKLOADS, Workload, make_inputs, ragged_lengths, ragged_rows,  # noqa: F401
                  to_numpy_inputs)
