"""Host-side logic on the CPU: the synthetic input recipes (shapes, seeding,
drafts drawn from the stated laws, tree layouts) and the benchmark's
accounting of the rows a tree walk reads."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from workload import WORKLOADS, make_inputs, make_tree_inputs, ragged_lengths, tree_parents

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_tree_parents_are_breadth_first_and_topological():
    par = tree_parents((4, 2, 1))
    assert par.size == 4 + 8 + 8
    assert list(par[:4]) == [-1] * 4
    assert list(par[4:12]) == [0, 0, 1, 1, 2, 2, 3, 3]
    assert list(par[12:]) == list(range(4, 12))
    assert all(-1 <= p < i for i, p in enumerate(par))
    assert tree_parents(()).size == 0
    assert list(tree_parents((1, 1, 1))) == [-1, 0, 1]


def test_inputs_are_seeded_and_shaped():
    w = WORKLOADS["C2"].sized(B=3, V=513)
    a = make_inputs(w, seed=4)
    b = make_inputs(w, seed=4)
    c = make_inputs(w, seed=5)
    assert a["target"].shape == (3, w.K + 1, 513) and a["draft"].shape == (3, w.K, 513)
    assert a["target"].dtype == torch.bfloat16 and a["tokens"].dtype == torch.int32
    for k in ("target", "draft", "tokens", "temperature"):
        assert torch.equal(a[k], b[k])
    assert not torch.equal(a["target"], c["target"])
    lens = ragged_lengths(w, 4, "cpu")
    assert lens.shape == (3,) and int(lens.min()) >= 0 and int(lens.max()) <= w.K


def test_tree_inputs_draw_children_from_their_context():
    """Greedy sequences pick the draft argmax of the parent's context row;
    every token is in range; rows have the stated shapes."""
    w = WORKLOADS["C3"].sized(B=4, V=301)
    shape = (3, 2)
    inp = make_tree_inputs(w, shape, seed=2)
    N = 3 + 6
    assert inp["target"].shape == (4, N + 1, 301) and inp["draft"].shape == (4, N, 301)
    assert torch.equal(inp["parent"][0], torch.from_numpy(tree_parents(shape)))
    am = torch.argmax(inp["draft"].float(), dim=2)
    ctx = (inp["parent"] + 1).long()
    assert torch.equal(inp["tokens"].long(), torch.gather(am, 1, ctx))
    w2 = WORKLOADS["C4"].sized(B=4, V=301)
    t2 = make_tree_inputs(w2, shape, seed=2)["tokens"]
    assert int(t2.min()) >= 0 and int(t2.max()) < 301


def test_tree_rows_read_counts_the_walks_passes():
    """At each visited context: one pass over its target row (and draft row
    if it has children), two rows per rejected child, and a target-row pass
    for a bonus drawn where no child was rejected."""
    import bench
    par = tree_parents((4, 2, 1))
    none = np.full(20, -1)
    # all four root children rejected: stats (2) + 4 rejections (8)
    assert bench.tree_rows_read(par, none, 0, False) == 10
    # node 1 accepted after one rejection (2 + 2), node 6 at once (2), node 14 at
    # once (2), then a leaf: its target row twice (statistics, bonus masses)
    path = np.array([1, 6, 14] + [-1] * 17)
    assert bench.tree_rows_read(par, path, 3, False) == 10
    # node 0 accepted at once (2), then both its children rejected (2 + 4)
    assert bench.tree_rows_read(par, np.array([0] + [-1] * 19), 1, False) == 8
    # greedy: one target row per visited context
    assert bench.tree_rows_read(par, path, 3, True) == 4
    assert bench.tree_rows_read(np.zeros(0, dtype=np.int32), np.zeros(0), 0, False) == 2
