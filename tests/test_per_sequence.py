"""Per-sequence layout (host side): root-to-leaf paths of every workload's
tree shape, checked against the oracle's ancestor and child masks (a leaf is
a node with no child; its path is its ancestor set in index order)."""
import numpy as np
import pytest

import synth
from oracle import tree as o_tree
from tree_speculative_verification_attn_amd.per_sequence import leaf_paths


def _paths_from_masks(parent_row):
    anc, child, _, st = o_tree.build_mask(list(parent_row))
    assert st == 0
    out = []
    for i, p in enumerate(parent_row):
        if int(p) == -2 or child[i + 1]:
            continue
        out.append([j for j in range(len(parent_row)) if (anc[i] >> j) & 1])
    return out


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_leaf_paths_match_masks(cfg):
    w = synth.make_workload(cfg, B=3, L=8, H=1, V=64)
    for b in range(w.B):
        assert leaf_paths(w.parent[b]) == _paths_from_masks(w.parent[b])


def test_leaf_paths_padding_and_empty():
    assert leaf_paths([]) == []
    assert leaf_paths([-2, -2]) == []
    # padding in the middle; node 3 hangs off node 1
    assert leaf_paths([-1, 0, -2, 1, -1]) == [[0, 1, 3], [4]]
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 65))
        par = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
        assert leaf_paths(par) == _paths_from_masks(par)
