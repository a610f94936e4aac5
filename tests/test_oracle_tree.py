"""Pins for the oracle's tree masks (TreeMask rule, SpecInfer summary section
"Topology-Aware Causal Mask")."""
import numpy as np
import pytest

from oracle import tree
from oracle.status import ST_BAD_PARENT, ST_OK
from tests.golden.load import read_mask_fixture


def _rows_to_words(rows):
    return [sum(bit << j for j, bit in enumerate(r)) for _, r in rows]


@pytest.mark.parametrize("fixture", ["p3_tree_mask.txt", "fig3_tree.txt"])
def test_mask_matches_printed_or_figure_values(fixture):
    parent, rows = read_mask_fixture(fixture)
    anc, child, depth, st = tree.build_mask(parent)
    assert st == ST_OK
    assert anc == _rows_to_words(rows)


def test_p3_words_literal():
    # Row words of the printed 6x6 matrix, bit j = column j.
    anc, _, _, _ = tree.build_mask([-1, 0, 0, 1, 1, 2])
    assert anc == [0x1, 0x3, 0x5, 0xB, 0x13, 0x25]


def test_chain_is_lower_triangular():
    # A chain (width-1 tree) reduces TreeMask to the standard causal mask (Eq. 3).
    for n in (1, 2, 7, 64):
        anc, child, depth, st = tree.build_mask([-1] + list(range(n - 1)))
        assert st == ST_OK
        for i in range(n):
            assert anc[i] == (1 << (i + 1)) - 1
        assert depth == list(range(1, n + 1))


def test_star_is_diagonal():
    anc, child, depth, st = tree.build_mask([-1] * 64)
    assert anc == [1 << i for i in range(64)]
    assert child[0] == (1 << 64) - 1 and all(c == 0 for c in child[1:])


def _random_parent(rng, n):
    return [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]


def test_invariants_random_trees():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 65))
        par = _random_parent(rng, n)
        anc, child, depth, st = tree.build_mask(par)
        assert st == ST_OK
        for i in range(n):
            assert bin(anc[i]).count("1") == depth[i]
            assert (anc[i] >> i) & 1
            if par[i] >= 0:
                assert anc[i] & anc[par[i]] == anc[par[i]]
            # ancestor bits agree with walking the parent chain
            assert anc[i] == sum(1 << v for v in tree.path_to(par, i))
        # every node is the child of exactly one entry
        seen = 0
        for c in child:
            assert seen & c == 0
            seen |= c
        assert seen == (1 << n) - 1
        for i in range(n):
            assert (child[par[i] + 1] >> i) & 1


@pytest.mark.parametrize("bad", [[0], [-3], [-1, 1], [-1, 0, 3], [-1, 5, 0], [-2, 0], [-1, -2, 1]])
def test_bad_parent_status(bad):
    anc, child, depth, st = tree.build_mask(bad)
    assert st == ST_BAD_PARENT
    assert all(a == 0 for a in anc) and all(c == 0 for c in child) and all(d == 0 for d in depth)


def test_too_many_nodes():
    _, _, _, st = tree.build_mask([-1] * 65)
    assert st == ST_BAD_PARENT


def test_empty_tree():
    anc, child, depth, st = tree.build_mask([])
    assert st == ST_OK and anc == [] and child == [0] and depth == []


def test_padding_slots():
    # -2 marks an unused slot: no ancestors, nobody's child, never a parent
    anc, child, depth, st = tree.build_mask([-1, -2, 0, -2, 2])
    assert st == ST_OK
    assert anc == [0b1, 0, 0b101, 0, 0b10101]
    assert depth == [1, 0, 2, 0, 3]
    assert child == [0b1, 0b100, 0, 0b10000, 0, 0]
    assert tree.children_of([-1, -2, 0], -1) == [0]
    anc, child, depth, st = tree.build_mask([-2, -2])
    assert st == ST_OK and anc == [0, 0] and child == [0, 0, 0]
