"""Checks of the synthetic workload generator (shapes, trees, determinism)."""
import numpy as np
import pytest

import synth
from oracle import tree


def test_tree_sizes():
    assert len(synth.expansion_tree((2, 2, 1))[0]) == 10
    assert len(synth.expansion_tree((2, 2, 2, 1, 1, 1, 1))[0]) == 46
    par, _ = synth.expansion_tree((4, 4, 2, 1, 1), max_nodes=64)
    assert len(par) == 64
    d = tree.build_mask(par)[2]
    assert sorted(d).count(1) == 4 and d.count(2) == 16 and d.count(3) == 32 and d.count(4) == 12


def _is_dfs_preorder(parent):
    # every node's subtree is a contiguous index range starting at the node
    n = len(parent)
    for i in range(n):
        sub = {i}
        for j in range(i + 1, n):
            if parent[j] in sub:
                sub.add(j)
        if sub != set(range(i, i + len(sub))):
            return False
    return all(-1 <= parent[i] < i for i in range(n))


@pytest.mark.parametrize("widths", [(2, 2, 1), (2, 2, 2, 1, 1, 1, 1), (3, 1, 2)])
def test_expansion_is_dfs(widths):
    assert _is_dfs_preorder(synth.expansion_tree(widths)[0])


def test_random_tree_limits():
    rng = np.random.default_rng(0)
    for _ in range(20):
        par, _ = synth.random_tree(rng, 64, 8, 8)
        assert _is_dfs_preorder(par)
        anc, child, depth, st = tree.build_mask(par)
        assert st == 0 and max(depth) <= 8
        assert all(bin(c).count("1") <= 8 for c in child[1:])
        assert par.count(-1) == 1


def test_tiny_config():
    w = synth.make_config(1)
    assert (w.B, w.N, w.H, w.D, w.V, w.R) == (1, 10, 4, 64, 512, 11)
    assert list(w.parent[0]) == [-1, 0, 1, 0, 3, -1, 5, 6, 5, 8]
    assert list(w.q_row[0]) == [p + 1 for p in w.parent[0]]
    # children are the SSM's top-w tokens in descending order at the parent's context
    for u in range(-1, w.N):
        kids = tree.children_of(w.parent[0], u)
        if kids:
            order = np.argsort(-w.ssm_probs[0, u + 1], kind="stable")
            assert [w.token[0, c] for c in kids] == list(order[: len(kids)])
    assert np.allclose(w.ssm_probs.sum(-1), 1.0, atol=1e-5)


def test_small_merge_and_random():
    w = synth.make_workload(3, B=2, L=40, H=2, V=300)
    assert w.N <= 24 and _is_dfs_preorder(list(w.parent[0]))
    assert w.R <= 3 * (w.N + 1)
    assert np.all((w.q_row >= 0) & (w.q_row < w.R))
    # each node's token is among its proposing SSM's top-4 at the parent's context
    for b in range(2):
        for i in range(w.N):
            top4 = np.argsort(-w.ssm_probs[b, w.q_row[b, i]], kind="stable")[:4]
            assert w.token[b, i] in top4
    w4 = synth.make_workload(4, B=3, H=2, V=100)
    assert w4.N == 64 and np.all((w4.prefix_len >= 512) & (w4.prefix_len <= 4096))


def test_paged_layout_and_determinism():
    a = synth.make_workload(2, B=2, L=50, H=2, V=64)
    b = synth.make_workload(2, B=2, L=50, H=2, V=64)
    for f in ("q", "k_cache", "v_cache", "block_table", "token", "target_logits", "ssm_probs"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    used = a.block_table[a.block_table >= 0]
    assert len(set(used.tolist())) == len(used) == a.num_blocks     # a permutation
    assert a.q.dtype == np.uint16 and a.k_cache.shape[1:] == (2, 16, 128)


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38], dtype=np.float32)
    r = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0078125) and r[3] == -2.5
