"""Pins for the oracle's accepted-path KV compaction ("KV-cache for verified
tokens", SpecInfer summary; "KV-cache rollback", wiki concept page)."""
import numpy as np

import synth
from oracle import attention, commit, tree
from oracle.status import ST_BAD_ACCEPTED, ST_OK


def _wl(parent, L=37, dtype="bf16"):
    return synth.make_workload(dict(name="t", B=1, H=3, D=16, L=L, dtype=dtype, V=16,
                                    tree=("parents", parent), sig_t=1.0, sig_s=1.0), 21)


def _slot(cache, bt, t):
    return cache[bt[t // 16], :, t % 16]


def test_hazard_path_1_2_4():
    # path (1,2,4): slot L+0 <- L+1, L+1 <- L+2, L+2 <- L+4; slot L+1 is both a
    # destination and an earlier source, so reads must see the old contents
    parent = [-1, -1, 1, 2, 2, 3]
    w = _wl(parent, L=14)
    L = int(w.prefix_len[0])
    acc = np.array([[1, 2, 4, -1, -1, -1]])
    k2, v2, pl, st = commit.kv_commit(w.k_cache, w.v_cache, w.block_table, w.prefix_len, acc,
                                      np.array([3]), [0], w.N)
    bt = w.block_table[0]
    for j, a in enumerate([1, 2, 4]):
        assert np.array_equal(_slot(k2, bt, L + j), _slot(w.k_cache, bt, L + a))
        assert np.array_equal(_slot(v2, bt, L + j), _slot(w.v_cache, bt, L + a))
    assert pl[0] == L + 3 and st[0] == ST_OK
    # prefix and other blocks untouched
    for t in range(L):
        assert np.array_equal(_slot(k2, bt, t), _slot(w.k_cache, bt, t))


def test_commit_then_attend_equals_prefix_plus_path():
    """After compaction, a new token attending to prefix L+k sees the same
    keys as a child of the last accepted node before compaction."""
    parent = [-1, 0, 0, 2, -1, 4]
    path = [0, 2, 3]
    w = _wl(parent + [3], L=23, dtype="f32")         # node 6 = the new token under node 3
    L = int(w.prefix_len[0])
    N = len(parent) + 1
    anc, _, _, st = tree.build_mask_batch(w.parent)
    before, _ = attention.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                         anc, st, "f32", w.scale)
    acc = np.full((1, N), -1)
    acc[0, :3] = path
    k2, v2, pl, _ = commit.kv_commit(w.k_cache, w.v_cache, w.block_table, w.prefix_len, acc,
                                     np.array([3]), [0], N)
    # new tree with one node at slot pl = L+3 holding node 6's K/V and query
    bt = w.block_table[0]
    k3, v3 = k2.copy(), v2.copy()
    dst = int(pl[0])
    k3[bt[dst // 16], :, dst % 16] = _slot(w.k_cache, bt, L + 6)
    v3[bt[dst // 16], :, dst % 16] = _slot(w.v_cache, bt, L + 6)
    anc1, _, _, st1 = tree.build_mask_batch(np.array([[-1]]))
    after, _ = attention.tree_attention(w.q[:, 6:7], k3, v3, w.block_table, pl, anc1, st1, "f32", w.scale)
    np.testing.assert_allclose(after[0, 0], before[0, 6], rtol=1e-12, atol=1e-13)


def test_empty_accept_and_skips():
    w = _wl([-1, 0], L=5)
    acc = np.array([[-1, -1]])
    k2, v2, pl, st = commit.kv_commit(w.k_cache, w.v_cache, w.block_table, w.prefix_len, acc,
                                      np.array([0]), [0], 2)
    assert pl[0] == 5 and np.array_equal(k2, w.k_cache)
    k2, v2, pl, st = commit.kv_commit(w.k_cache, w.v_cache, w.block_table, w.prefix_len, acc,
                                      np.array([-1]), [0], 2)
    assert pl[0] == 5
    k2, v2, pl, st = commit.kv_commit(w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                      np.array([[0, 1]]), np.array([2]), [4], 2)
    assert pl[0] == 5 and st[0] == 4
    k2, v2, pl, st = commit.kv_commit(w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                      np.array([[0, 2]]), np.array([2]), [0], 2)
    assert st[0] == ST_BAD_ACCEPTED and pl[0] == 5
