"""Pins for the oracle's tree attention.

* Definition 4.1 (SpecInfer summary, "Token Tree Verifier: Tree Attention"):
  each node's output equals ordinary causal attention over the sequence
  prefix + root-to-node path, here computed by torch's CPU
  scaled_dot_product_attention in float64.
* A chain tree reduces TreeMask to the standard causal mask (Equation 3).
* "Depth-First KV-Cache Management": a sequential DFS over one shared cache
  that holds exactly S_u when u is visited gives the same outputs.
* Softmax-weighted sums do not depend on the order of the prefix slots.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention, tree
from oracle.attention import gather_slots, widen
from oracle.status import ST_BAD_BLOCK, ST_KV_CAPACITY, ST_OK


def _wl(parent, L=37, H=2, D=16, dtype="f32", seed=5):
    return synth.make_workload(dict(name="t", B=1, H=H, D=D, L=L, dtype=dtype, V=16,
                                    tree=("parents", parent), sig_t=1.0, sig_s=1.0), seed)


def _oracle(w):
    anc, child, depth, st = tree.build_mask_batch(w.parent)
    out, st2 = attention.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                        anc, st, w.dtype, w.scale)
    return out, st2


def _sdpa_last(qv, K, V, scale):
    n, D = K.shape
    Q = torch.zeros((1, 1, n, D), dtype=torch.float64)
    Q[0, 0, -1] = torch.from_numpy(qv)
    o = torch.nn.functional.scaled_dot_product_attention(
        Q, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
        is_causal=True, scale=scale)
    return o[0, 0, -1].numpy()


PARENTS = {
    "fig3": [-1, 0, 1, 0, 3, -1, 5, 6, 5, 8],
    "p3": [-1, 0, 0, 1, 1, 2],
    "star": [-1] * 9,
    "deep": [-1, 0, 1, 2, 3, 4, 5, 2, 7, 7, 0],
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(PARENTS))
def test_definition_4_1_bruteforce(name, dtype):
    parent = PARENTS[name]
    w = _wl(parent, dtype=dtype)
    out, st = _oracle(w)
    assert st == [ST_OK]
    L = int(w.prefix_len[0])
    for h in range(w.H):
        for i in range(w.N):
            path = tree.path_to(parent, i)
            slots = list(range(L)) + [L + j for j in path]
            K = gather_slots(w.k_cache, w.block_table[0], slots, h, dtype)
            Vv = gather_slots(w.v_cache, w.block_table[0], slots, h, dtype)
            ref = _sdpa_last(widen(w.q[0, i, h], dtype), K, Vv, w.scale)
            np.testing.assert_allclose(out[0, i, h], ref, rtol=1e-12, atol=1e-12)


def test_chain_equals_causal_attention():
    n = 12
    w = _wl([-1] + list(range(n - 1)), L=29)
    out, _ = _oracle(w)
    L = int(w.prefix_len[0])
    for h in range(w.H):
        slots = list(range(L + n))
        K = torch.from_numpy(gather_slots(w.k_cache, w.block_table[0], slots, h, "f32"))
        Vv = torch.from_numpy(gather_slots(w.v_cache, w.block_table[0], slots, h, "f32"))
        Q = torch.zeros((L + n, w.D), dtype=torch.float64)
        Q[L:] = torch.from_numpy(widen(w.q[0, :, h], "f32"))
        o = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], Vv[None],
                                                             is_causal=True, scale=w.scale)[0]
        np.testing.assert_allclose(out[0, :, h], o[L:].numpy(), rtol=1e-12, atol=1e-12)


def test_dfs_kv_cache_formulation():
    parent = PARENTS["deep"]
    w = _wl(parent, L=21)
    out, _ = _oracle(w)
    L = int(w.prefix_len[0])
    depth = tree.build_mask(parent)[2]
    kids = [tree.children_of(parent, u) for u in range(-1, len(parent))]
    for h in range(w.H):
        cacheK = list(gather_slots(w.k_cache, w.block_table[0], range(L), h, "f32"))
        cacheV = list(gather_slots(w.v_cache, w.block_table[0], range(L), h, "f32"))
        stack = list(reversed(kids[0]))
        while stack:
            u = stack.pop()
            d = depth[u]
            del cacheK[L + d - 1:]
            del cacheV[L + d - 1:]
            cacheK.append(gather_slots(w.k_cache, w.block_table[0], [L + u], h, "f32")[0])
            cacheV.append(gather_slots(w.v_cache, w.block_table[0], [L + u], h, "f32")[0])
            K = np.array(cacheK)
            s = K @ widen(w.q[0, u, h], "f32") * w.scale
            p = np.exp(s - s.max())
            ref = (p[:, None] * np.array(cacheV)).sum(0) / p.sum()
            np.testing.assert_allclose(out[0, u, h], ref, rtol=1e-12, atol=1e-12)
            stack.extend(reversed(kids[u + 1]))


def test_prefix_order_invariance():
    w = _wl(PARENTS["fig3"], L=40)
    out, _ = _oracle(w)
    L = int(w.prefix_len[0])
    rng = np.random.default_rng(1)
    perm = rng.permutation(L)
    k2, v2 = w.k_cache.copy(), w.v_cache.copy()
    bt = w.block_table[0]
    for dst, src in enumerate(perm):
        db, do = bt[dst // 16], dst % 16
        sb, so = bt[src // 16], src % 16
        k2[db, :, do] = w.k_cache[sb, :, so]
        v2[db, :, do] = w.v_cache[sb, :, so]
    anc, _, _, st = tree.build_mask_batch(w.parent)
    out2, _ = attention.tree_attention(w.q, k2, v2, w.block_table, w.prefix_len, anc, st, "f32", w.scale)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-13)


def test_zero_prefix_root_children_see_only_themselves():
    w = _wl([-1, -1, 0], L=0)
    out, _ = _oracle(w)
    for h in range(w.H):
        for i in (0, 1):
            np.testing.assert_allclose(out[0, i, h], widen(w.v_cache[w.block_table[0, 0], h, i], "f32"))


def test_status_paths():
    w = _wl(PARENTS["p3"], L=20)
    anc, _, _, st = tree.build_mask_batch(w.parent)
    # incoming nonzero status: zero output, status kept
    out, s = attention.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len, anc,
                                      [1], "f32", w.scale)
    assert s == [1] and np.all(out == 0)
    # capacity
    out, s = attention.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table,
                                      np.array([w.max_blocks * 16]), anc, st, "f32", w.scale)
    assert s == [ST_KV_CAPACITY]
    bt = w.block_table.copy()
    bt[0, 0] = w.num_blocks
    out, s = attention.tree_attention(w.q, w.k_cache, w.v_cache, bt, w.prefix_len, anc, st, "f32", w.scale)
    assert s == [ST_BAD_BLOCK]
