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


# ----------------------------------------------------------------------------
# The bf16 widening and the paged-slot read, pinned without the oracle's own
# helpers: bfloat16 is the upper half of an IEEE-754 binary32 (1 sign bit,
# 8 exponent bits with bias 127, 7 fraction bits), so its value follows from
# the fields alone.
# ----------------------------------------------------------------------------
def _bf16_value(bits):
    """Value of a bfloat16 bit pattern from its fields (pure Python)."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * float("inf") if f == 0 else float("nan")
    if e == 0:
        return sign * (f / 128.0) * 2.0 ** -126
    return sign * (1.0 + f / 128.0) * 2.0 ** (e - 127)


BF16_TABLE = [
    (0x0000, 0.0), (0x8000, -0.0), (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0xC040, -3.0),
    (0x3F81, 1.0 + 2.0 ** -7), (0x3F00, 0.5), (0x4049, 3.140625), (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133), (0x007F, 127 * 2.0 ** -133), (0x7F80, float("inf")),
    (0xFF80, float("-inf")), (0x3DCD, 0.10009765625), (0x42F7, 123.5),
]


def test_widen_bf16_bit_patterns():
    bits = np.array([b for b, _ in BF16_TABLE], dtype=np.uint16)
    got = widen(bits, "bf16")
    for (b, v), g in zip(BF16_TABLE, got):
        assert g == v and np.signbit(g) == np.signbit(v), (hex(b), g, v)
        assert _bf16_value(b) == v
    # every finite pattern against the field formula
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((allb >> 7) & 0xFF) != 0xFF
    g = widen(allb[finite], "bf16")
    ref = np.array([_bf16_value(int(b)) for b in allb[finite]])
    assert np.array_equal(g, ref)
    assert np.all(np.isnan(widen(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_read_against_contiguous(dtype):
    """The oracle's attention over a paged cache equals attention computed by
    hand on the same keys held contiguously: the test scatters contiguous
    K/V into blocks of 16 slots through its own permuted block table."""
    rng = np.random.default_rng(17)
    H, D, L = 3, 16, 45
    parent = [-1, 0, 0, 1, -1, 4]
    N = len(parent)
    T = L + N
    nblk = (T + 15) // 16
    if dtype == "bf16":
        bits = rng.integers(0x3C00, 0x4100, size=(3, T, H, D)) | (rng.integers(0, 2, size=(3, T, H, D)) << 15)
        bits = bits.astype(np.uint16)
        vals = np.vectorize(_bf16_value)(bits.astype(np.int64))
        kc_cont, vc_cont, q_cont = bits[0], bits[1], bits[2][:N]
        kf, vf, qf = vals[0], vals[1], vals[2][:N]
        dt_np = np.uint16
    else:
        vals = rng.standard_normal((3, T, H, D)).astype(np.float32)
        kc_cont, vc_cont, q_cont = vals[0], vals[1], vals[2][:N]
        kf, vf, qf = (x.astype(np.float64) for x in (vals[0], vals[1], vals[2][:N]))
        dt_np = np.float32
    # physical blocks in a random order, with unused blocks between them
    num_blocks = 3 * nblk
    table = rng.permutation(num_blocks)[:nblk].astype(np.int32)
    kc = np.zeros((num_blocks, H, 16, D), dtype=dt_np)
    vc = np.zeros((num_blocks, H, 16, D), dtype=dt_np)
    for t in range(T):
        for h in range(H):
            kc[table[t // 16], h, t % 16] = kc_cont[t, h]
            vc[table[t // 16], h, t % 16] = vc_cont[t, h]
    q = q_cont[None]                                # [1][N][H][D]
    anc, _, _, st = tree.build_mask_batch(np.array([parent], dtype=np.int32))
    scale = 1.0 / np.sqrt(D)
    out, st2 = attention.tree_attention(q, kc, vc, table[None], np.array([L], dtype=np.int32), anc, st,
                                        dtype, scale)
    assert st2 == [ST_OK]
    for i in range(N):
        path = tree.path_to(parent, i)
        keys = list(range(L)) + [L + j for j in path]
        for h in range(H):
            s = np.array([sum(qf[i, h, d] * kf[t, h, d] for d in range(D)) * scale for t in keys])
            p = np.exp(s - s.max())
            ref = (p[:, None] * vf[keys, h]).sum(axis=0) / p.sum()
            np.testing.assert_allclose(out[0, i, h], ref, rtol=1e-12, atol=1e-13)
