"""Tree attention over a paged KV cache, float64 (oracle side).

Sources (SpecInfer summary, page 1):
  * Equations 1-4 ("Standard sequence attention"): scores Q K^T / sqrt(d),
    mask, softmax, times V, per head.
  * Definition 4.1: TreeAttention(u) = Attention(S_u) for every node u.
  * "Topology-Aware Causal Mask" (TreeMask equation): all tree tokens are
    appended after the verified tokens and one masked attention is computed;
    node u sees the prefix, its ancestors and itself.
  * "KV-cache for verified tokens": prefix K/V are cached; the speculated
    tokens' K/V are added to the same cache.

Layout: the K/V of request b at logical slot t live in physical block
block_table[b][t // 16], row t % 16 of k_cache[block][head].  Slots
0..L_b-1 hold the verified prefix, slot L_b + j holds tree node j.  bf16 inputs
(uint16 bit patterns) widen exactly to float64.
"""
import numpy as np

from .status import ST_OK, ST_KV_CAPACITY, ST_BAD_BLOCK

BLOCK = 16


def widen(x, dtype):
    """fp32 or bf16-bit array -> float64, exactly."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def kv_status(block_table, prefix_len, N, num_blocks):
    """Status after the KV-range checks of one request: capacity, then block ids."""
    L = int(prefix_len)
    max_blocks = len(block_table)
    if L < 0 or L + N > max_blocks * BLOCK:
        return ST_KV_CAPACITY
    nblk = (L + N + BLOCK - 1) // BLOCK
    for j in range(nblk):
        if not (0 <= int(block_table[j]) < num_blocks):
            return ST_BAD_BLOCK
    return ST_OK


def gather_slots(cache, block_table_row, slots, head, dtype):
    """K or V rows of the given logical slots for one head, float64 [len(slots)][D]."""
    slots = np.asarray(slots, dtype=np.int64)
    blk = np.asarray(block_table_row, dtype=np.int64)[slots // BLOCK]
    return widen(cache[blk, head, slots % BLOCK, :], dtype)


def masked_attention_one(qv, K, V, visible, scale):
    """softmax(mask(K qv / sqrt(d))) V for one query: Equations 2-4, with -inf
    outside `visible` (scale = 1/sqrt(d))."""
    if not visible.any():            # a padding slot over an empty prefix
        return np.zeros(V.shape[1])
    s = (K @ qv) * scale
    s = np.where(visible, s, -np.inf)
    m = s.max()
    w = np.exp(s - m)
    w = np.where(visible, w, 0.0)
    return (w[:, None] * V).sum(axis=0) / w.sum()


def tree_attention(q, k_cache, v_cache, block_table, prefix_len, anc, status, dtype, scale,
                   pairs=None, nodes=None):
    """TreeMask attention for every (request b, node i, head h).

    Returns (out, status_out).  out is float64 [B][N][H][D]; entries of
    requests whose incoming status is nonzero are 0; entries not selected by
    `pairs` (list of (b, h)) / `nodes` (list of node ids) are NaN.  A request
    that fails the KV-range checks gets its status set (6 or 7) and
    unspecified output (0 here).
    """
    B, N, H, D = q.shape
    out = np.full((B, N, H, D), np.nan)
    st_out = [int(s) for s in status]
    num_blocks = k_cache.shape[0]
    sel = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    node_sel = list(range(N)) if nodes is None else list(nodes)
    by_b: dict[int, list[int]] = {}
    for b, h in sel:
        by_b.setdefault(b, []).append(h)
    for b, heads in by_b.items():
        if st_out[b] != ST_OK:
            out[b] = 0.0
            continue
        st = kv_status(block_table[b], prefix_len[b], N, num_blocks)
        if st != ST_OK:
            st_out[b] = st
            out[b] = 0.0
            continue
        L = int(prefix_len[b])
        slots = np.arange(L + N)
        for h in heads:
            K = gather_slots(k_cache, block_table[b], slots, h, dtype)
            Vv = gather_slots(v_cache, block_table[b], slots, h, dtype)
            for i in node_sel:
                visible = np.zeros(L + N, dtype=bool)
                visible[:L] = True
                for j in range(N):
                    if (int(anc[b][i]) >> j) & 1:
                        visible[L + j] = True
                qv = widen(q[b, i, h], dtype)
                out[b, i, h] = masked_attention_one(qv, K, Vv, visible, float(scale))
    return out, st_out
