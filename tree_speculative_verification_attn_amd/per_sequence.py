"""Per-sequence layout of a token tree, to compare tree attention with
sequence-based verification.

SpecInfer summary, "Evaluation", Figure 11 (tree-based against sequence-based
parallel decoding): sequence-based decoding verifies every root-to-leaf path
of the token tree as a sequence of its own, so each path reads the verified
prefix's keys and values again; tree-based decoding reads them once for the
whole tree ("Token Tree Verifier: Tree Attention").

`build` lays a batch of trees out as such a batch of sequences for the same
`tree_attn_verify` call: request s = (b, leaf) is the chain of nodes on the
path from the root to that leaf, over request b's prefix.  Whole prefix blocks
are shared (the block tables of b's paths point at b's physical blocks), so the
prefix is stored once and read once per path; the block that holds the
prefix's end, and the chain's own slots, are private to each path.  Chains
shorter than the longest path end in padding slots (parent -2).  Node j of
chain s attends to the prefix and to chain nodes 0..j, which are exactly the
prefix, the ancestors and the node itself in the tree: its output equals the
tree output of the node it copies.

This is data movement with torch on the device, done once before anything is
timed; the attention is the library's.
"""
from dataclasses import dataclass

import numpy as np
import torch

BLOCK = 16


def leaf_paths(parent_row):
    """Root-to-leaf node lists of one tree (-1 = child of the root,
    -2 = padding slot), leaves in index order, each path root end first."""
    parent_row = [int(p) for p in parent_row]
    has_child = [False] * len(parent_row)
    for p in parent_row:
        if p >= 0:
            has_child[p] = True
    paths = []
    for i, p in enumerate(parent_row):
        if p == -2 or has_child[i]:
            continue
        path = [i]
        while parent_row[path[-1]] >= 0:
            path.append(parent_row[path[-1]])
        paths.append(path[::-1])
    return paths


@dataclass
class SequenceBatch:
    parent: torch.Tensor        # [S][N2] int32 chains, -2 padding
    q: torch.Tensor             # [S][N2][H][D]
    k_cache: torch.Tensor       # original blocks + private blocks
    v_cache: torch.Tensor
    block_table: torch.Tensor   # [S][MB2] int32
    prefix_len: torch.Tensor    # [S] int32
    paths: list                 # (b, [node ids]) per sequence
    kv_bytes: int               # K/V bytes one attention call reads: prefix and N2 slots per path

    @property
    def S(self):
        return self.parent.shape[0]

    @property
    def N(self):
        return self.parent.shape[1]


def build(parent, prefix_len, q, k_cache, v_cache, block_table):
    """Sequence batch of a tree batch.

    parent [B][N] and prefix_len [B] are host int arrays; q [B][N][H][D],
    k_cache / v_cache [blocks][H][16][D] and block_table [B][max_blocks]
    (int32) are device tensors in the tree layout (node i at slot L_b + i)."""
    parent = np.asarray(parent)
    prefix_len = np.asarray(prefix_len)
    bt = block_table.cpu().numpy()
    dev = q.device
    B, N = parent.shape
    H, D = q.shape[2], q.shape[3]
    seqs = [(b, p) for b in range(B) for p in leaf_paths(parent[b])]
    S = len(seqs)
    N2 = max((len(p) for _, p in seqs), default=1)
    nb0 = k_cache.shape[0]

    par2 = np.full((S, N2), -2, dtype=np.int32)
    pl2 = np.zeros(S, dtype=np.int32)
    first_fresh = [int(prefix_len[b]) // BLOCK for b, _ in seqs]
    last_fresh = [(int(prefix_len[b]) + N2 - 1) // BLOCK for b, _ in seqs]
    mb2 = max(last_fresh, default=0) + 1
    bt2 = np.zeros((S, mb2), dtype=np.int32)
    init_src = []                 # original block copied into each private block
    dst_blk, dst_row, src_blk, src_row = [], [], [], []
    q_s, q_j, q_b, q_i = [], [], [], []
    nxt = nb0
    for s, (b, path) in enumerate(seqs):
        L = int(prefix_len[b])
        pl2[s] = L
        par2[s, :len(path)] = np.arange(-1, len(path) - 1, dtype=np.int32)
        f0, f1 = first_fresh[s], last_fresh[s]
        bt2[s, :f0] = bt[b, :f0]
        fresh = {}
        for f in range(f0, f1 + 1):
            bt2[s, f] = nxt
            fresh[f] = nxt
            init_src.append(int(bt[b, f]))      # carries the prefix tail into block f0
            nxt += 1
        for j, node in enumerate(path):
            d, sl = divmod(L + j, BLOCK)
            dst_blk.append(fresh[d])
            dst_row.append(sl)
            d0, sl0 = divmod(L + node, BLOCK)
            src_blk.append(int(bt[b, d0]))
            src_row.append(sl0)
            q_s.append(s)
            q_j.append(j)
            q_b.append(b)
            q_i.append(node)

    def idx(a):
        return torch.as_tensor(np.asarray(a, dtype=np.int64), device=dev)

    caches = []
    for c in (k_cache, v_cache):
        c2 = torch.cat([c, c[idx(init_src)]]) if init_src else c.clone()
        if dst_blk:
            c2[idx(dst_blk), :, idx(dst_row), :] = c[idx(src_blk), :, idx(src_row), :]
        caches.append(c2)
    q2 = torch.zeros((S, N2, H, D), dtype=q.dtype, device=dev)
    if q_s:
        q2[idx(q_s), idx(q_j)] = q[idx(q_b), idx(q_i)]
    elem = q.element_size()
    kv_bytes = sum(2 * H * D * elem * (int(prefix_len[b]) + N2) for b, _ in seqs)
    return SequenceBatch(parent=torch.as_tensor(par2, device=dev), q=q2, k_cache=caches[0],
                         v_cache=caches[1], block_table=torch.as_tensor(bt2, device=dev),
                         prefix_len=torch.as_tensor(pl2, device=dev), paths=seqs, kv_bytes=kv_bytes)
