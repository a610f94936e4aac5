"""Seeded synthetic workloads for tree-based speculative verification.

This module builds inputs only: query/key/value tensors in a paged KV cache,
token trees, target-model logits and draft-model (SSM) probabilities.  It holds
none of the verification arithmetic (masking, attention, row statistics,
greedy/MSS walks, compaction); both the CPU oracle and the GPU path consume what
it returns.

Shapes follow the models the SpecInfer summary evaluates (LLaMA-7B, OPT-30B,
LLaMA-65B; page "SpecInfer: Accelerating Large Language Model Serving with
Tree-based Speculative Inference and Verification", section 6 "Experimental
Setup").  Trees follow its two construction methods: expansion with a width
vector <k1..km> (section "Learning-based Speculator: Expansion-Based Token Tree
Construction", Figure 3) and merge of several SSM sequences into one trie
(Definition 3.2).  There are no model weights or prompt datasets here: every
value is drawn from seeded NumPy PCG64 streams.

Layouts (all row-major):
  q            [B][N][H][D]          float32, or uint16 holding bfloat16 bits
  k_cache      [num_blocks][H][16][D] same dtype as q
  v_cache      [num_blocks][H][16][D]
  block_table  [B][max_blocks] int32  physical block of logical block j (-1 unused)
  prefix_len   [B] int32              verified prefix length L_b
  parent       [B][N] int32           parent node index, -1 for children of the root,
                                      -2 for padding slots of a smaller tree
  token        [B][N] int32           speculated token of each node
  target_logits[B][N+1][V] float32    row 0 = root context, row 1+i = node i's context
  ssm_probs    [B][R][V] float32      draft distributions (softmaxed)
  q_row        [B][N] int32           row of ssm_probs that proposed node i
Tree nodes exclude the root; the root is the end of the verified prefix, whose
KV is already in the cache.  Node i's own K/V sits at logical slot L_b + i.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16

__all__ = [
    "BLOCK", "CONFIGS", "Workload", "make_config", "make_workload",
    "expansion_tree", "random_tree", "dfs_relabel", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "iid_tree_batch",
]


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Configurations (the five page-shaped workloads)
# ----------------------------------------------------------------------------
CONFIGS = {
    1: dict(name="tiny", B=1, H=4, D=64, L=128, dtype="f32", V=512,
            tree=("fig3",), sig_t=2.0, sig_s=1.0, verify=("greedy", "mss")),
    2: dict(name="llama7b_layer", B=8, H=32, D=128, L=1024, dtype="bf16", V=32000,
            tree=("expand", (2, 2, 2, 1, 1, 1, 1)), sig_t=3.0, sig_s=1.5, verify=("mss",)),
    3: dict(name="opt30b_layer", B=16, H=56, D=128, L=2048, dtype="bf16", V=50272,
            tree=("merge", 3, 8, 4), sig_t=3.0, sig_s=1.5, verify=("greedy", "mss")),
    4: dict(name="llama65b_layer", B=32, H=64, D=128, L=("uniform", 512, 4096), dtype="bf16",
            V=32000, tree=("random", 64, 8, 8), sig_t=3.0, sig_s=1.5, verify=("mss",)),
    5: dict(name="long_context", B=4, H=32, D=128, L=32768, dtype="bf16", V=32000,
            tree=("expand_trunc", (4, 4, 2, 1, 1), 64), sig_t=3.0, sig_s=1.5,
            verify=("mss", "commit")),
}


@dataclass
class Workload:
    name: str
    B: int
    N: int
    H: int
    D: int
    V: int
    R: int
    dtype: str                      # "f32" or "bf16"
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    prefix_len: np.ndarray
    parent: np.ndarray
    token: np.ndarray
    target_logits: np.ndarray
    ssm_probs: np.ndarray
    q_row: np.ndarray
    seed: int                       # Philox key for MSS
    offset: int = 0                 # Philox stream offset
    scale: float = 0.0
    meta: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


# ----------------------------------------------------------------------------
# Tree shapes
# ----------------------------------------------------------------------------
def dfs_relabel(parent: list[int], child_order: list[list[int]] | None = None):
    """Relabel a tree (parent[i] < 0 means child of the root) to DFS preorder.

    child_order[u+1] lists the children of u (u = -1 is the root) in the order
    they must be visited; by default, ascending original index.  Returns
    (new_parent, perm) with perm[new] = old.
    """
    n = len(parent)
    if child_order is None:
        child_order = [[] for _ in range(n + 1)]
        for i, p in enumerate(parent):
            child_order[p + 1].append(i)
    perm: list[int] = []
    stack = list(reversed(child_order[0]))
    while stack:
        u = stack.pop()
        perm.append(u)
        stack.extend(reversed(child_order[u + 1]))
    assert len(perm) == n
    inv = {old: new for new, old in enumerate(perm)}
    new_parent = [(-1 if parent[old] < 0 else inv[parent[old]]) for old in perm]
    return new_parent, perm


def expansion_tree(widths, max_nodes: int | None = None):
    """Parent array (DFS preorder) of a static expansion tree <k1..km>.

    The tree grows level by level: every node at depth d-1 gets widths[d-1]
    children (Expansion-Based Token Tree Construction).  With max_nodes the
    level-by-level growth stops once that many nodes exist.  Returns
    (parent, rank) where rank[i] is node i's rank among its siblings (0 = the
    SSM's top-1 token).
    """
    parent_bfs: list[int] = []
    rank_bfs: list[int] = []
    frontier = [-1]
    for w in widths:
        nxt = []
        for u in frontier:
            for r in range(w):
                if max_nodes is not None and len(parent_bfs) >= max_nodes:
                    break
                parent_bfs.append(u)
                rank_bfs.append(r)
                nxt.append(len(parent_bfs) - 1)
        frontier = nxt
    parent, perm = dfs_relabel(parent_bfs)
    rank = [rank_bfs[old] for old in perm]
    return parent, rank


def random_tree(rng: np.random.Generator, n: int, max_depth: int, max_children: int):
    """Random tree: node 0 is the only child of the root; node i >= 1 picks its
    parent uniformly among earlier nodes that still have depth < max_depth and
    fewer than max_children children.  Relabelled to DFS preorder with children
    visited by original index.  Returns (parent, rank)."""
    par = [-1]
    depth = [1]
    nchild = [0]
    for i in range(1, n):
        cand = [u for u in range(i) if depth[u] < max_depth and nchild[u] < max_children]
        u = cand[int(rng.integers(len(cand)))]
        par.append(u)
        depth.append(depth[u] + 1)
        nchild.append(0)
        nchild[u] += 1
    rank_old = [0] * n
    seen = [0] * (n + 1)
    for i, p in enumerate(par):
        rank_old[i] = seen[p + 1]
        seen[p + 1] += 1
    parent, perm = dfs_relabel(par)
    rank = [rank_old[old] for old in perm]
    return parent, rank


# ----------------------------------------------------------------------------
# Random value helpers
# ----------------------------------------------------------------------------
def _softmax_rows(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def _fill_normal_parallel(out: np.ndarray, seedseq: np.random.SeedSequence, chunk_rows: int,
                          to_bf16: bool, scale: float = 1.0):
    """Fill out[i] (first axis) with N(0, scale^2) draws, chunked so that the
    values depend only on the seed and chunk_rows, not on the thread count."""
    n = out.shape[0]
    nchunks = (n + chunk_rows - 1) // chunk_rows
    children = seedseq.spawn(nchunks)

    def work(c):
        lo, hi = c * chunk_rows, min(n, (c + 1) * chunk_rows)
        g = np.random.Generator(np.random.PCG64(children[c]))
        vals = g.standard_normal(size=(hi - lo,) + out.shape[1:], dtype=np.float32)
        if scale != 1.0:
            vals *= np.float32(scale)
        out[lo:hi] = f32_to_bf16_bits(vals) if to_bf16 else vals

    workers = max(1, min(16, os.cpu_count() or 1))
    if nchunks == 1 or workers == 1:
        for c in range(nchunks):
            work(c)
    else:
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nchunks)))


def _alloc_paged_kv(ss: np.random.SeedSequence, B, H, D, lens, N, dtype):
    """Paged KV cache with a random permutation of physical blocks.

    Each request owns ceil((L_b + N) / 16) blocks; the table maps logical block
    j of request b to a physical block.  Every slot gets N(0,1) values."""
    s_perm, s_k, s_v = ss.spawn(3)
    need = [(int(l) + N + BLOCK - 1) // BLOCK for l in lens]
    nb = int(sum(need))
    max_blocks = max(need)
    perm = np.random.Generator(np.random.PCG64(s_perm)).permutation(nb).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, : need[b]] = perm[off: off + need[b]]
        off += need[b]
    st = np.uint16 if dtype == "bf16" else np.float32
    k = np.empty((nb, H, BLOCK, D), dtype=st)
    v = np.empty((nb, H, BLOCK, D), dtype=st)
    chunk = max(1, (1 << 22) // (H * BLOCK * D))
    _fill_normal_parallel(k, s_k, chunk, dtype == "bf16")
    _fill_normal_parallel(v, s_v, chunk, dtype == "bf16")
    return k, v, table


def _make_q(ss, B, N, H, D, dtype):
    st = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((B, N, H, D), dtype=st)
    _fill_normal_parallel(q.reshape(B * N, H, D) if N else q.reshape(0, H, D), ss, 64, dtype == "bf16")
    return q


# ----------------------------------------------------------------------------
# Logits and trees per request
# ----------------------------------------------------------------------------
def _expansion_request(rng, parent, rank, V, sig_t, sig_s):
    """Logits rows for the root and every node, SSM rows per context, and the
    children's tokens = the SSM's top-w tokens at the parent's context."""
    N = len(parent)
    tl = (rng.standard_normal((N + 1, V), dtype=np.float32) * np.float32(sig_t))
    sl = tl + rng.standard_normal((N + 1, V), dtype=np.float32) * np.float32(sig_s)
    sp = _softmax_rows(sl)
    q_row = np.array([p + 1 for p in parent], dtype=np.int32)
    token = np.empty(N, dtype=np.int32)
    order_cache: dict[int, np.ndarray] = {}
    for i in range(N):
        r = q_row[i]
        if r not in order_cache:
            order_cache[r] = np.argsort(-sp[r], kind="stable")
        token[i] = order_cache[r][rank[i]]
    return tl, sp, token, q_row


def _merge_request(rng, V, n_ssm, chain_len, topk, sig_t, sig_s):
    """Merge-based tree: n_ssm draft chains of length chain_len; at each step
    SSM j samples from its renormalised top-k at the current context.  The
    chains are merged into one trie (Definition 3.2), children in first
    appearance order.  SSM j's logits at a context = that context's target
    logits + SSM-specific noise, drawn once per (context, j)."""
    trie_children: list[dict[int, int]] = [dict()]    # trie node 0 = root
    trie_parent = [-1]
    trie_token = [-1]
    target_rows = [rng.standard_normal(V, dtype=np.float32) * np.float32(sig_t)]
    ssm_rows: list[np.ndarray] = []
    ssm_row_of: dict[tuple[int, int], int] = {}
    proposer: dict[int, int] = {}
    for j in range(n_ssm):
        u = 0
        for _ in range(chain_len):
            key = (u, j)
            if key not in ssm_row_of:
                noisy = target_rows[u] + rng.standard_normal(V, dtype=np.float32) * np.float32(sig_s)
                ssm_row_of[key] = len(ssm_rows)
                ssm_rows.append(_softmax_rows(noisy[None])[0])
            p = ssm_rows[ssm_row_of[key]].astype(np.float64)
            top = np.argsort(-p, kind="stable")[:topk]
            w = p[top] / p[top].sum()
            x = int(top[int(rng.choice(topk, p=w))])
            nxt = trie_children[u].get(x)
            if nxt is None:
                nxt = len(trie_parent)
                trie_children[u][x] = nxt
                trie_children.append(dict())
                trie_parent.append(u)
                trie_token.append(x)
                target_rows.append(rng.standard_normal(V, dtype=np.float32) * np.float32(sig_t))
                proposer[nxt] = j
            else:
                proposer[nxt] = min(proposer[nxt], j)
            u = nxt
    # trie nodes 1.. -> tree nodes 0.. ; relabel to DFS preorder
    n = len(trie_parent) - 1
    par = [trie_parent[t + 1] - 1 for t in range(n)]
    order = [[c - 1 for c in trie_children[u].values()] for u in range(n + 1)]
    parent, perm = dfs_relabel(par, order)
    token = np.array([trie_token[old + 1] for old in perm], dtype=np.int32)
    tl = np.stack([target_rows[0]] + [target_rows[old + 1] for old in perm])
    q_row = np.array([ssm_row_of[(trie_parent[old + 1], proposer[old + 1])] for old in perm],
                     dtype=np.int32)
    sp = np.stack(ssm_rows)
    return parent, tl, sp, token, q_row


def _fig3_tree():
    """Figure 3's tree (expansion <2,2,1> from "machine"): learning{algorithm{is},
    system{design}}, translation{models{are}, system{design}} in DFS preorder."""
    parent = [-1, 0, 1, 0, 3, -1, 5, 6, 5, 8]
    words = ["learning", "algorithm", "is", "system", "design",
             "translation", "models", "are", "system", "design"]
    rank = [0, 0, 0, 1, 0, 1, 0, 0, 1, 0]
    return parent, rank, words


def make_workload(cfg: int | dict, seed: int | None = None, *, B=None, L=None, H=None,
                  D=None, V=None, dtype=None, tree=None, philox_seed=None) -> Workload:
    """Build one workload.  `cfg` is a config id (1..5) or a dict of the same
    keys as CONFIGS entries; keyword overrides shrink a config for tests."""
    if isinstance(cfg, int):
        cid = cfg
        c = dict(CONFIGS[cfg])
    else:
        cid = 0
        c = dict(cfg)
    for k_, v_ in dict(B=B, L=L, H=H, D=D, V=V, dtype=dtype, tree=tree).items():
        if v_ is not None:
            c[k_] = v_
    if seed is None:
        seed = 1000 + cid
    if philox_seed is None:
        philox_seed = 2000 + cid
    Bn, Hn, Dn, Vn = int(c["B"]), int(c["H"]), int(c["D"]), int(c["V"])
    ss = np.random.SeedSequence(seed)
    s_qkv, s_logit, s_tree = ss.spawn(3)
    rng_tree = np.random.Generator(np.random.PCG64(s_tree))

    # prefix lengths
    Lspec = c["L"]
    if isinstance(Lspec, tuple) and Lspec[0] == "uniform":
        lens = rng_tree.integers(Lspec[1], Lspec[2] + 1, size=Bn).astype(np.int32)
    else:
        lens = np.full(Bn, int(Lspec), dtype=np.int32)

    # trees + logits, per request
    tspec = c["tree"]
    kind = tspec[0]
    per_req = []
    lrngs = [np.random.Generator(np.random.PCG64(s)) for s in s_logit.spawn(Bn)]
    for b in range(Bn):
        rng = lrngs[b]
        if kind == "fig3":
            parent, rank, _ = _fig3_tree()
            per_req.append((parent,) + _expansion_request(rng, parent, rank, Vn, c["sig_t"], c["sig_s"]))
        elif kind == "expand":
            parent, rank = expansion_tree(tspec[1])
            per_req.append((parent,) + _expansion_request(rng, parent, rank, Vn, c["sig_t"], c["sig_s"]))
        elif kind == "expand_trunc":
            parent, rank = expansion_tree(tspec[1], max_nodes=tspec[2])
            per_req.append((parent,) + _expansion_request(rng, parent, rank, Vn, c["sig_t"], c["sig_s"]))
        elif kind == "random":
            parent, rank = random_tree(rng_tree, tspec[1], tspec[2], tspec[3])
            per_req.append((parent,) + _expansion_request(rng, parent, rank, Vn, c["sig_t"], c["sig_s"]))
        elif kind == "merge":
            per_req.append(_merge_request(rng, Vn, tspec[1], tspec[2], tspec[3], c["sig_t"], c["sig_s"]))
        elif kind == "parents":
            parent = list(tspec[1])
            rank = _sibling_rank(parent)
            per_req.append((parent,) + _expansion_request(rng, parent, rank, Vn, c["sig_t"], c["sig_s"]))
        else:
            raise ValueError(f"unknown tree kind {kind!r}")

    # Trees of different sizes (merge-built ones) share the batch: the extra
    # slots are padding (parent -2), which no node attends or verifies.
    N = max(len(r[0]) for r in per_req)
    R = max(r[2].shape[0] for r in per_req)
    parent = np.full((Bn, N), -2, dtype=np.int32)
    token = np.zeros((Bn, N), dtype=np.int32)
    q_row = np.zeros((Bn, N), dtype=np.int32)
    tl = np.zeros((Bn, N + 1, Vn), dtype=np.float32)
    sp = np.zeros((Bn, R, Vn), dtype=np.float32)
    for b, (par, tl_b, sp_b, tok_b, qr_b) in enumerate(per_req):
        n_b = len(par)
        parent[b, :n_b] = par
        token[b, :n_b] = tok_b
        q_row[b, :n_b] = qr_b
        tl[b, : n_b + 1] = tl_b
        sp[b, : sp_b.shape[0]] = sp_b

    dt = c["dtype"]
    s_q, s_kv = s_qkv.spawn(2)
    q = _make_q(s_q, Bn, N, Hn, Dn, dt)
    k, v, table = _alloc_paged_kv(s_kv, Bn, Hn, Dn, lens, N, dt)
    return Workload(name=c.get("name", "custom"), B=Bn, N=N, H=Hn, D=Dn, V=Vn, R=R, dtype=dt,
                    q=q, k_cache=k, v_cache=v, block_table=table, prefix_len=lens,
                    parent=parent, token=token, target_logits=tl, ssm_probs=sp, q_row=q_row,
                    seed=int(philox_seed), offset=0, scale=1.0 / float(np.sqrt(Dn)),
                    meta=dict(config=cid, tree=tspec))


def _sibling_rank(parent):
    seen: dict[int, int] = {}
    rank = []
    for p in parent:
        rank.append(seen.get(p, 0))
        seen[p] = seen.get(p, 0) + 1
    return rank


def make_config(cfg_id: int, seed: int | None = None) -> Workload:
    """One of the five named workloads at full size."""
    return make_workload(cfg_id, seed)


# ----------------------------------------------------------------------------
# Trees of i.i.d. draft draws (for distribution tests)
# ----------------------------------------------------------------------------
def iid_tree_batch(seed: int, n_req: int, p: np.ndarray, q: np.ndarray, shape: str = "star3"):
    """Many requests sharing one target distribution p and one draft
    distribution q; each request's children are independent draws from q,
    duplicates kept as separate nodes.

    shape "starK": K root children (N = K).  shape "d2": two root children,
    each with two children of its own (N = 6; the second level's draft and
    target rows equal the first level's).  Returns (parent[N], token[n_req][N],
    target_logits[n_req][N+1][V], ssm_probs[n_req][R][V], q_row[n_req][N]).
    Logits are log(p) so that the verifier's softmax gives p back."""
    rng = np.random.Generator(np.random.PCG64(seed))
    V = len(p)
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    if shape.startswith("star"):
        parent = [-1] * int(shape[4:])
    elif shape == "d2":
        parent = [-1, 0, 0, -1, 3, 3]
    else:
        raise ValueError(shape)
    N = len(parent)
    cq = np.cumsum(q)
    cq[-1] = 1.0
    draws = np.searchsorted(cq, rng.random((n_req, N)), side="right").astype(np.int32)
    draws = np.minimum(draws, V - 1)
    with np.errstate(divide="ignore"):
        lp = np.log(p).astype(np.float32)
    tl = np.broadcast_to(lp, (n_req, N + 1, V)).copy()
    sp = np.broadcast_to(q.astype(np.float32), (n_req, 1, V)).copy()
    q_row = np.zeros((n_req, N), dtype=np.int32)
    return np.array(parent, dtype=np.int32), draws, tl, sp, q_row


def merged_tree_batch(seed: int, n_req: int, p: np.ndarray, qs: list):
    """Many requests sharing one target distribution p; SSM i proposes one
    root child drawn from its own distribution qs[i] (independent draws), and
    proposals of the same token share one node (first appearance order).

    Returns parent[N] with N = len(qs) (nodes past the request's distinct
    tokens are padding, parent -2: the tree shape differs per request, so
    parent is [n_req][N]), token[n_req][N], target_logits[n_req][N+1][V] =
    log p, ssm_probs[n_req][R][V] with row i = qs[i], prop_node[n_req][S] and
    prop_row[n_req][S] (S = len(qs): slot i is SSM i's proposal), and q_row
    [n_req][N] = the row of each node's first proposer."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = len(qs)
    V = len(p)
    draws = np.zeros((n_req, k), dtype=np.int64)
    for i, q in enumerate(qs):
        cq = np.cumsum(np.asarray(q, dtype=np.float64))
        cq[-1] = 1.0
        draws[:, i] = np.minimum(np.searchsorted(cq, rng.random(n_req), side="right"), V - 1)
    parent = np.full((n_req, k), -2, dtype=np.int32)
    token = np.zeros((n_req, k), dtype=np.int32)
    prop_node = np.zeros((n_req, k), dtype=np.int32)
    prop_row = np.tile(np.arange(k, dtype=np.int32), (n_req, 1))
    q_row = np.zeros((n_req, k), dtype=np.int32)
    for b in range(n_req):
        node_of = {}
        for i in range(k):
            x = int(draws[b, i])
            if x not in node_of:
                c = len(node_of)
                node_of[x] = c
                parent[b, c] = -1
                token[b, c] = x
                q_row[b, c] = i
            prop_node[b, i] = node_of[x]
    with np.errstate(divide="ignore"):
        lp = np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)
    tl = np.broadcast_to(lp, (n_req, k + 1, V)).copy()
    sp = np.broadcast_to(np.asarray(qs, dtype=np.float32), (n_req, k, V)).copy()
    return parent, token, tl, sp, prop_node, prop_row, q_row
