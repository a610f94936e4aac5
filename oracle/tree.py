"""Tree topology: ancestor masks, child sets, depths (oracle side).

Source: SpecInfer summary, section "Tree-based Parallel Decoding:
Topology-Aware Causal Mask" (TreeMask equation): node u may attend node v iff
v is an ancestor of u in the token tree or v = u; the verified prefix is
visible to every node (the blog summary of SpecInfer on page 2 states the
prefix + own-ancestors rule explicitly).

Representation: nodes 0..N-1 in an order where every parent precedes its
children (DFS preorder in practice); parent[i] = -1 marks a child of the
root, the root being the end of the verified prefix (not a node).
parent[i] = -2 marks an unused padding slot, so that trees of different sizes
share one batch: it is nobody's child, has no ancestors (anc 0, depth 0) and
cannot be a parent.
  anc[i]      bit j set iff node j is node i itself or one of its ancestors
  child[0]    bit j set iff node j is a child of the root
  child[u+1]  bit j set iff node j is a child of node u
  depth[i]    number of nodes on the root-to-i path (1 for root children)
"""
from .status import ST_OK, ST_BAD_PARENT


def build_mask(parent):
    """Return (anc, child, depth, status) for one request, as Python ints.

    A request whose parent array is malformed (parent[i] not in {-2, -1} U
    {j < i : j not padding}) or longer than 64 nodes gets status 1 and
    all-zero outputs.
    """
    n = len(parent)
    anc = [0] * n
    depth = [0] * n
    child = [0] * (n + 1)
    ok = n <= 64 and all(int(parent[i]) in (-2, -1) or
                         (0 <= int(parent[i]) < i and int(parent[int(parent[i])]) != -2)
                         for i in range(n))
    if not ok:
        return anc, child, depth, ST_BAD_PARENT
    for i in range(n):
        p = int(parent[i])
        if p == -2:
            continue
        if p < 0:
            depth[i] = 1
            anc[i] = 1 << i
        else:
            depth[i] = depth[p] + 1
            anc[i] = anc[p] | (1 << i)
        child[p + 1] |= 1 << i
    return anc, child, depth, ST_OK


def build_mask_batch(parent_2d):
    """build_mask for every row of a [B][N] parent array."""
    out = [build_mask(list(row)) for row in parent_2d]
    return ([o[0] for o in out], [o[1] for o in out], [o[2] for o in out], [o[3] for o in out])


def is_node(parent, i):
    """False for a padding slot."""
    return int(parent[i]) != -2


def children_of(parent, u):
    """Children of node u (u = -1: the root), ascending node index."""
    return [i for i, p in enumerate(parent) if int(p) == u]


def path_to(parent, i):
    """Root-to-i node path S_i (Definition 3.1), excluding the root."""
    path = []
    while i >= 0:
        path.append(i)
        i = int(parent[i])
    return path[::-1]
