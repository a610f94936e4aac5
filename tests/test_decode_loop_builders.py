"""Tree builders of the toy decode loop, on the CPU: expansion trees and the
merge of several drafters' chains (SpecInfer summary, "Learning-based
Speculator", Definition 3.2), against brute-force constructions."""
import numpy as np
import torch

from tree_speculative_verification_attn_amd.decode_loop import expand_tree, merge_tree


class TableDrafter:
    """Bigram drafters with given tables (the loop distils them from the target)."""

    def __init__(self, n, V, seed, peaked=False):
        g = torch.Generator().manual_seed(seed)
        s = 3.0 if peaked else 1.0
        self.tables = [torch.softmax(s * torch.randn(V, V, generator=g), -1) for _ in range(n)]
        self.V = V

    def probs(self, j, ctx):
        return self.tables[j][ctx]


def _ancestors_ok(parent):
    for i, p in enumerate(parent):
        assert p in (-2, -1) or 0 <= p < i


def test_expand_top_k():
    d = TableDrafter(1, 50, 3)
    ctx = torch.tensor([4, 17, 4])
    parent, token, q_row, ssm = expand_tree(d, ctx, (3, 2, 1), sample=False, gen=None)
    B, N = token.shape
    assert N == 3 + 6 + 6 and ssm.shape == (B, N + 1, 50)
    for b in range(B):
        par, tok = parent[b].tolist(), token[b].tolist()
        _ancestors_ok(par)
        assert q_row[b].tolist() == [p + 1 for p in par]
        for u in [-1] + list(range(N)):
            kids = [i for i in range(N) if par[i] == u]
            if not kids:
                continue
            ctx_tok = int(ctx[b]) if u < 0 else tok[u]
            want = torch.topk(d.tables[0][ctx_tok], len(kids)).indices.tolist()
            assert [tok[i] for i in kids] == want
            assert torch.equal(ssm[b, u + 1], d.tables[0][ctx_tok])


def test_expand_sampled_keeps_duplicates():
    d = TableDrafter(1, 3, 4, peaked=True)
    g = torch.Generator().manual_seed(0)
    parent, token, q_row, ssm = expand_tree(d, torch.zeros(200, dtype=torch.int64), (4,), sample=True, gen=g)
    # with a peaked 3-token table, some request draws the same token twice
    dup = [len(set(row.tolist())) < 4 for row in token]
    assert any(dup)
    assert (parent == -1).all()


def _trie(chains):
    """Brute-force merge: node per distinct prefix, owner = lowest chain."""
    nodes = {}
    for j, ch in enumerate(chains):
        for l in range(len(ch)):
            key = tuple(ch[:l + 1])
            if key not in nodes:
                nodes[key] = j
    return nodes


def test_merge_matches_trie():
    for seed in range(20):
        d = TableDrafter(4, 6, seed, peaked=True)      # small vocabulary: chains often agree
        ctx = torch.tensor([0, 1, 2, 3, 5])
        parent, token, q_row, ssm = merge_tree(d, ctx, 4, sample=False, gen=None)
        B, N = token.shape
        for b in range(B):
            chains = []
            for j in range(4):
                prev, ch = int(ctx[b]), []
                for _ in range(4):
                    prev = int(torch.argmax(d.tables[j][prev]))
                    ch.append(prev)
                chains.append(ch)
            want = _trie(chains)
            par, tok, qr = parent[b].tolist(), token[b].tolist(), q_row[b].tolist()
            _ancestors_ok(par)
            got = {}
            for i in range(N):
                if par[i] == -2:
                    continue
                path, u = [], i
                while u >= 0:
                    path.append(tok[u])
                    u = par[u]
                key = tuple(path[::-1])
                assert key not in got
                got[key] = qr[i]
            assert set(got) == set(want)
            for key, row in got.items():
                j, l = divmod(row, 4)
                assert j == want[key] and l == len(key) - 1
                prev = int(ctx[b]) if l == 0 else chains[j][l - 1]
                assert torch.equal(ssm[b, row], d.tables[j][prev])
