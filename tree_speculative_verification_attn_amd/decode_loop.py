"""A toy speculative decoding loop on one GPU, around the verification path.

SpecInfer summary, "Overview" and "Learning-based Speculator": a speculator
proposes a token tree, either by expansion (the top-k tokens of a small
speculative model at every step) or by merging the token sequences of several
small models into one tree (Definition 3.2); the verifier scores every node of
the tree in one target pass ("Token Tree Verifier: Tree Attention"), keeps the
accepted path and its bonus token (VerifyGreedy / VerifyStochastic), and the
accepted path's K/V is kept ("Tree-based Parallel Decoding: Depth-First
KV-Cache Management").  The wiki concept page "Speculative decoding",
"Implementation sketch", gives the loop: draft, one target pass, accept,
commit, and the bonus token costs no extra target call in that iteration.

Here the bonus token is the next iteration's pending token: its K/V is not in
the cache yet and the target's distribution after it is not known, so each
iteration starts with a one-node target pass over it (its row is the root row
of the new tree), commits it, drafts a tree from it, scores the tree, verifies
and commits the accepted path.

The models are toys with random weights: the target is one transformer layer
(token and position embeddings, one attention block through the library's
tree attention over a paged cache, a residual, an LM head); each drafter is a
bigram table distilled from the target (the target's next-token logits after
each single token) plus noise.  Their dense layers use torch; masks,
attention, verification and KV compaction run in the library's kernels.  The
loop exists to check the path end to end: greedy speculative decoding must
emit exactly what plain greedy decoding of the target emits, and stochastic
speculative decoding (MSS, or the naive draw-then-check rule that Theorem 4.3
compares it with) must sample the target's own distribution.
"""
import numpy as np
import torch

import tree_speculative_verification_attn_amd as tv

BLOCK = 16


class ToyTarget:
    """One-layer toy language model with random weights."""

    def __init__(self, V, d=64, H=2, D=64, max_pos=1024, seed=0, dtype=torch.float32,
                 sharpness=2.5, device="cuda:0"):
        g = torch.Generator().manual_seed(seed)

        def rnd(*shape, s):
            return (torch.randn(*shape, generator=g, dtype=torch.float64) * s).float().to(device)

        self.V, self.d, self.H, self.D, self.dtype, self.device = V, d, H, D, dtype, device
        self.E = rnd(V, d, s=1.0)
        self.P = rnd(max_pos, d, s=0.3)
        self.Wq = rnd(d, H * D, s=d ** -0.5)
        self.Wk = rnd(d, H * D, s=d ** -0.5)
        self.Wv = rnd(d, H * D, s=d ** -0.5)
        self.Wo = rnd(H * D, d, s=(H * D) ** -0.5)
        self.Wout = rnd(d, V, s=sharpness * d ** -0.5)

    def embed(self, tokens, pos):
        return self.E[tokens] + self.P[pos]

    def qkv(self, x):
        B, N, _ = x.shape
        shape = (B, N, self.H, self.D)
        return tuple((x @ W).view(shape).to(self.dtype) for W in (self.Wq, self.Wk, self.Wv))

    def head(self, x, o):
        B, N, _ = x.shape
        return (x + o.float().reshape(B, N, self.H * self.D) @ self.Wo) @ self.Wout


class PagedState:
    """Per-request paged K/V cache of the target (blocks in a shuffled order)."""

    def __init__(self, model, B, capacity, seed=0):
        self.model, self.B = model, B
        self.mb = (capacity + BLOCK - 1) // BLOCK
        nb = B * self.mb
        dev = model.device
        perm = np.random.default_rng(seed).permutation(nb).astype(np.int32)
        self.block_table = torch.as_tensor(perm.reshape(B, self.mb), device=dev)
        shape = (nb, model.H, BLOCK, model.D)
        self.k = torch.zeros(shape, dtype=model.dtype, device=dev)
        self.v = torch.zeros(shape, dtype=model.dtype, device=dev)
        self.prefix_len = torch.zeros(B, dtype=torch.int32, device=dev)

    def write(self, slots, k, v):
        """K/V of node i of request b to logical slot slots[b][i]."""
        blk = torch.gather(self.block_table, 1, (slots // BLOCK).long())
        row = slots % BLOCK
        self.k[blk.long(), :, row.long(), :] = k
        self.v[blk.long(), :, row.long(), :] = v

    def target_pass(self, parent, tokens):
        """Score a batch of trees (node i of request b at slot prefix_len[b] + i):
        returns (logits [B][N][V] fp32, child masks, status)."""
        m = self.model
        B, N = parent.shape
        dev = m.device
        anc = torch.zeros((B, N), dtype=torch.int64, device=dev)
        child = torch.zeros((B, N + 1), dtype=torch.int64, device=dev)
        depth = torch.zeros((B, N), dtype=torch.int32, device=dev)
        status = torch.zeros((B,), dtype=torch.int32, device=dev)
        tv.tree_build_mask(parent, anc, child, depth, status)
        L = self.prefix_len.long()[:, None]
        pos = (L + depth.long() - 1).clamp(min=0)
        x = m.embed(tokens, pos)
        q, k, v = m.qkv(x)
        self.write(L.int() + torch.arange(N, device=dev, dtype=torch.int32)[None, :], k, v)
        code = tv.TV_BF16 if m.dtype == torch.bfloat16 else tv.TV_F32
        n = tv.tree_attn_verify_workspace(code, B, N, m.H, m.D, self.mb)
        ws = torch.zeros(n, dtype=torch.uint8, device=dev) if n else None
        out = torch.empty_like(q)
        tv.tree_attn_verify(q, self.k, self.v, self.block_table, self.prefix_len, anc, status, out, ws)
        return m.head(x, out), child, status

    def commit(self, accepted, num_accepted, status):
        tv.kv_commit_accepted(self.k, self.v, self.block_table, self.prefix_len, accepted, num_accepted,
                              status)

    def prefill(self, prompt):
        """Commit the K/V of prompt tokens [B][m] (m <= 64) as a chain over an empty prefix."""
        B, m = prompt.shape
        dev = self.model.device
        parent = torch.arange(-1, m - 1, dtype=torch.int32, device=dev).repeat(B, 1)
        _, _, status = self.target_pass(parent, prompt)
        acc = torch.arange(m, dtype=torch.int32, device=dev).repeat(B, 1)
        self.commit(acc, torch.full((B,), m, dtype=torch.int32, device=dev), status)

    def pending_pass(self, tokens):
        """One-node pass over the pending tokens [B]: commits their K/V and
        returns the target's next-token logits after them [B][V]."""
        B = tokens.shape[0]
        dev = self.model.device
        parent = torch.full((B, 1), -1, dtype=torch.int32, device=dev)
        logits, _, status = self.target_pass(parent, tokens[:, None])
        self.commit(torch.zeros((B, 1), dtype=torch.int32, device=dev),
                    torch.ones(B, dtype=torch.int32, device=dev), status)
        return logits[:, 0]


def first_token_logits(model):
    """The target's next-token logits after each single token t at position
    0 (an empty prefix): [V][V]."""
    st = PagedState(model, model.V, capacity=BLOCK)
    toks = torch.arange(model.V, device=model.device)
    return st.pending_pass(toks)


class BigramDrafter:
    """n small models q_j(x | t) = softmax(S_j[t] / temp) over the last token
    t, S_j = the target's single-token logits plus Gaussian noise."""

    def __init__(self, model, n_ssm=1, noise=1.0, temp=1.0, seed=1):
        g = torch.Generator().manual_seed(seed)
        base = first_token_logits(model).float().cpu()
        self.tables = [torch.softmax((base + noise * torch.randn(base.shape, generator=g)) / temp, dim=-1)
                       .to(model.device) for _ in range(n_ssm)]
        self.V = model.V

    def probs(self, j, ctx):
        return self.tables[j][ctx]


def expand_tree(drafter, ctx, widths, sample, gen):
    """Expansion tree from the context tokens ctx [B]: at level l every node
    gets widths[l] children, the top-widths[l] tokens of q(. | node's token)
    (sample=False, distinct) or widths[l] independent draws from it
    (sample=True, duplicates kept as separate nodes).  Nodes are numbered level
    by level, so parents precede children.  Returns parent, token, q_row (all
    [B][N]) and ssm_probs [B][N+1][V]: row 0 proposes the root's children,
    row 1+i node i's children."""
    B = ctx.shape[0]
    dev = ctx.device
    parents, tokens = [], []
    frontier_tok = ctx[:, None]                      # [B][F]
    frontier_id = torch.full((B, 1), -1, dtype=torch.int64, device=dev)
    n = 0
    for w in widths:
        F = frontier_tok.shape[1]
        q = drafter.probs(0, frontier_tok)           # [B][F][V]
        if sample:
            ch = torch.multinomial(q.reshape(B * F, -1), w, replacement=True, generator=gen).view(B, F, w)
        else:
            ch = torch.topk(q, w, dim=-1).indices    # [B][F][w], distinct
        par = frontier_id[:, :, None].expand(B, F, w)
        tokens.append(ch.reshape(B, F * w))
        parents.append(par.reshape(B, F * w))
        frontier_tok = ch.reshape(B, F * w)
        frontier_id = torch.arange(n, n + F * w, device=dev)[None, :].expand(B, F * w)
        n += F * w
    parent = torch.cat(parents, 1).int()
    token = torch.cat(tokens, 1)
    N = token.shape[1]
    assert N <= 64, "trees hold at most 64 nodes"
    ssm = torch.cat([drafter.probs(0, ctx)[:, None], drafter.probs(0, token)], 1)
    q_row = (parent + 1).int()
    return parent, token, q_row, ssm.contiguous()


def merge_tree(drafter, ctx, chain_len, sample, gen):
    """Merge the chains of the drafter's n models (Definition 3.2): model j
    drafts chain_len tokens from ctx (argmax, or a draw per step); chains that
    share a token prefix share its nodes.  Slot (l, j) holds the node for
    chain j's prefix of length l + 1 if chain j is the lowest-numbered chain
    with that prefix, otherwise it is a padding slot (parent -2).  A node's
    draft row is that of its lowest-numbered proposing model."""
    B = ctx.shape[0]
    dev = ctx.device
    n = len(drafter.tables)
    chains = torch.empty((B, n, chain_len), dtype=torch.int64, device=dev)
    rows = torch.empty((B, n, chain_len, drafter.V), dtype=torch.float32, device=dev)
    for j in range(n):
        prev = ctx
        for l in range(chain_len):
            q = drafter.probs(j, prev)
            rows[:, j, l] = q
            prev = (torch.multinomial(q, 1, generator=gen)[:, 0] if sample else q.argmax(-1))
            chains[:, j, l] = prev
    # same[b, j, j2, l]: chains j and j2 agree on positions 0..l
    same = torch.cumprod((chains[:, :, None, :] == chains[:, None, :, :]).int(), dim=3).bool()
    rep = same.int().argmax(dim=2)                   # lowest j2 sharing the prefix: [B][n][c]
    exists = rep == torch.arange(n, device=dev)[None, :, None]
    slot = lambda l, j: l * n + j                    # level-major numbering: parents first
    N = n * chain_len
    assert N <= 64, "trees hold at most 64 nodes"
    parent = torch.full((B, N), -2, dtype=torch.int32, device=dev)
    token = torch.zeros((B, N), dtype=torch.int64, device=dev)
    q_row = torch.zeros((B, N), dtype=torch.int32, device=dev)
    for l in range(chain_len):
        for j in range(n):
            e = exists[:, j, l]
            par = torch.full((B,), -1, dtype=torch.int32, device=dev) if l == 0 else \
                slot(l - 1, 0) + rep[:, j, l - 1].int()
            parent[:, slot(l, j)] = torch.where(e, par, torch.full_like(par, -2))
            token[:, slot(l, j)] = chains[:, j, l]
            q_row[:, slot(l, j)] = j * chain_len + l
    return parent, token, q_row, rows.reshape(B, n * chain_len, drafter.V).contiguous()


class SpecDecoder:
    """Batched speculative decoding of B independent requests."""

    def __init__(self, model, drafter, B, mode="mss", tree=("expand", (2, 2)), capacity=512,
                 seed=0, draft_seed=0):
        assert mode in ("greedy", "mss", "naive")
        self.model, self.drafter, self.B, self.mode, self.tree = model, drafter, B, mode, tree
        self.state = PagedState(model, B, capacity, seed=seed)
        self.seed, self.it = seed + 12345, 0
        self.gen = torch.Generator(device=model.device).manual_seed(draft_seed)
        self.pending = None
        self.out = [[] for _ in range(B)]
        self.iters = 0
        self.accepted_total = 0

    def prefill(self, prompt):
        """prompt [B][m]: the first m - 1 tokens go to the cache, the last is pending."""
        if prompt.shape[1] > 1:
            self.state.prefill(prompt[:, :-1])
        self.pending = prompt[:, -1].clone()

    def step(self):
        """One iteration: emits the accepted tokens and the bonus token of every request."""
        st, dev, B = self.state, self.model.device, self.B
        root = st.pending_pass(self.pending)                     # row 0 of the new tree
        kind, arg = self.tree
        sample = self.mode != "greedy"
        if kind == "expand":
            parent, token, q_row, ssm = expand_tree(self.drafter, self.pending, arg, sample, self.gen)
        else:
            parent, token, q_row, ssm = merge_tree(self.drafter, self.pending, arg, sample, self.gen)
        logits, child, status = st.target_pass(parent, token)
        tl = torch.cat([root[:, None], logits], 1).contiguous()
        N, V = token.shape[1], self.model.V
        acc = torch.empty((B, N), dtype=torch.int32, device=dev)
        num = torch.empty((B,), dtype=torch.int32, device=dev)
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
        ws = torch.zeros(tv.tree_verify_workspace(B, N, V), dtype=torch.uint8, device=dev)
        tok32 = token.int().contiguous()
        if self.mode == "greedy":
            tv.tree_verify_greedy(tl, tok32, child, status, acc, num, bonus, ws)
        elif self.mode == "naive":
            tv.tree_verify_naive(tl, tok32, child, status, self.seed, self.it, acc, num, bonus, ws)
        else:
            rounds = torch.empty((B,), dtype=torch.int32, device=dev)
            tv.tree_verify_mss(tl, ssm, q_row, tok32, child, status, self.seed, self.it, acc, num, bonus,
                               rounds, ws)
        st.commit(acc, num, status)
        self.it += 1
        self.iters += 1
        if int((status != 0).sum()):
            raise RuntimeError(f"verification failed: status {status.cpu().numpy().tolist()}")
        acc_c, num_c, bonus_c, tok_c = (t.cpu().numpy() for t in (acc, num, bonus, token))
        for b in range(B):
            k = int(num_c[b])
            self.out[b].extend(int(tok_c[b, i]) for i in acc_c[b, :k])
            self.out[b].append(int(bonus_c[b]))
        self.accepted_total += int(num_c.sum())
        self.pending = bonus.long()

    def generate(self, T):
        while min(len(o) for o in self.out) < T:
            self.step()
        return [o[:T] for o in self.out]


def plain_greedy(model, prompt, T, capacity=512, seed=0):
    """Plain greedy decoding: one target pass per token.  Returns the tokens
    [B][T] and the margin between the two largest logits at each step."""
    st = PagedState(model, prompt.shape[0], capacity, seed=seed)
    if prompt.shape[1] > 1:
        st.prefill(prompt[:, :-1])
    cur = prompt[:, -1].clone()
    toks, margins = [], []
    for _ in range(T):
        lg = st.pending_pass(cur)
        top2 = torch.topk(lg, 2, dim=-1).values
        margins.append((top2[:, 0] - top2[:, 1]).cpu().numpy())
        cur = lg.argmax(-1)
        toks.append(cur.cpu().numpy())
    return np.stack(toks, 1), np.stack(margins, 1)


def continuation_probs(model, prompt_row, T, capacity=512):
    """Exact probabilities of every T-token continuation of one prompt under
    the target (T = 1 or 2): a [V] or [V][V] array."""
    V = model.V
    dev = model.device
    st = PagedState(model, 1, capacity)
    p = prompt_row[None, :].to(dev)
    if p.shape[1] > 1:
        st.prefill(p[:, :-1])
    p1 = torch.softmax(st.pending_pass(p[:, -1]).double(), -1)[0]
    if T == 1:
        return p1.cpu().numpy()
    assert T == 2
    st2 = PagedState(model, V, capacity)
    pv = p.repeat(V, 1)
    if pv.shape[1] > 1:
        st2.prefill(pv[:, :-1])
    st2.pending_pass(pv[:, -1])
    p2 = torch.softmax(st2.pending_pass(torch.arange(V, device=dev)).double(), -1)
    return (p1[:, None] * p2).cpu().numpy()
