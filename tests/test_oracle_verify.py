"""Pins for the oracle's verification (SpecInfer summary, "Token
Verification: Greedy Decoding" and "... Multi-Step Speculative Sampling").

Greedy: the spec walk's boundary cases, and token-for-token equality with
plain greedy decoding on a toy one-layer model (the page's quality guarantee).
MSS: exact enumeration (oracle.exact) of the emitted token's distribution is
checked against Theorem 4.2 (i.i.d. drafts -> exactly P_LLM), against a
hand-computed fixed-tree example, and against Theorem 4.3; the sampled oracle
is checked against the exact distribution with a total-variation test, and
planted mistakes (one-hot residual, reused accept uniform, deduplicated
siblings, value-sorted child order) must fail that same test.
"""
import math
from fractions import Fraction as F
from itertools import product

import numpy as np
import pytest

import synth
from oracle import exact, philox, verify
from oracle.status import ST_BAD_QROW, ST_BAD_TOKEN, ST_NONFINITE, ST_OK


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def _onehot_logits(V, tok, big=30.0):
    row = np.zeros(V, dtype=np.float32)
    row[tok] = big
    return row


def _first_token(res, token, b):
    if res["num_accepted"][b] > 0:
        return int(token[b][res["accepted"][b][0]])
    return int(res["bonus"][b])


P8 = [F(x, 100) for x in [5, 10, 15, 20, 5, 25, 10, 10]]
Q8 = [F(x, 100) for x in [30, 5, 5, 10, 25, 5, 15, 5]]


def _sample_first_tokens(parent, tok, tl, sp, qr, seed, n):
    st = [0] * n
    res = verify.verify_mss(np.tile(parent, (n, 1)), tok, tl, sp, qr, st, seed)
    assert np.all(res["status"] == 0)
    return np.array([_first_token(res, tok, b) for b in range(n)]), res


# ----------------------------------------------------------------------------
# greedy
# ----------------------------------------------------------------------------
def test_greedy_full_match_and_root_miss():
    parent = [-1, 0, 1, -1, 3]          # two chains of depth 3 and 2
    token = np.array([[5, 6, 7, 1, 2]])
    V = 16
    tl = np.zeros((1, 6, V), dtype=np.float32)
    # full match along 0-1-2, bonus from node 2's row
    for r, t in [(0, 5), (1, 6), (2, 7), (3, 9), (4, 0), (5, 0)]:
        tl[0, r] = _onehot_logits(V, t)
    res = verify.verify_greedy(np.array([parent]), token, tl, [0])
    assert list(res["accepted"][0][:3]) == [0, 1, 2] and res["num_accepted"][0] == 3
    assert res["bonus"][0] == 9                    # depth + 1 tokens
    # root miss: 1 token, the LLM's own
    tl[0, 0] = _onehot_logits(V, 11)
    res = verify.verify_greedy(np.array([parent]), token, tl, [0])
    assert res["num_accepted"][0] == 0 and res["bonus"][0] == 11


def test_greedy_duplicate_siblings_lowest_index():
    parent = np.array([[-1, -1, 1]])
    token = np.array([[4, 4, 3]])
    tl = np.zeros((1, 4, 8), dtype=np.float32)
    tl[0, 0] = _onehot_logits(8, 4)
    tl[0, 1] = _onehot_logits(8, 2)
    res = verify.verify_greedy(parent, token, tl, [0])
    assert res["num_accepted"][0] == 1 and res["accepted"][0][0] == 0 and res["bonus"][0] == 2


def test_greedy_argmax_first_index_on_ties():
    row = np.array([1.0, 3.0, 3.0, -2.0], dtype=np.float32)
    assert verify.argmax_row(row) == 1


class _Toy:
    """One-layer, multi-head toy transformer with position embeddings
    (float64 weights, fp32 logits)."""

    def __init__(self, rng, V=64, H=2, D=16, base=None, noise=0.0):
        dm = H * D
        self.V, self.H, self.D = V, H, D
        if base is None:
            self.E = rng.normal(0, 1, (V, dm))
            self.P = rng.normal(0, 0.5, (256, dm))
            self.Wq = rng.normal(0, dm ** -0.5, (dm, dm))
            self.Wk = rng.normal(0, dm ** -0.5, (dm, dm))
            self.Wv = rng.normal(0, dm ** -0.5, (dm, dm))
            self.Wo = rng.normal(0, dm ** -0.5, (dm, dm))
            self.Wout = rng.normal(0, 3 * dm ** -0.5, (dm, V))
        else:
            for n in ("E", "P", "Wq", "Wk", "Wv", "Wo", "Wout"):
                a = getattr(base, n)
                setattr(self, n, a + rng.normal(0, noise * a.std(), a.shape))

    def qkv(self, tok, pos):
        h = self.E[tok] + self.P[pos]
        sh = (self.H, self.D)
        return h, (h @ self.Wq).reshape(sh), (h @ self.Wk).reshape(sh), (h @ self.Wv).reshape(sh)

    def head(self, h, att):
        return ((att.reshape(-1) @ self.Wo + h) @ self.Wout).astype(np.float32)

    def full_logits(self, seq):
        """Logits after the last token of seq, recomputing everything."""
        K, Vv = [], []
        for pos, t in enumerate(seq):
            h, q, k, v = self.qkv(t, pos)
            K.append(k)
            Vv.append(v)
        K, Vv = np.array(K), np.array(Vv)
        s = np.einsum("hd,nhd->hn", q, K) / math.sqrt(self.D)
        w = np.exp(s - s.max(1, keepdims=True))
        w /= w.sum(1, keepdims=True)
        return self.head(h, np.einsum("hn,nhd->hd", w, Vv))


def test_greedy_tree_loop_equals_greedy_decoding():
    """Tree-based greedy speculation reproduces incremental greedy decoding
    token for token (VerifyGreedy quality guarantee), with every tree step
    done by the oracle: masks, tree attention over a paged cache, greedy walk,
    accepted-path compaction."""
    from oracle import attention, commit, tree

    rng = np.random.default_rng(11)
    tgt = _Toy(rng)
    drf = _Toy(rng, base=tgt, noise=0.15)
    prompt = [3, 17, 42, 8, 25]
    n_new = 64

    # plain greedy decoding
    seq = list(prompt)
    while len(seq) < len(prompt) + n_new:
        seq.append(int(np.argmax(tgt.full_logits(seq))))
    want = seq[len(prompt):]

    # tree-based loop
    H, D = tgt.H, tgt.D
    nblk = 32
    bt = np.array([np.random.default_rng(1).permutation(nblk)], dtype=np.int32)
    kc = np.zeros((nblk, H, 16, D), dtype=np.float32)
    vc = np.zeros_like(kc)

    def put(slot, k, v):
        b, o = bt[0, slot // 16], slot % 16
        kc[b, :, o], vc[b, :, o] = k, v

    scale = 1.0 / math.sqrt(D)
    out_seq = list(prompt)
    for pos, t in enumerate(prompt[:-1]):
        _, _, k, v = tgt.qkv(t, pos)
        put(pos, k, v)
    L = len(prompt) - 1
    pending = prompt[-1]
    widths = (2, 2, 1)
    steps = 0
    while len(out_seq) < len(prompt) + n_new:
        steps += 1
        # 1. the pending token: its KV joins the cache, its output gives row 0
        h0, q0, k0, v0 = tgt.qkv(pending, L)
        put(L, k0, v0)
        anc1, _, _, st1 = tree.build_mask_batch(np.array([[-1]]))
        o1, _ = attention.tree_attention(q0[None, None].astype(np.float32), kc, vc, bt, np.array([L]),
                                         anc1, st1, "f32", scale)
        row0 = tgt.head(h0, o1[0, 0])
        L += 1
        # 2. draft tree by expansion from the draft model (top-w per level)
        parent, tokens = [], []
        frontier = [(-1, [])]
        for w_ in widths:
            nxt = []
            for u, path in frontier:
                lg = drf.full_logits(out_seq + path)
                for t in np.argsort(-lg, kind="stable")[:w_]:
                    parent.append(u)
                    tokens.append(int(t))
                    nxt.append((len(parent) - 1, path + [int(t)]))
            frontier = nxt
        parent, perm = synth.dfs_relabel(parent)
        tokens = [tokens[o] for o in perm]
        N = len(parent)
        anc, _, depth, st = tree.build_mask_batch(np.array([parent]))
        # 3. target tree pass: KV of every node at slot L + i, then tree attention
        qs = np.zeros((1, N, H, D), dtype=np.float32)
        hs = []
        for i in range(N):
            h, q, k, v = tgt.qkv(tokens[i], L + depth[0][i] - 1)
            put(L + i, k, v)
            qs[0, i] = q
            hs.append(h)
        out, _ = attention.tree_attention(qs, kc, vc, bt, np.array([L]), anc, st, "f32", scale)
        tl = np.stack([row0] + [tgt.head(hs[i], out[0, i]) for i in range(N)])[None]
        # 4. verify, 5. commit
        res = verify.verify_greedy(np.array([parent]), np.array([tokens]), tl, [0])
        k_acc = int(res["num_accepted"][0])
        kc2, vc2, pl, _ = commit.kv_commit(kc, vc, bt, np.array([L]), res["accepted"],
                                           res["num_accepted"], [0], N)
        kc[...], vc[...] = kc2, vc2
        L = int(pl[0])
        out_seq += [tokens[a] for a in res["accepted"][0][:k_acc]] + [int(res["bonus"][0])]
        pending = int(res["bonus"][0])
    got = out_seq[len(prompt): len(prompt) + n_new]
    assert got == want
    assert steps < n_new          # speculation actually accepted tokens


# ----------------------------------------------------------------------------
# MSS: exact enumeration pins
# ----------------------------------------------------------------------------
def _rand_dist(rng, V, zeros=0):
    w = [int(x) for x in rng.integers(1, 20, size=V)]
    for z in rng.choice(V, size=zeros, replace=False):
        w[z] = 0
    s = sum(w)
    return [F(x, s) for x in w]


@pytest.mark.parametrize("V,k", [(3, 1), (3, 2), (4, 3), (5, 2), (5, 3)])
def test_theorem_4_2_iid_drafts_exact(V, k):
    rng = np.random.default_rng(V * 10 + k)
    for trial in range(4):
        p = _rand_dist(rng, V, zeros=trial % 2)
        q = _rand_dist(rng, V, zeros=(trial // 2) % 2)
        assert exact.iid_marginal(p, q, k) == p


def test_single_draft_is_speculative_sampling():
    # P(X=x) = min(p,q)(x) + (sum max(0, q-p)) * norm(max(0, p-q))(x) = p(x)
    p = [F(1, 2), F(1, 3), F(1, 6)]
    q = [F(1, 6), F(1, 6), F(2, 3)]
    for x_draft in range(3):
        d = exact.node_output_dist(p, [(x_draft, q)])
        a = min(F(1), p[x_draft] / q[x_draft])
        res = [max(F(0), pi - qi) for pi, qi in zip(p, q)]
        z = sum(res)
        want = [(a if x == x_draft else 0) + (1 - a) * res[x] / z for x in range(3)]
        assert d == want
    assert exact.iid_marginal(p, q, 1) == p


def test_fixed_top2_children_hand_computed():
    # p=(.3,.3,.4), q=(.6,.3,.1), children = q's top-2 tokens {0, 1}:
    # order (0,1): emit 0 w.p. 1/2, else residual (0,0,1) rejects token 1 -> emit 2;
    # order (1,0): ratio 1 -> emit 1.   Result (1/4, 1/2, 1/4), not p.
    p = [F(3, 10), F(3, 10), F(4, 10)]
    q = [F(6, 10), F(3, 10), F(1, 10)]
    assert exact.node_output_dist(p, [(0, q), (1, q)]) == [F(1, 4), F(1, 2), F(1, 4)]


def test_theorem_4_3_rejection_bound_over_drafts():
    """Theorem 4.3 read as a statement in expectation over the speculated
    tokens: children drawn from their proposing SSM (one q per child, possibly
    different), MSS all-reject probability <= naive rejection probability."""
    rng = np.random.default_rng(3)
    for _ in range(120):
        V = int(rng.integers(2, 5))
        k = int(rng.integers(1, 4))
        p = _rand_dist(rng, V, zeros=int(rng.integers(0, 2)))
        qs = [_rand_dist(rng, V, zeros=int(rng.integers(0, 2))) for _ in range(k)]
        m_mss = m_naive = 0
        for draw in product(range(V), repeat=k):
            w = 1
            for s_, x in enumerate(draw):
                w = w * qs[s_][x]
            if w == 0:
                continue
            m_mss += w * exact.all_reject_prob(p, [(x, qs[s_]) for s_, x in enumerate(draw)])
            m_naive += w * (1 - sum(p[t] for t in set(draw)))
        assert m_mss <= m_naive


def test_theorem_4_3_fails_for_a_fixed_tree():
    """For one fixed tree the bound need not hold: child A (token 2, p = 0)
    is always rejected and its full q row wipes out the mass of child B's
    token.  Orders (A,B) and (B,A) give all-reject 1 and 0: total 1/2 > 3/7."""
    p = [F(4, 7), F(3, 7), F(0)]
    qa = [F(3, 5), F(0), F(2, 5)]
    qb = [F(17, 31), F(2, 31), F(12, 31)]
    assert exact.all_reject_prob(p, [(2, qa), (0, qb)]) == F(1, 2)
    assert 1 - p[2] - p[0] == F(3, 7)


# ----------------------------------------------------------------------------
# MSS: the sampled oracle against the exact distributions
# ----------------------------------------------------------------------------
def _star_fixed(n, p, q, tokens):
    V = len(p)
    tl = np.broadcast_to(np.log(np.array(p, dtype=np.float64)).astype(np.float32), (n, len(tokens) + 1, V)).copy()
    sp = np.broadcast_to(np.array(q, dtype=np.float32), (n, 1, V)).copy()
    tok = np.tile(np.array(tokens, dtype=np.int32), (n, 1))
    return np.array([-1] * len(tokens)), tok, tl, sp, np.zeros((n, len(tokens)), dtype=np.int32)


def test_sampled_fixed_tree_matches_exact():
    p = [F(3, 10), F(3, 10), F(4, 10)]
    q = [F(6, 10), F(3, 10), F(1, 10)]
    n = 20000
    parent, tok, tl, sp, qr = _star_fixed(n, p, q, [0, 1])
    first, _ = _sample_first_tokens(parent, tok, tl, sp, qr, seed=77, n=n)
    hist = np.bincount(first, minlength=3) / n
    assert exact.tv(hist, [0.25, 0.5, 0.25]) < 1.5e-2


def _iid_first_tokens(n, seed, dedup=False, p=None, q=None, shape="star3"):
    p = np.array([float(x) for x in (P8 if p is None else p)])
    q = np.array([float(x) for x in (Q8 if q is None else q)])
    parent, tok, tl, sp, qr = synth.iid_tree_batch(seed, n, p, q, shape)
    if not dedup:
        return _sample_first_tokens(parent, tok, tl, sp, qr, seed=seed + 1, n=n)[0]
    out = []
    for b in range(n):
        toks = list(dict.fromkeys(int(t) for t in tok[b]))
        r = verify.verify_mss(np.array([[-1] * len(toks)]), np.array([toks]), tl[b:b + 1, : len(toks) + 1],
                              sp[b:b + 1], np.zeros((1, len(toks)), dtype=np.int32), [0], seed + 1)
        out.append(_first_token(r, np.array([toks]), 0))
    return np.array(out)


N_TV = 30000
TV_MAX = 2e-2      # mean sampling TV at V=8, n=3e4 is about 6.5e-3


def test_sampled_iid_tree_matches_target():
    first = _iid_first_tokens(N_TV, 500)
    hist = np.bincount(first, minlength=8) / N_TV
    assert exact.tv(hist, P8) < TV_MAX


@pytest.mark.parametrize("mutation", ["onehot_residual", "reuse_accept_uniform", "dedup_siblings",
                                      "sorted_by_q"])
def test_planted_mistakes_fail_tv(monkeypatch, mutation):
    if mutation == "onehot_residual":
        orig = verify.residual

        def onehot(p_cur, q):
            x = int(np.argmax(q * (p_cur < q)))  # the tested token is where p < q dominates
            qq = np.zeros_like(q)
            qq[x] = q[x]
            return orig(p_cur, qq)
        # apply the one-hot rule at the tested token: wrap mss_one's call site
        calls = {}
        orig_select = verify.select_child

        def sel(untested, word0):
            s = orig_select(untested, word0)
            calls["s"] = s
            return s
        monkeypatch.setattr(verify, "select_child", sel)

        def onehot_at_tested(p_cur, q):
            tok = calls["tok"][calls["s"]]
            qq = np.zeros_like(q)
            qq[tok] = q[tok]
            return orig(p_cur, qq)
        monkeypatch.setattr(verify, "residual", onehot_at_tested)
        p = np.array([float(x) for x in P8])
        q = np.array([float(x) for x in Q8])
        parent, tok, tl, sp, qr = synth.iid_tree_batch(600, N_TV, p, q, "star3")
        first = []
        for b in range(N_TV):
            calls["tok"] = tok[b]
            r = verify.verify_mss(parent[None], tok[b:b + 1], tl[b:b + 1], sp[b:b + 1], qr[b:b + 1], [0], 601)
            first.append(_first_token(r, tok[b:b + 1], 0))
        first = np.array(first)
    elif mutation == "reuse_accept_uniform":
        last = {}
        orig_u = philox.unit_open0

        def rec_u(word):
            u = orig_u(word)
            last.setdefault("seq", []).append(u)
            return u
        monkeypatch.setattr(philox, "unit_open0", rec_u)
        orig_sample = verify.sample_from

        def sample_reuse(p_cur, u):
            seq = last.get("seq", [])
            # the accept uniforms precede the final one; reuse the previous if any
            u_prev = seq[-2] if len(seq) >= 2 else u
            last["seq"] = []
            return orig_sample(p_cur, u_prev)
        monkeypatch.setattr(verify, "sample_from", sample_reuse)
        # single draft (the chain case where the defect appears): a rejection
        # leaves the reused uniform in (1/2, 1], which the residual's CDF
        # maps to its upper half only
        pr = [F(15, 100)] * 4 + [F(10, 100)] * 4
        qr_ = [F(5, 100)] * 4 + [F(20, 100)] * 4
        first = _iid_first_tokens(N_TV, 700, p=pr, q=qr_, shape="star1")
        hist = np.bincount(first, minlength=8) / N_TV
        assert exact.iid_marginal(pr, qr_, 1) == pr
        assert exact.tv(hist, pr) > TV_MAX
        return
    elif mutation == "dedup_siblings":
        first = _iid_first_tokens(N_TV, 800, dedup=True)
    else:
        def sel_sorted(untested, word0):
            return untested[0]
        monkeypatch.setattr(verify, "select_child", sel_sorted)
        # children ordered by descending q so "first untested" is the q-sorted order
        p = np.array([float(x) for x in P8])
        q = np.array([float(x) for x in Q8])
        parent, tok, tl, sp, qr = synth.iid_tree_batch(900, N_TV, p, q, "star3")
        order = np.argsort(-q[tok], axis=1, kind="stable")
        tok = np.take_along_axis(tok, order, axis=1)
        first = _sample_first_tokens(parent, tok, tl, sp, qr, seed=901, n=N_TV)[0]
    hist = np.bincount(first, minlength=8) / N_TV
    assert exact.tv(hist, P8) > TV_MAX, mutation


# ----------------------------------------------------------------------------
# MSS: rules of the walk
# ----------------------------------------------------------------------------
def test_sample_from_bruteforce():
    rng = np.random.default_rng(4)
    for _ in range(300):
        V = int(rng.integers(1, 12))
        p = rng.random(V) * (rng.random(V) < 0.7)
        if p.sum() == 0:
            p[0] = 1.0
        u = float(rng.random()) or 1.0
        x, _ = verify.sample_from(p, u)
        c = np.cumsum(p)
        want = next(i for i in range(V) if c[i] >= u * c[-1])
        assert x == want


def test_leaf_accept_samples_leaf_row():
    # chain of 2; drafts have tiny q so every ratio test accepts; the leaf's
    # own target row is one-hot, so the bonus is that token.
    V = 32
    parent = np.array([[-1, 0]])
    token = np.array([[3, 4]])
    tl = np.zeros((1, 3, V), dtype=np.float32)
    tl[0, 0] = _onehot_logits(V, 3)
    tl[0, 1] = _onehot_logits(V, 4)
    tl[0, 2] = _onehot_logits(V, 19, big=120.0)
    sp = np.full((1, 1, V), 1e-6, dtype=np.float32)
    res = verify.verify_mss(parent, token, tl, sp, np.zeros((1, 2), dtype=np.int32), [0], 9)
    assert res["num_accepted"][0] == 2 and list(res["accepted"][0]) == [0, 1]
    assert res["bonus"][0] == 19 and res["rounds"][0] == 2


def test_zero_residual_keeps_distribution():
    # q = 2 p (not normalised): max(0, p - q) = 0 everywhere -> p unchanged
    V = 6
    p = np.array([0.1, 0.2, 0.3, 0.1, 0.2, 0.1])
    pn, z = verify.residual(p, 2 * p)
    assert z == 0.0 and np.array_equal(pn, p)


def test_q_zero_ratio_reading():
    assert verify.ratio_of(0.2, 0.0) == math.inf
    assert verify.ratio_of(0.0, 0.0) == 0.0


def test_status_codes():
    V = 8
    parent = np.array([[-1, 0]])
    tl = np.zeros((1, 3, V), dtype=np.float32)
    sp = np.full((1, 2, V), 1 / V, dtype=np.float32)
    qr = np.zeros((1, 2), dtype=np.int32)
    r = verify.verify_mss(parent, np.array([[1, 8]]), tl, sp, qr, [0], 1)
    assert r["status"][0] == ST_BAD_TOKEN and r["num_accepted"][0] == -1 and r["bonus"][0] == -1
    r = verify.verify_mss(parent, np.array([[1, 2]]), tl, sp, np.array([[0, 2]]), [0], 1)
    assert r["status"][0] == ST_BAD_QROW
    tl2 = tl.copy()
    tl2[0, 0, 5] = np.inf           # the root row is always visited
    r = verify.verify_mss(parent, np.array([[1, 2]]), tl2, sp, qr, [0], 1)
    assert r["status"][0] == ST_NONFINITE
    tl3 = tl.copy()
    tl3[0, 0, :] = -np.inf
    tl3[0, 0, 1] = 0.0              # -inf entries are masked tokens, not errors
    tl3[0, 2, 4] = np.nan           # a row the walk never visits
    sp3 = np.full((1, 2, V), 1e-3, dtype=np.float32)
    r = verify.verify_mss(np.array([[-1, -1]]), np.array([[3, 2]]), tl3, sp3, qr, [0], 1)
    assert r["status"][0] == ST_OK and r["bonus"][0] == 1
    sp2 = sp.copy()
    sp2[0, 0, 1] = -0.5             # the tested child's own probability
    r = verify.verify_mss(parent, np.array([[1, 2]]), tl, sp2, qr, [0], 1)
    assert r["status"][0] == ST_NONFINITE
    assert not verify.q_row_ok(np.array([0.5, np.nan])) and verify.q_row_ok(np.array([0.0, 1.0]))
    r = verify.verify_mss(parent, np.array([[1, 2]]), tl, sp, qr, [3], 1)
    assert r["status"][0] == 3 and r["num_accepted"][0] == -1
    g = verify.verify_greedy(parent, np.array([[1, -1]]), tl, [0])
    assert g["status"][0] == ST_BAD_TOKEN
    g = verify.verify_greedy(parent, np.array([[1, 2]]), tl2, [0])
    assert g["status"][0] == ST_NONFINITE


def test_rounds_and_determinism():
    w = synth.make_workload(1)
    st = [0]
    a = verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, st, w.seed)
    b = verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, st, w.seed)
    assert a["bonus"][0] == b["bonus"][0] and np.array_equal(a["accepted"], b["accepted"])
    assert a["rounds"][0] >= a["num_accepted"][0]


# ----------------------------------------------------------------------------
# Flipped decisions: the near-tie comparison replays the oracle's walk with
# one decision taken the other way.
# ----------------------------------------------------------------------------
def test_sample_other_neighbours():
    p = np.array([0.2, 0.0, 0.3, 0.0, 0.5])
    # threshold just below the sum up to token 2 (0.5): drawn 2, other side 4
    x, m = verify.sample_from(p, 0.5 - 1e-9)
    assert x == 2 and m < 1e-8 and verify.sample_other(p, 0.5 - 1e-9, x) == 4
    # threshold just above the sum up to token 0 (0.2): drawn 2, other side 0
    x, m = verify.sample_from(p, 0.2 + 1e-9)
    assert x == 2 and verify.sample_other(p, 0.2 + 1e-9, x) == 0
    # no token on the other side
    assert verify.sample_other(p, 1e-12, 0) is None
    assert verify.sample_other(p, 1.0, 4) is None


def test_flip_inverts_one_decision():
    # one root child whose ratio test rejects (p(x) tiny, q(x) large); with
    # the test flipped the child is accepted and the bonus comes from its
    # own one-hot row; flipping the final draw moves it to a neighbour
    V = 16
    parent = np.array([[-1]])
    token = np.array([[5]])
    tl = np.zeros((1, 2, V), dtype=np.float32)
    tl[0, 0] = _onehot_logits(V, 9)
    tl[0, 1] = _onehot_logits(V, 11, big=120.0)
    sp = np.full((1, 1, V), 0.5 / (V - 1), dtype=np.float32)
    sp[0, 0, 5] = 0.5
    qr = np.zeros((1, 1), dtype=np.int32)
    r = verify.verify_mss(parent, token, tl, sp, qr, [0], 3)
    assert r["num_accepted"][0] == 0 and [k for k, _ in r["traces"][0]] == ["ratio", "sample"]
    f0 = r["redo"](0, 0)
    assert f0["num_accepted"][0] == 1 and list(f0["accepted"][0][:1]) == [0] and f0["bonus"][0] == 11
    assert f0["rounds"][0] == 1
    # decisions past the end of the walk change nothing
    f9 = r["redo"](0, 9)
    assert f9["bonus"][0] == r["bonus"][0] and f9["num_accepted"][0] == r["num_accepted"][0]
    # the draw: its neighbour on the nearer side, or itself if it has none
    f1 = r["redo"](0, 1)
    p_res = np.maximum(0.0, verify.softmax_row(tl[0, 0]) - sp[0, 0].astype(np.float64))
    p_res /= p_res.sum()
    u2 = philox.unit_open0(philox.words(3, 0, 0, 0, 0)[2])
    alt = verify.sample_other(p_res, u2, int(r["bonus"][0]))
    assert f1["bonus"][0] == (r["bonus"][0] if alt is None else alt)


def test_zero_residual_is_an_event_not_a_decision():
    # q = 2p on the root row: the rejection leaves p unchanged and the trace
    # records the event without a margin
    V = 6
    parent = np.array([[-1]])
    token = np.array([[2]])
    logits = np.log(np.array([0.1, 0.2, 0.3, 0.1, 0.2, 0.1])).astype(np.float32)
    tl = np.stack([logits, logits])[None]
    p = verify.softmax_row(logits)
    sp = (2 * p).astype(np.float32)[None, None]
    r = verify.verify_mss(parent, token, tl, sp, np.zeros((1, 1), dtype=np.int32), [0], 0)
    assert r["num_accepted"][0] == 0            # (this seed rejects the child)
    assert [k for k, _ in r["traces"][0]] == ["ratio", "zero_residual", "sample"]
    assert r["traces"][0][1][1] is None
    # the draw is decision 1, so flipping decision 1 moves the bonus
    x = int(r["bonus"][0])
    alt = r["redo"](0, 1)["bonus"][0]
    assert alt != x and abs(alt - x) >= 1


def test_naive_redo_flips_the_draw():
    w = synth.make_workload(1)
    r = verify.verify_naive(w.parent, w.token, w.target_logits, [0], w.seed)
    n = len(r["traces"][0])
    f = r["redo"](0, n - 1)          # the last draw taken the other way
    assert f["num_accepted"][0] == r["num_accepted"][0]
    assert np.array_equal(f["accepted"], r["accepted"])
