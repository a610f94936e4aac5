"""Token verification, float64 (oracle side).

Sources (SpecInfer summary, page 1):
  * "Token Verification: Greedy Decoding (VerifyGreedy)": walk down from the
    root; while some child v of u carries the LLM's predicted token O(u),
    append it and move to v; at the first miss append O(u) and stop.
  * "Token Verification: Stochastic Decoding and Multi-Step Speculative
    Sampling (VerifyStochastic)": at node u, pick an untested child s uniformly
    at random, accept it with probability min(1, P_LLM(x_s|u) / P_SSM_s(x_s|u));
    on rejection replace P_LLM(.|u) by norm(max(0, P_LLM(.|u) - P_SSM_s(.|u)))
    and drop s from the untested set; once every child is rejected, sample the
    next token from the current P_LLM(.|u).  The same page's comparison with
    naive sampling (Theorem 4.3) defines the naive verifier.
  * Wiki concept page "Speculative decoding", section "Implementation sketch":
    when the walk ends at a leaf by acceptance, the bonus token comes from the
    leaf's own target distribution; the normaliser after a rejection can be 0
    (guard).

Readings where the pages are silent:
  * target distributions are softmax(logits) at temperature 1;
  * O(u) is the lowest index among maximal raw fp32 logits; among children
    with the same token the lowest node index wins;
  * the random child is the idx-th untested child in ascending node order,
    idx = (top 24 bits of word 0) * m >> 24; the accept uniform is in (0, 1];
  * q(x) = 0 gives ratio +inf when p(x) > 0 and 0 otherwise;
  * -inf logits are allowed (probability 0); a visited row with NaN, +inf or
    no finite entry, and a draft probability read by the walk that is NaN,
    infinite or negative, stop the request with status 4;
  * a zero normaliser after a rejection leaves the distribution unchanged;
  * the final sample is the smallest x whose cumulative mass reaches
    u * sum(p) (falling back to the last x with p(x) > 0 if rounding leaves
    the total short).

Rows: target_logits[b][0] is the root's context, row 1 + i node i's context.
Outputs per request: accepted node ids (list), bonus token, number of ratio
tests ("rounds"), status, and a trace of the walk's decisions in the order they
are taken, each with its margin, used to count near ties: ("ratio", |u -
ratio|) for every ratio test and ("sample", distance of u*sum(p) to the nearer
of the two cumulative sums bracketing the sampled token, relative to sum(p))
for every inverse-CDF draw.  A zero normaliser after a rejection is recorded
as ("zero_residual", None): an event, not a decision.

For the comparison with an implementation in other arithmetic, the walks take
`flip`, the index of one decision (in trace order) to take the other way: a
ratio test's outcome inverted, or a draw's neighbouring token on the side of
the nearer cumulative sum.  Everything else is unchanged, so a result that
equals the walk with decision k flipped, k a near tie, differs from the
oracle first at that near tie.
"""
import math

import numpy as np

from . import philox
from .status import ST_OK, ST_BAD_TOKEN, ST_BAD_QROW, ST_NONFINITE
from .tree import children_of


# ----------------------------------------------------------------------------
# Target distributions
# ----------------------------------------------------------------------------
def softmax_row(logits_row):
    """P_LLM(.|u) = softmax of one fp32 logits row, float64, temperature 1."""
    l = np.asarray(logits_row, dtype=np.float32).astype(np.float64)
    m = l.max()
    e = np.exp(l - m)
    return e / e.sum()


def argmax_row(logits_row):
    """O(u): the first index of the maximal raw fp32 logit."""
    return int(np.argmax(np.asarray(logits_row, dtype=np.float32)))


def _request_checks(parent_b, token_b, V, q_row_b=None, R=None):
    """Status of one request after the up-front checks, in a fixed order:
    tokens in [0, V), then draft-row indices in [0, R) (padding slots,
    parent -2, are not checked)."""
    nodes = [i for i in range(len(token_b)) if int(parent_b[i]) != -2]
    if any(not (0 <= int(token_b[i]) < V) for i in nodes):
        return ST_BAD_TOKEN
    if q_row_b is not None and any(not (0 <= int(q_row_b[i]) < R) for i in nodes):
        return ST_BAD_QROW
    return ST_OK


def row_ok(logits_row):
    """A visited logits row is usable iff it holds no NaN, no +inf and at least
    one finite value (-inf entries are allowed: probability 0)."""
    l = np.asarray(logits_row, dtype=np.float32)
    return not (np.isnan(l).any() or np.isposinf(l).any() or not np.isfinite(l.max()))


def q_row_ok(q):
    """A draft row read in full is usable iff every entry is finite and >= 0."""
    return bool(np.all(np.isfinite(q)) and np.all(q >= 0.0))


# ----------------------------------------------------------------------------
# VerifyGreedy
# ----------------------------------------------------------------------------
def verify_greedy_one(parent, token, logits):
    """Greedy walk for one request (tokens already checked).

    Returns (accepted node ids, bonus token, status); a visited row that
    fails row_ok stops the walk with status 4."""
    accepted = []
    u = -1
    while True:
        if not row_ok(logits[u + 1]):
            return accepted, -1, ST_NONFINITE
        o = argmax_row(logits[u + 1])
        nxt = None
        for c in children_of(parent, u):
            if int(token[c]) == o:
                nxt = c
                break
        if nxt is None:
            return accepted, o, ST_OK
        accepted.append(nxt)
        u = nxt


def verify_greedy(parent, token, target_logits, status):
    """Batched VerifyGreedy.  Returns dict of accepted [B][N] (-1 padded),
    num_accepted [B], bonus [B], status [B]."""
    B, N = token.shape
    V = target_logits.shape[2]
    acc = np.full((B, N), -1, dtype=np.int64)
    num = np.full(B, -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    st = [int(s) for s in status]
    for b in range(B):
        if st[b] == ST_OK:
            st[b] = _request_checks(parent[b], token[b], V)
        if st[b] != ST_OK:
            continue
        path, bn, s_b = verify_greedy_one(parent[b], token[b], target_logits[b])
        st[b] = s_b
        if s_b != ST_OK:
            continue
        acc[b, : len(path)] = path
        num[b] = len(path)
        bonus[b] = bn
    return dict(accepted=acc, num_accepted=num, bonus=bonus, status=np.array(st))


# ----------------------------------------------------------------------------
# VerifyStochastic: multi-step speculative sampling
# ----------------------------------------------------------------------------
def ratio_of(p_x, q_x):
    """P_LLM(x) / P_SSM(x) with the q(x) = 0 reading."""
    if q_x > 0.0:
        return p_x / q_x
    return math.inf if p_x > 0.0 else 0.0


def residual(p_cur, q):
    """Distribution after rejecting a child proposed from q:
    norm(max(0, p_cur - q)); unchanged if the normaliser is 0.
    Returns (new distribution, normaliser)."""
    r = np.maximum(0.0, p_cur - q)
    z = r.sum()
    if z > 0.0:
        return r / z, z
    return p_cur, z


def sample_from(p_cur, u):
    """Smallest x with sum_{y<=x} p_cur(y) >= u * sum(p_cur).

    Returns (x, margin), margin = distance of the threshold to the nearer of the
    two cumulative sums bracketing x, relative to sum(p_cur)."""
    c = np.cumsum(p_cur)
    total = c[-1]
    t = u * total
    idx = np.nonzero(c >= t)[0]
    if len(idx):
        x = int(idx[0])
    else:
        x = int(np.nonzero(p_cur > 0)[0][-1])
    lo = c[x - 1] if x > 0 else 0.0
    margin = min(abs(t - lo), abs(c[x] - t)) / total if total > 0 else 0.0
    return x, margin


def sample_other(p_cur, u, x):
    """The token a draw at u lands on when the cumulative sum nearer to the
    threshold u*sum(p) falls on its other side: the last token before x with
    nonzero mass (threshold near the sum below x) or the first one after x
    (near the sum at x).  None if there is no such token."""
    c = np.cumsum(p_cur)
    t = u * c[-1]
    lo = c[x - 1] if x > 0 else 0.0
    if abs(t - lo) <= abs(c[x] - t):
        nz = np.nonzero(p_cur[:x] > 0)[0]
        return int(nz[-1]) if len(nz) else None
    nz = np.nonzero(p_cur[x + 1:] > 0)[0]
    return int(x + 1 + nz[0]) if len(nz) else None


def _draw(p_cur, u, trace, flip):
    """One inverse-CDF draw as a traced decision (see `flip` above)."""
    x, margin = sample_from(p_cur, u)
    if len([e for e in trace if e[1] is not None]) == flip:
        alt = sample_other(p_cur, u, x)
        x = x if alt is None else alt
    trace.append(("sample", margin))
    return x


def _ratio_test(u1, ratio, trace, flip):
    """One accept test as a traced decision (see `flip` above)."""
    accept = u1 <= ratio
    if len([e for e in trace if e[1] is not None]) == flip:
        accept = not accept
    trace.append(("ratio", abs(u1 - ratio) if math.isfinite(ratio) else math.inf))
    return accept


def select_child(untested, word0):
    """The random untested child: idx-th in ascending node order."""
    idx = philox.pick_index(word0, len(untested))
    return untested[idx]


def mss_one(b, parent, token, logits, ssm, q_row, seed, offset, flip=None):
    """Multi-step speculative sampling for request b (assumes the data checks
    passed).  Returns (accepted, bonus, rounds, status, trace)."""
    accepted = []
    trace = []
    rounds = 0
    u = -1
    if not row_ok(logits[0]):
        return accepted, -1, rounds, ST_NONFINITE, trace
    p_cur = softmax_row(logits[0])
    while True:
        untested = children_of(parent, u)
        slot = u + 1
        j = 0
        moved = False
        while untested:
            w = philox.words(seed, offset, b, slot, j)
            s = select_child(untested, w[0])
            x = int(token[s])
            qrow = np.asarray(ssm[q_row[s]], dtype=np.float32).astype(np.float64)
            q_x = qrow[x]
            if not math.isfinite(q_x) or q_x < 0.0:
                return accepted, -1, rounds, ST_NONFINITE, trace
            ratio = ratio_of(p_cur[x], q_x)
            u1 = philox.unit_open0(w[1])
            rounds += 1
            if _ratio_test(u1, ratio, trace, flip):
                accepted.append(s)
                u = s
                if not row_ok(logits[s + 1]):
                    return accepted, -1, rounds, ST_NONFINITE, trace
                p_cur = softmax_row(logits[s + 1])
                moved = True
                break
            if not q_row_ok(qrow):
                return accepted, -1, rounds, ST_NONFINITE, trace
            p_new, z = residual(p_cur, qrow)
            if z == 0.0:
                trace.append(("zero_residual", None))
            p_cur = p_new
            untested = [c for c in untested if c != s]
            j += 1
        if moved:
            continue
        # every child rejected, or a leaf reached by acceptance
        w = philox.words(seed, offset, b, slot, 0)
        x = _draw(p_cur, philox.unit_open0(w[2]), trace, flip)
        return accepted, x, rounds, ST_OK, trace


def verify_mss(parent, token, target_logits, ssm_probs, q_row, status, seed, offset=0,
               requests=None, flips=None):
    """Batched MSS verification.  Returns dict of accepted [B][N] (-1 padded),
    num_accepted [B], bonus [B], rounds [B], status [B], traces (list per
    request) and redo(b, k), the same call for request b alone with its
    decision k flipped.  `requests` restricts the work to a subset (others
    stay -1); `flips` maps a request to the decision to flip."""
    B, N = token.shape
    V = target_logits.shape[2]
    R = ssm_probs.shape[1]
    acc = np.full((B, N), -1, dtype=np.int64)
    num = np.full(B, -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    rounds = np.full(B, -1, dtype=np.int64)
    st = [int(s) for s in status]
    traces = [[] for _ in range(B)]
    for b in (range(B) if requests is None else requests):
        if st[b] == ST_OK:
            st[b] = _request_checks(parent[b], token[b], V, q_row[b], R)
        if st[b] != ST_OK:
            continue
        path, bn, rd, s_b, tr = mss_one(b, parent[b], token[b], target_logits[b], ssm_probs[b],
                                        q_row[b], seed, offset, (flips or {}).get(b))
        traces[b] = tr
        st[b] = s_b
        if s_b != ST_OK:
            continue
        acc[b, : len(path)] = path
        num[b] = len(path)
        bonus[b] = bn
        rounds[b] = rd
    return dict(accepted=acc, num_accepted=num, bonus=bonus, rounds=rounds,
                status=np.array(st), traces=traces,
                redo=lambda b, k: verify_mss(parent, token, target_logits, ssm_probs, q_row, status, seed,
                                             offset, requests=[b], flips={b: k}))


# ----------------------------------------------------------------------------
# VerifyStochastic with several proposers per node (merged token trees)
# ----------------------------------------------------------------------------
# When several SSMs propose the same token at the same place, a merged token
# tree holds one node for it (SpecInfer summary, "Token Tree Merge" and the
# multi-SSM remark of VerifyStochastic).  VerifyStochastic tests a child with
# the distribution of the SSM that proposed it; the variant here keeps every
# proposal: a node proposed by m SSMs takes part in m rounds, each with its
# proposer's draft row, exactly as if the m proposals were separate children
# carrying the same token.  Accepting any of them enters the node; rejecting
# one drops only that proposal.  With one proposal per node this is
# VerifyStochastic itself, and for independent draws (one per SSM, each from
# its own distribution) the emitted token follows P_LLM (Theorem 4.2), which
# testing a merged node once does not give.
#
# A request's proposals are slots s = 0..S-1: prop_node[s] is the node
# (-1: unused slot) and prop_row[s] its proposer's row of ssm_probs.  The
# random proposal is the idx-th untested one in ascending slot order, idx as
# for a child; the Philox counter still counts rounds at the node.
def proposals_of(parent, prop_node, u):
    """Slots whose node is a child of u (u = -1: the root), ascending slot order."""
    return [s for s, c in enumerate(prop_node) if int(c) >= 0 and int(parent[int(c)]) == u]


def _proposal_checks(parent_b, token_b, V, prop_node_b, prop_row_b, R):
    """Status after the up-front checks: tokens of the tree's nodes in [0, V),
    then every used slot names a node of the tree (not a padding slot) and a
    draft row in [0, R)."""
    st = _request_checks(parent_b, token_b, V)
    if st != ST_OK:
        return st
    N = len(parent_b)
    for c, r in zip(prop_node_b, prop_row_b):
        c, r = int(c), int(r)
        if c == -1:
            continue
        if not (0 <= c < N) or int(parent_b[c]) == -2 or not (0 <= r < R):
            return ST_BAD_QROW
    return ST_OK


def mss_multi_one(b, parent, token, logits, ssm, prop_node, prop_row, seed, offset, flip=None):
    """VerifyStochastic over proposals for request b (assumes the checks
    passed).  Returns (accepted nodes, bonus, rounds, status, trace) as
    mss_one."""
    accepted = []
    trace = []
    rounds = 0
    u = -1
    if not row_ok(logits[0]):
        return accepted, -1, rounds, ST_NONFINITE, trace
    p_cur = softmax_row(logits[0])
    while True:
        untested = proposals_of(parent, prop_node, u)
        slot = u + 1
        j = 0
        moved = False
        while untested:
            w = philox.words(seed, offset, b, slot, j)
            s = select_child(untested, w[0])
            c = int(prop_node[s])
            x = int(token[c])
            qrow = np.asarray(ssm[prop_row[s]], dtype=np.float32).astype(np.float64)
            q_x = qrow[x]
            if not math.isfinite(q_x) or q_x < 0.0:
                return accepted, -1, rounds, ST_NONFINITE, trace
            ratio = ratio_of(p_cur[x], q_x)
            u1 = philox.unit_open0(w[1])
            rounds += 1
            if _ratio_test(u1, ratio, trace, flip):
                accepted.append(c)
                u = c
                if not row_ok(logits[c + 1]):
                    return accepted, -1, rounds, ST_NONFINITE, trace
                p_cur = softmax_row(logits[c + 1])
                moved = True
                break
            if not q_row_ok(qrow):
                return accepted, -1, rounds, ST_NONFINITE, trace
            p_new, z = residual(p_cur, qrow)
            if z == 0.0:
                trace.append(("zero_residual", None))
            p_cur = p_new
            untested = [t for t in untested if t != s]
            j += 1
        if moved:
            continue
        w = philox.words(seed, offset, b, slot, 0)
        x = _draw(p_cur, philox.unit_open0(w[2]), trace, flip)
        return accepted, x, rounds, ST_OK, trace


def verify_mss_multi(parent, token, target_logits, ssm_probs, prop_node, prop_row, status, seed,
                     offset=0, requests=None, flips=None):
    """Batched VerifyStochastic over proposals; outputs (redo included),
    `requests` and `flips` as verify_mss.  prop_node, prop_row: [B][S] int
    arrays (S <= 64)."""
    B, N = token.shape
    V = target_logits.shape[2]
    R = ssm_probs.shape[1]
    acc = np.full((B, N), -1, dtype=np.int64)
    num = np.full(B, -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    rounds = np.full(B, -1, dtype=np.int64)
    st = [int(x) for x in status]
    traces = [[] for _ in range(B)]
    for b in (range(B) if requests is None else requests):
        if st[b] == ST_OK:
            st[b] = _proposal_checks(parent[b], token[b], V, prop_node[b], prop_row[b], R)
        if st[b] != ST_OK:
            continue
        path, bn, rd, s_b, tr = mss_multi_one(b, parent[b], token[b], target_logits[b], ssm_probs[b],
                                              prop_node[b], prop_row[b], seed, offset, (flips or {}).get(b))
        traces[b] = tr
        st[b] = s_b
        if s_b != ST_OK:
            continue
        acc[b, : len(path)] = path
        num[b] = len(path)
        bonus[b] = bn
        rounds[b] = rd
    return dict(accepted=acc, num_accepted=num, bonus=bonus, rounds=rounds,
                status=np.array(st), traces=traces,
                redo=lambda b, k: verify_mss_multi(parent, token, target_logits, ssm_probs, prop_node, prop_row,
                                                   status, seed, offset, requests=[b], flips={b: k}))


# ----------------------------------------------------------------------------
# Naive sampling verification (Theorem 4.3's comparator)
# ----------------------------------------------------------------------------
def naive_reject_prob(p, child_tokens):
    """Naive verifier: draw x ~ P_LLM and accept iff x is a child token, so it
    rejects with probability 1 - (mass of the distinct child tokens)."""
    toks = sorted(set(int(t) for t in child_tokens))
    return 1.0 - float(sum(p[t] for t in toks))


def naive_one(b, parent, token, logits, seed, offset, flip=None):
    """Naive sampling verification for request b (Theorem 4.3's comparator):
    at node u draw x from P_LLM(.|u); if a child of u carries token x, move to
    the lowest such child, otherwise x is the bonus token and the walk stops.

    Readings: the draw uses the same word as MSS's final sample (word 2 of
    round 0 at u's slot, inverse CDF as in sample_from), and a miss emits the
    drawn token, so every emitted token is distributed as P_LLM given the
    tokens before it; the pages' remark that naive sampling never emits a
    token outside the tree describes a variant that would be biased.
    Returns (accepted, bonus, status, trace)."""
    accepted = []
    trace = []
    u = -1
    while True:
        if not row_ok(logits[u + 1]):
            return accepted, -1, ST_NONFINITE, trace
        p = softmax_row(logits[u + 1])
        w = philox.words(seed, offset, b, u + 1, 0)
        x = _draw(p, philox.unit_open0(w[2]), trace, flip)
        nxt = next((c for c in children_of(parent, u) if int(token[c]) == x), None)
        if nxt is None:
            return accepted, x, ST_OK, trace
        accepted.append(nxt)
        u = nxt


def verify_naive(parent, token, target_logits, status, seed, offset=0, requests=None, flips=None):
    """Batched naive sampling verification; same outputs as verify_greedy plus
    traces and redo, with `requests` and `flips` as verify_mss."""
    B, N = token.shape
    V = target_logits.shape[2]
    acc = np.full((B, N), -1, dtype=np.int64)
    num = np.full(B, -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    st = [int(s) for s in status]
    traces = [[] for _ in range(B)]
    for b in (range(B) if requests is None else requests):
        if st[b] == ST_OK:
            st[b] = _request_checks(parent[b], token[b], V)
        if st[b] != ST_OK:
            continue
        path, bn, s_b, tr = naive_one(b, parent[b], token[b], target_logits[b], seed, offset,
                                      (flips or {}).get(b))
        traces[b] = tr
        st[b] = s_b
        if s_b != ST_OK:
            continue
        acc[b, : len(path)] = path
        num[b] = len(path)
        bonus[b] = bn
    return dict(accepted=acc, num_accepted=num, bonus=bonus, status=np.array(st), traces=traces,
                redo=lambda b, k: verify_naive(parent, token, target_logits, status, seed, offset,
                                               requests=[b], flips={b: k}))
