"""Exact output distributions of multi-step speculative sampling (oracle side).

Instead of drawing random numbers, these functions sum over every random
choice the verifier makes at one node (which untested child is picked, accept
or reject) and return the exact distribution of the token the node emits:
the accepted child's token, or a draw from the final residual.  With
fractions.Fraction inputs the arithmetic is exact.

They encode the rule of VerifyStochastic (SpecInfer summary, section "Token
Verification: Stochastic Decoding and Multi-Step Speculative Sampling") and
are used to check two statements from the same page:
  * Theorem 4.2: the emitted token follows P_LLM.  It holds when the children
    are independent draws from the draft distribution with duplicates kept as
    separate nodes (iid_marginal); it does not hold for a fixed child set.
  * Theorem 4.3: the probability that every child is rejected is at most the
    naive verifier's rejection probability, 1 - P_LLM(child tokens).
  * merged trees (several SSMs proposing one token): Theorem 4.2 holds when
    every proposal keeps its own round (multi_marginal), not when the merged
    node is tested once.
The single-child case is classic speculative sampling (wiki concept page
"Speculative decoding", "Shared invariant"; the single-draft proof in "How
Speculative Decoding in LLM Serving Actually Works", "Exact Proof of
Distributional Invariance").
"""
from fractions import Fraction
from itertools import product


def _ratio_accept(p_x, q_x):
    """min(1, p/q) with q = 0 giving 1 if p > 0 else 0."""
    if q_x > 0:
        r = p_x / q_x
        return r if r < 1 else type(r)(1)
    return 1 if p_x > 0 else 0


def _residual(p, q):
    r = [max(0, a - b) for a, b in zip(p, q)]
    z = sum(r)
    if z > 0:
        return tuple(x / z for x in r)
    return tuple(p)


def node_output_dist(p, children):
    """Exact distribution of the token emitted at a node.

    p: target distribution (sequence), children: list of (token, q) where q is
    the proposing draft distribution.  Returns a list of probabilities."""
    V = len(p)

    def rec(pc, untested):
        if not untested:
            return list(pc)
        out = [0] * V
        w = Fraction(1, len(untested)) if isinstance(pc[0], Fraction) else 1.0 / len(untested)
        for s in untested:
            tok, q = children[s]
            a = _ratio_accept(pc[tok], q[tok])
            out[tok] += w * a
            if a != 1:
                rest = rec(_residual(pc, q), tuple(c for c in untested if c != s))
                for x in range(V):
                    out[x] += w * (1 - a) * rest[x]
        return out

    return rec(tuple(p), tuple(range(len(children))))


def all_reject_prob(p, children):
    """Exact probability that every child of the node is rejected."""
    def rec(pc, untested):
        if not untested:
            return 1
        w = Fraction(1, len(untested)) if isinstance(pc[0], Fraction) else 1.0 / len(untested)
        tot = 0
        for s in untested:
            tok, q = children[s]
            a = _ratio_accept(pc[tok], q[tok])
            if a != 1:
                tot += w * (1 - a) * rec(_residual(pc, q), tuple(c for c in untested if c != s))
        return tot

    return rec(tuple(p), tuple(range(len(children))))


def iid_marginal(p, q, k):
    """Distribution of the emitted token when the node's k children are
    independent draws from q (duplicates kept), averaged over the draws."""
    V = len(p)
    out = [0] * V
    for draw in product(range(V), repeat=k):
        w = 1
        for x in draw:
            w = w * q[x]
        if w == 0:
            continue
        d = node_output_dist(p, [(x, q) for x in draw])
        for x in range(V):
            out[x] += w * d[x]
    return out


def accept_prob_first_level(p, q, k):
    """Probability that some child is accepted when the k children are
    independent draws from q."""
    tot = 0
    for draw in product(range(len(p)), repeat=k):
        w = 1
        for x in draw:
            w = w * q[x]
        if w == 0:
            continue
        tot += w * (1 - all_reject_prob(p, [(x, q) for x in draw]))
    return tot


def multi_marginal(p, qs, dedup=False):
    """Distribution of the emitted token when SSM i proposes one token drawn
    from its own distribution qs[i] (independent draws), averaged over the
    draws.  Equal tokens are merged into one node:
      * dedup=False: every proposal takes part as its own round with its
        proposer's q (the multiplicity variant);
      * dedup=True: the merged node is tested once, with the q of its
        lowest-numbered proposer."""
    V = len(p)
    out = [0] * V
    for draw in product(range(V), repeat=len(qs)):
        w = 1
        for i, x in enumerate(draw):
            w = w * qs[i][x]
        if w == 0:
            continue
        if dedup:
            first = {}
            for i, x in enumerate(draw):
                first.setdefault(x, i)
            props = [(x, qs[i]) for x, i in sorted(first.items(), key=lambda t: t[1])]
        else:
            props = [(x, qs[i]) for i, x in enumerate(draw)]
        d = node_output_dist(p, props)
        for x in range(V):
            out[x] += w * d[x]
    return out


def tv(a, b):
    """Total variation distance between two distributions."""
    return 0.5 * sum(abs(float(x) - float(y)) for x, y in zip(a, b))
