"""Pins for the oracle's sampling transforms and naive verification.

Transforms (wiki concept page "Speculative decoding", "Implementation
sketch"; definitions in oracle/sampling.py): checked against independent
constructions -- scipy's softmax, probability ratios under temperature, the
kept set built from "how many entries beat x" ranks instead of a sorted
cumulative sum, and hand-made ties and invalid rows.

Naive verification (SpecInfer summary, Theorem 4.3's comparator): its
root-rejection frequency against the closed form 1 - (mass of the distinct
child tokens), its emitted first token against P_LLM (a draw-then-check rule
that emits the drawn token on a miss is unbiased), and deterministic trees.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import philox, sampling, verify
from oracle.status import ST_NONFINITE, ST_OK


def _beats(l, x):
    """Entries ranked above x: larger value, or equal value and lower index."""
    return [y for y in range(len(l)) if np.isfinite(l[y]) and (l[y] > l[x] or (l[y] == l[x] and y < x))]


def _kept_by_rank(l, T, k, p):
    l = np.asarray(l, dtype=np.float64) / T      # ranks and masses on l / T
    fin = [x for x in range(len(l)) if np.isfinite(l[x])]
    keep = [x for x in fin if k == 0 or len(_beats(l, x)) < k]
    if p < 1.0:
        top = max(l[x] for x in keep)
        m = {x: math.exp(l[x] - top) for x in keep}
        tot = sum(m.values())
        keep = [x for x in keep if sum(m[y] for y in _beats(l, x) if y in m) < p * tot]
    return sorted(keep)


def test_plain_softmax_and_temperature():
    rng = np.random.default_rng(1)
    l = rng.normal(0, 3, 40).astype(np.float32)
    np.testing.assert_allclose(sampling.transform_row(l, kind="probs"), softmax(l.astype(np.float64)),
                               rtol=1e-13, atol=1e-300)
    for T in (0.3, 0.7, 2.5):
        p = sampling.transform_row(l, temperature=T, kind="probs")
        i, j = 3, 17
        # the ratio of two probabilities is exp of the logit difference over T
        assert math.isclose(p[i] / p[j], math.exp((float(l[i]) - float(l[j])) / T), rel_tol=1e-12)
        lg = sampling.transform_row(l, temperature=T, kind="logits")
        assert (lg == l.astype(np.float64) / T).all()
    assert (sampling.transform_row(l, kind="logits") == l.astype(np.float64)).all()
    # low temperature concentrates on the argmax, high temperature flattens
    assert sampling.transform_row(l, temperature=0.01, kind="probs")[int(np.argmax(l))] > 0.999
    assert np.ptp(sampling.transform_row(l, temperature=1e4, kind="probs")) < 1e-3


@pytest.mark.parametrize("seed", range(12))
def test_kept_set_matches_rank_construction(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 60))
    l = np.round(rng.normal(0, 2, V), 1).astype(np.float32)      # rounding makes ties
    l[rng.random(V) < 0.1] = -np.inf
    if not np.isfinite(l).any():
        l[0] = 0.0
    T = float(rng.choice([0.5, 1.0, 1.7]))
    for k in (0, 1, 3, V):
        for p in (1.0, 0.9, 0.5, 0.05):
            got = sorted(sampling.kept_in_rank_order(l, T, k, p))
            assert got == _kept_by_rank(l.astype(np.float64), T, k, p), (k, p)
            probs = sampling.transform_row(l, T, k, p, kind="probs")
            assert math.isclose(probs.sum(), 1.0, rel_tol=1e-12)
            assert set(np.nonzero(probs)[0].tolist()) <= set(got)


def test_ties_invalid_rows_and_extremes():
    l = np.zeros(6, dtype=np.float32)
    assert sampling.kept_in_rank_order(l, 1.0, 3, 1.0) == [0, 1, 2]
    assert sampling.kept_in_rank_order(l, 1.0, 0, 0.5) == [0, 1, 2]      # 3 of 6 equal masses reach 1/2
    assert sampling.kept_in_rank_order(l, 1.0, 0, 0.51) == [0, 1, 2, 3]
    l2 = np.array([1.0, 5.0, 5.0, -np.inf, 2.0], dtype=np.float32)
    assert sampling.kept_in_rank_order(l2, 1.0, 1, 1.0) == [1]
    assert sampling.kept_in_rank_order(l2, 1.0, 10, 1.0) == [1, 2, 4, 0]   # -inf never kept
    p = sampling.transform_row(l2, 1.0, 1, 1.0, kind="probs")
    assert p.tolist() == [0.0, 1.0, 0.0, 0.0, 0.0]
    lg = sampling.transform_row(l2, 2.0, 2, 1.0, kind="logits")
    assert lg.tolist() == [-np.inf, 2.5, 2.5, -np.inf, -np.inf]       # 5 * 0.5 is exact in fp32
    for bad in ([0.0, np.nan], [0.0, np.inf], [-np.inf, -np.inf]):
        assert np.isnan(sampling.transform_row(np.array(bad, dtype=np.float32), kind="probs")).all()
    # the output is fp32: a scaled logit past the fp32 range makes the row
    # invalid (above) or drops the entry (below); up to FLT_MAX it is kept
    assert np.isnan(sampling.transform_row(np.array([3e38, 1.0], dtype=np.float32), 0.5)).all()
    assert sampling.kept_in_rank_order(np.array([-3e38, 1.0], dtype=np.float32), 0.5) == [1]
    big = np.array([1.7e38, 1.0], dtype=np.float32)
    assert sampling.kept_in_rank_order(big, 0.5) == [0, 1]
    assert sampling.transform_row(big, 0.5)[0] == float(big[0]) * 2.0
    # rounding-level ties at the top-k cut are recognised, others are not
    one = np.float32(1.0)
    assert sampling.rounding_tie_at_topk(np.array([one, np.nextafter(one, np.float32(2))]), 1.0, 1)
    assert not sampling.rounding_tie_at_topk(np.array([1.0, 1.5], dtype=np.float32), 0.7, 1)
    assert not sampling.rounding_tie_at_topk(np.array([1.0, 1.0], dtype=np.float32), 1.0, 0)
    # a tiny top-p keeps only the largest entry
    assert sampling.kept_in_rank_order(l2, 1.0, 0, 1e-9) == [1]


# ----------------------------------------------------------------------------
# naive verification
# ----------------------------------------------------------------------------
def _tree_root_children(tokens):
    return np.array([[-1] * len(tokens)], dtype=np.int64), np.array([tokens], dtype=np.int64)


def test_naive_root_rejection_matches_closed_form():
    rng = np.random.default_rng(3)
    V = 12
    logits = rng.normal(0, 1.5, (1, 4, V)).astype(np.float32)
    parent, token = _tree_root_children([4, 9, 4])               # a duplicate sibling token
    p = verify.softmax_row(logits[0, 0])
    want = verify.naive_reject_prob(p, [4, 9, 4])
    n = 20000
    rej = sum(verify.naive_one(0, parent[0], token[0], logits[0], 77, off)[0] == [] for off in range(n))
    sd = math.sqrt(want * (1 - want) / n)
    assert abs(rej / n - want) < 4 * sd
    # and the accepted child of a duplicate token is the lower node
    accs = {tuple(verify.naive_one(0, parent[0], token[0], logits[0], 77, off)[0]) for off in range(200)}
    assert (2,) not in accs


def test_naive_first_token_is_unbiased():
    rng = np.random.default_rng(4)
    V = 8
    logits = rng.normal(0, 1.0, (1, 3, V)).astype(np.float32)
    parent, token = _tree_root_children([1, 6])
    p = verify.softmax_row(logits[0, 0])
    counts = np.zeros(V)
    n = 20000
    for off in range(n):
        acc, bonus, st, _ = verify.naive_one(0, parent[0], token[0], logits[0], 5, off)
        assert st == ST_OK
        counts[token[0, acc[0]] if acc else bonus] += 1
    tv = 0.5 * np.abs(counts / n - p).sum()
    assert tv < 0.02


def test_naive_deterministic_trees_and_status():
    V = 5
    logits = np.full((1, 4, V), -np.inf, dtype=np.float32)
    logits[0, 0, 2] = 0.0              # root: token 2 surely
    logits[0, 1, 0] = 0.0              # node 0 (token 2): token 0 surely
    logits[0, 2, 3] = 0.0              # node 1 (token 0): token 3 surely, not in the tree
    logits[0, 3, :] = 0.0
    parent = np.array([[-1, 0, -1]])
    token = np.array([[2, 0, 4]])
    out = verify.verify_naive(parent, token, logits, [0], seed=1)
    assert out["accepted"][0, :2].tolist() == [0, 1] and out["num_accepted"][0] == 2
    assert out["bonus"][0] == 3 and out["status"][0] == ST_OK
    logits[0, 1, 0] = np.nan
    out = verify.verify_naive(parent, token, logits, [0], seed=1)
    assert out["status"][0] == ST_NONFINITE and out["num_accepted"][0] == -1
