"""Pins of the multiplicity variant of VerifyStochastic (oracle side):
several SSMs propose the same token, the merged node keeps every proposal as
a round of its own with its proposer's draft row.

  * with one proposal per node it is VerifyStochastic: verify_mss_multi with
    the identity proposal list equals verify_mss on every workload shape,
    output for output and trace for trace;
  * Theorem 4.2 on merged trees: with independent draws, one per SSM, each
    from its own distribution, the emitted token follows P_LLM exactly
    (exact enumeration over fractions), while testing a merged node once
    (each node with its first proposer's row) does not;
  * the sampled oracle on such trees matches the target distribution, and
    the test separates it from the once-per-node rule;
  * on a fixed merged tree the sampled frequencies match the exact node
    distribution of its proposal list;
  * the up-front checks of the proposal lists."""
from fractions import Fraction as F

import numpy as np
import pytest

import synth
from oracle import exact, verify
from oracle.status import ST_BAD_QROW, ST_BAD_TOKEN, ST_OK


def _rand_dist(rng, V, zeros=0):
    w = [int(x) for x in rng.integers(1, 20, size=V)]
    for z in rng.choice(V, size=zeros, replace=False):
        w[z] = 0
    s = sum(w)
    return [F(x, s) for x in w]


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(B=3, L=40, H=1, V=300)), (3, dict(B=3, L=20, H=1, V=257)),
                                    (4, dict(B=2, H=1, V=200)), (5, dict(B=2, L=50, H=1, V=100))])
def test_identity_proposals_equal_mss(cfg, kw):
    w = synth.make_workload(cfg, **kw)
    B, N = w.token.shape
    st = [0] * B
    ref = verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, st, w.seed, w.offset)
    prop_node = np.where(np.asarray(w.parent) == -2, -1, np.arange(N)).astype(np.int32)   # padding: unused
    got = verify.verify_mss_multi(w.parent, w.token, w.target_logits, w.ssm_probs, prop_node, w.q_row, st,
                                  w.seed, w.offset)
    for key in ("accepted", "num_accepted", "bonus", "rounds", "status"):
        assert np.array_equal(ref[key], got[key]), key
    assert ref["traces"] == got["traces"]


def test_theorem_4_2_merged_trees_exact():
    rng = np.random.default_rng(11)
    worst_once = 0.0
    for trial in range(24):
        V = int(rng.integers(2, 5))
        k = int(rng.integers(2, 4))
        p = _rand_dist(rng, V, zeros=trial % 2)
        qs = [_rand_dist(rng, V, zeros=(trial // 2) % 2) for _ in range(k)]
        assert exact.multi_marginal(p, qs) == p
        worst_once = max(worst_once, exact.tv(exact.multi_marginal(p, qs, dedup=True), p))
    assert worst_once > 0.05


# a case where testing a merged node once is far from the target
P_M = [F(1, 8), F(1, 2), F(3, 8)]
Q_M = [[F(3, 4), F(1, 8), F(1, 8)], [F(2, 5), F(8, 15), F(1, 15)]]


def test_merged_case_exact_bias():
    assert exact.multi_marginal(P_M, Q_M) == P_M
    assert exact.tv(exact.multi_marginal(P_M, Q_M, dedup=True), P_M) > 0.12


def _first(res, token, b):
    if res["num_accepted"][b] > 0:
        return int(token[b][res["accepted"][b][0]])
    return int(res["bonus"][b])


def test_sampled_merged_trees_match_target():
    n = 30000
    p = np.array([float(x) for x in P_M])
    qs = [np.array([float(x) for x in q]) for q in Q_M]
    parent, token, tl, sp, prop_node, prop_row, q_row = synth.merged_tree_batch(21, n, p, qs)
    st = [0] * n
    res = verify.verify_mss_multi(parent, token, tl, sp, prop_node, prop_row, st, seed=5)
    assert np.all(res["status"] == ST_OK)
    hist = np.bincount([_first(res, token, b) for b in range(n)], minlength=3) / n
    tv_multi = exact.tv(hist, P_M)
    once = verify.verify_mss(parent, token, tl, sp, q_row, st, seed=5)
    hist_once = np.bincount([_first(once, token, b) for b in range(n)], minlength=3) / n
    tv_once = exact.tv(hist_once, P_M)
    want_once = exact.multi_marginal(P_M, Q_M, dedup=True)
    print(f"TV multiplicity {tv_multi:.4f}, once per node {tv_once:.4f} (exact {exact.tv(want_once, P_M):.4f})")
    assert tv_multi < 1.5e-2
    assert tv_once > 8e-2
    assert exact.tv(hist_once, want_once) < 1.5e-2


def test_sampled_fixed_merged_tree_matches_exact():
    # root children: node 0 (token 0, proposed by SSMs 0 and 1), node 1
    # (token 2, proposed by SSM 1); proposal order = slot order
    p = [F(2, 10), F(5, 10), F(3, 10)]
    q0 = [F(6, 10), F(2, 10), F(2, 10)]
    q1 = [F(3, 10), F(1, 10), F(6, 10)]
    want = exact.node_output_dist(p, [(0, q0), (0, q1), (2, q1)])
    n = 30000
    parent = np.tile(np.array([-1, -1], dtype=np.int32), (n, 1))
    token = np.tile(np.array([0, 2], dtype=np.int32), (n, 1))
    tl = np.broadcast_to(np.log(np.array([float(x) for x in p])).astype(np.float32), (n, 3, 3)).copy()
    sp = np.broadcast_to(np.array([[float(x) for x in q0], [float(x) for x in q1]], dtype=np.float32),
                         (n, 2, 3)).copy()
    prop_node = np.tile(np.array([0, 0, 1], dtype=np.int32), (n, 1))
    prop_row = np.tile(np.array([0, 1, 1], dtype=np.int32), (n, 1))
    res = verify.verify_mss_multi(parent, token, tl, sp, prop_node, prop_row, [0] * n, seed=9)
    hist = np.bincount([_first(res, token, b) for b in range(n)], minlength=3) / n
    assert exact.tv(hist, want) < 1.5e-2
    # the node's second proposal is tested only after its first was rejected:
    # some requests take three rounds
    assert res["rounds"].max() == 3


def test_deeper_merged_node_is_entered_once_per_path():
    # a merged node with a child: accepting either proposal enters node 0,
    # and the walk continues from node 0's own row with node 2's proposals
    rng = np.random.default_rng(4)
    V = 6
    parent = np.array([[-1, -1, 0]], dtype=np.int32)
    token = np.array([[1, 3, 4]], dtype=np.int32)
    tl = rng.normal(size=(1, 4, V)).astype(np.float32)
    sp = rng.dirichlet(np.ones(V), size=(1, 3)).astype(np.float32)
    prop_node = np.array([[0, 0, 1, 2, -1]], dtype=np.int32)
    prop_row = np.array([[0, 1, 2, 2, 0]], dtype=np.int32)
    seen = set()
    for off in range(300):
        r = verify.verify_mss_multi(parent, token, tl, sp, prop_node, prop_row, [0], seed=3, offset=off)
        assert r["status"][0] == ST_OK
        path = tuple(r["accepted"][0][: r["num_accepted"][0]].tolist())
        assert path in {(), (0,), (1,), (0, 2)}
        seen.add(path)
        assert r["rounds"][0] <= 4
    assert (0, 2) in seen and () in seen


def test_proposal_checks():
    parent = np.array([[-1, 0, -2]], dtype=np.int32)
    token = np.array([[1, 2, 0]], dtype=np.int32)
    tl = np.zeros((1, 4, 5), dtype=np.float32)
    sp = np.full((1, 2, 5), 0.2, dtype=np.float32)

    def st(pn, pr, tok=token):
        return int(verify.verify_mss_multi(parent, tok, tl, sp, np.array([pn], dtype=np.int32),
                                           np.array([pr], dtype=np.int32), [0], seed=1)["status"][0])
    assert st([0, 1, -1], [0, 1, 0]) == ST_OK
    assert st([0, 1, -1], [0, 2, 0]) == ST_BAD_QROW         # row outside [0, R)
    assert st([0, 2, -1], [0, 1, 0]) == ST_BAD_QROW         # a padding slot
    assert st([0, 3, -1], [0, 1, 0]) == ST_BAD_QROW         # not a node
    assert st([0, 1, -3], [0, 1, 0]) == ST_BAD_QROW         # only -1 marks an unused slot
    assert st([0, 1, -1], [0, 1, 0], np.array([[1, 9, 0]], dtype=np.int32)) == ST_BAD_TOKEN
    assert st([-1, -1, -1], [0, 0, 0]) == ST_OK             # nothing proposed: the root samples
