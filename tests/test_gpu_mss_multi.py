"""tree_verify_mss_multi (VerifyStochastic over proposals, for merged
multi-SSM trees) against the oracle's verify_mss_multi and against
tree_verify_mss, on both walk kernels (one workgroup per request up to
V = 16384, several above; float4 and scalar row loads)."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth
from oracle import exact, verify as o_verify
from tests.gpu_util import DEV, DeviceRun, compare_mss, to_dev

pytestmark = pytest.mark.gpu

SHAPES = {
    "row_c3": (3, dict(B=4, L=20, H=1, V=3000)),
    "row_c1": (1, dict()),
    "sliced_c3": (3, dict(B=3, L=20, H=1, V=20000)),
    "sliced_c3_scalar": (3, dict(B=3, L=20, H=1, V=17003)),
    # on a 256-CU device these take 8 and 16 vocabulary entries per thread
    "sliced_c3_w8": (3, dict(B=12, L=20, H=1, V=40000)),
    "sliced_c3_w16": (3, dict(B=24, L=20, H=1, V=40000)),
}


def _case(*a):
    print("[case]", *a, flush=True)


def _identity(w):
    return (np.where(np.asarray(w.parent) == -2, -1, np.arange(w.N)).astype(np.int32),
            np.asarray(w.q_row, dtype=np.int32))


@pytest.mark.parametrize("name", list(SHAPES))
def test_identity_proposals_equal_mss(name):
    cfg, kw = SHAPES[name]
    _case("multi identity", name)
    w = synth.make_workload(cfg, **kw)
    one = DeviceRun(w).mask().mss()
    pn, pr = _identity(w)
    multi = DeviceRun(w).mask().mss_multi(pn, pr)
    torch.cuda.synchronize()
    for k in ("m_acc", "m_num", "m_bonus", "m_rounds", "status"):
        assert np.array_equal(getattr(one, k).cpu().numpy(), getattr(multi, k).cpu().numpy()), k


def _random_proposals(w, rng, max_per_node=3, S=None):
    """Each node of the tree gets 1..max_per_node proposals from random rows,
    in a shuffled slot order (unused slots -1 at random places)."""
    B, N = w.token.shape
    R = w.ssm_probs.shape[1]
    lists = []
    for b in range(B):
        props = []
        for i in range(N):
            if int(w.parent[b][i]) == -2:
                continue
            for _ in range(int(rng.integers(1, max_per_node + 1))):
                props.append((i, int(rng.integers(0, R))))
        lists.append(props)
    S = S or min(64, max(len(p) for p in lists) + 3)
    pn = np.full((B, S), -1, dtype=np.int32)
    pr = np.zeros((B, S), dtype=np.int32)
    for b, props in enumerate(lists):
        props = props[:S]
        slots = rng.permutation(S)[: len(props)]
        for (i, r), s in zip(props, slots):
            pn[b, s], pr[b, s] = i, r
    return pn, pr


@pytest.mark.parametrize("name", list(SHAPES))
def test_merged_trees_vs_oracle(name):
    cfg, kw = SHAPES[name]
    _case("multi vs oracle", name)
    w = synth.make_workload(cfg, **kw)
    rng = np.random.default_rng(len(name))
    per_node = 3 if w.N <= 21 else 2
    for off in range(3):
        pn, pr = _random_proposals(w, rng, per_node)
        run = DeviceRun(w).mask().mss_multi(pn, pr, offset=w.offset + off)
        torch.cuda.synchronize()
        ref = o_verify.verify_mss_multi(w.parent, w.token, w.target_logits, w.ssm_probs, pn, pr, [0] * w.B,
                                        w.seed, w.offset + off)
        exact_n, excused, bad = compare_mss(run, ref)
        print(f"{name} offset {off}: exact {exact_n}, near-tie {excused}, rounds {run.m_rounds.cpu().numpy().tolist()}")
        assert not bad, bad


def _run_arrays(parent, token, tl, sp, prop_node, prop_row, q_row, seed, multi=True):
    """One call on raw arrays (a workload-free run for distribution tests)."""
    import tree_speculative_verification_attn_amd as tv
    B, N = token.shape
    V = tl.shape[2]
    w = SimpleNamespace(B=B, N=N, V=V, seed=seed, offset=0)
    run = SimpleNamespace(w=w)
    par = to_dev(np.asarray(parent, dtype=np.int32))
    anc = torch.zeros((B, N), dtype=torch.int64, device=DEV)
    child = torch.zeros((B, N + 1), dtype=torch.int64, device=DEV)
    depth = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    run.status = torch.zeros((B,), dtype=torch.int32, device=DEV)
    tv.tree_build_mask(par, anc, child, depth, run.status)
    ws = torch.zeros(tv.tree_verify_workspace(B, N, V), dtype=torch.uint8, device=DEV)
    run.m_acc = torch.empty((B, N), dtype=torch.int32, device=DEV)
    run.m_num = torch.empty((B,), dtype=torch.int32, device=DEV)
    run.m_bonus = torch.empty((B,), dtype=torch.int32, device=DEV)
    run.m_rounds = torch.empty((B,), dtype=torch.int32, device=DEV)
    tl_d, sp_d, tok_d = to_dev(tl), to_dev(sp), to_dev(np.asarray(token, dtype=np.int32))
    if multi:
        tv.tree_verify_mss_multi(tl_d, sp_d, to_dev(prop_node), to_dev(prop_row), tok_d, child, run.status, seed, 0,
                                 run.m_acc, run.m_num, run.m_bonus, run.m_rounds, ws)
    else:
        tv.tree_verify_mss(tl_d, sp_d, to_dev(np.asarray(q_row, dtype=np.int32)), tok_d, child, run.status, seed, 0,
                           run.m_acc, run.m_num, run.m_bonus, run.m_rounds, ws)
    torch.cuda.synchronize()
    return run




def test_merged_trees_distribution():
    # two SSMs with their own distributions, one proposal each, equal tokens
    # merged: every proposal its own round gives P_LLM; one round per node
    # does not (exact bias 0.131 on this case)
    from fractions import Fraction as F
    p = [F(1, 8), F(1, 2), F(3, 8)]
    qs = [[F(3, 4), F(1, 8), F(1, 8)], [F(2, 5), F(8, 15), F(1, 15)]]
    n = 30000
    pf = np.array([float(x) for x in p])
    qf = [np.array([float(x) for x in q]) for q in qs]
    _case("multi distribution", n)
    parent, token, tl, sp, pn, pr, q_row = synth.merged_tree_batch(33, n, pf, qf)
    run = _run_arrays(parent, token, tl, sp, pn, pr, q_row, seed=7)
    num, acc, bonus, st = (t.cpu().numpy() for t in (run.m_num, run.m_acc, run.m_bonus, run.status))
    assert np.all(st == 0)
    first = np.where(num > 0, token[np.arange(n), np.maximum(acc[:, 0], 0)], bonus)
    tv_multi = exact.tv(np.bincount(first, minlength=3) / n, p)
    once = _run_arrays(parent, token, tl, sp, pn, pr, q_row, seed=7, multi=False)
    num1, acc1, bonus1 = (t.cpu().numpy() for t in (once.m_num, once.m_acc, once.m_bonus))
    first1 = np.where(num1 > 0, token[np.arange(n), np.maximum(acc1[:, 0], 0)], bonus1)
    tv_once = exact.tv(np.bincount(first1, minlength=3) / n, p)
    print(f"TV multiplicity {tv_multi:.4f}, once per node {tv_once:.4f}")
    assert tv_multi < 1.5e-2 and tv_once > 8e-2


def test_proposal_status_paths():
    # request 0 fine (with unused slots); 1 a row outside [0, R); 2 a slot on
    # a padding node; 3 a slot naming a node past N; 4 no proposal at all
    _case("multi status")
    w = synth.make_workload(2, B=5, L=20, H=1, V=500)
    B, N = w.token.shape
    R = w.ssm_probs.shape[1]
    parent = np.array(w.parent).copy()
    parent[2, N - 1] = -2                    # make the last node of request 2 padding
    w.parent = parent
    pn, pr = _identity(w)
    pn = np.concatenate([pn, np.full((B, 3), -1, dtype=np.int32)], axis=1)
    pr = np.concatenate([pr, np.zeros((B, 3), dtype=np.int32)], axis=1)
    pr[1, 0] = R
    pn[2, N] = N - 1
    pn[3, N + 1] = N
    pn[4, :] = -1
    run = DeviceRun(w).mask().mss_multi(pn, pr)
    torch.cuda.synchronize()
    st = run.status.cpu().numpy()
    assert st.tolist()[1:4] == [3, 3, 3], st
    ref = o_verify.verify_mss_multi(w.parent, w.token, w.target_logits, w.ssm_probs, pn, pr, [0] * B, w.seed,
                                    w.offset)
    exact_n, excused, bad = compare_mss(run, ref)
    assert not bad, bad
    assert run.m_num.cpu().numpy()[4] == 0   # nothing to test: the root samples the bonus
