"""MSS walks driven through long runs of one outcome, on both walk kernels
(one workgroup per request, and rows sliced over workgroups), against the
oracle.

- Draft equals target: every node's draft row is the target distribution at
  that node, so p(x) / q(x) = 1 and every test accepts ([SpecInfer]
  "Multi-Step Speculative Sampling": acceptance with probability
  min(1, p/q)); the walk goes down to a leaf, and the next pass's candidate
  always comes from the accepted child.
- Children starved: the target gives every child's token about e^-60 of the
  mass at its parent, so every test rejects; the walk runs through all of the
  root's children one round after another and draws the bonus from the
  residual at the root.

tree_verify_mss_commit must return the same path as tree_verify_mss."""
import numpy as np
import pytest
import torch

import synth
from oracle import verify as o_verify
from tests.gpu_util import DeviceRun, compare_mss

pytestmark = pytest.mark.gpu

SHAPES = {
    "row": dict(B=3, L=20, H=1, V=3000),
    "sliced": dict(B=3, L=20, H=1, V=40000),
}
SEEDS = (11, 12, 13, 14)


def _softmax32(x):
    z = np.exp(x.astype(np.float64) - np.max(x))
    return (z / z.sum()).astype(np.float32)


def _children(parent_b, u):
    return [i for i, p in enumerate(parent_b) if p == u]


def _check(w, expect):
    run = DeviceRun(w).mask()
    fus = DeviceRun(w).mask()
    for seed in SEEDS:
        print(f"[case] walk extremes B={w.B} V={w.V} seed={seed}", flush=True)
        run.mss(seed=seed)
        fus.mss_commit(seed=seed)
        torch.cuda.synchronize()
        ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B, seed,
                                  w.offset)
        exact, excused, bad = compare_mss(run, ref)
        assert not bad, (seed, bad)
        for name in ("m_acc", "m_num", "m_bonus", "m_rounds"):
            a, b = getattr(run, name).cpu().numpy(), getattr(fus, name).cpu().numpy()
            if name == "m_acc":
                n = run.m_num.cpu().numpy()
                a = [a[r][:max(n[r], 0)].tolist() for r in range(w.B)]
                b = [b[r][:max(n[r], 0)].tolist() for r in range(w.B)]
                assert a == b, (seed, name)
            else:
                assert np.array_equal(a, b), (seed, name, a, b)
        expect(run, seed)
        # restore the prefix lengths the commit advanced, for the next seed
        fus = DeviceRun(w).mask()


@pytest.mark.parametrize("shape", list(SHAPES))
def test_draft_equals_target_accepts_to_a_leaf(shape):
    w = synth.make_workload(2, **SHAPES[shape])
    assert w.R == w.N + 1
    for b in range(w.B):
        assert np.array_equal(w.q_row[b], np.asarray(w.parent[b]) + 1)
        for r in range(w.N + 1):             # row u + 1: the draft at node u is the target at u
            w.ssm_probs[b, r] = _softmax32(w.target_logits[b, r])

    def expect(run, seed):
        num = run.m_num.cpu().numpy()
        acc = run.m_acc.cpu().numpy()
        rounds = run.m_rounds.cpu().numpy()
        for b in range(w.B):
            assert num[b] >= 1 and rounds[b] == num[b], (seed, b, num[b], rounds[b])
            assert not _children(w.parent[b], acc[b][num[b] - 1]), "the walk stopped above a leaf"

    _check(w, expect)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_starved_children_reject_every_round(shape):
    w = synth.make_workload(2, **SHAPES[shape])
    for b in range(w.B):
        for u in range(-1, w.N):
            row = w.target_logits[b, u + 1]
            top = np.max(row)
            for c in _children(w.parent[b], u):
                row[w.token[b][c]] = top - 60.0

    def expect(run, seed):
        num = run.m_num.cpu().numpy()
        rounds = run.m_rounds.cpu().numpy()
        for b in range(w.B):
            assert num[b] == 0 and rounds[b] == len(_children(w.parent[b], -1)), (seed, b, num[b], rounds[b])

    _check(w, expect)
