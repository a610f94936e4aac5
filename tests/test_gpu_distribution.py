"""Distribution tests of the GPU MSS kernel (Theorem 4.2 of the SpecInfer
summary): one launch over 10^6 tiny requests, each a star of three i.i.d.
draft children over V = 8, must give a first-token histogram within total
variation 5e-3 of the target distribution; a fixed (deterministic top-2)
tree must match its exact enumerated distribution instead."""
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import synth
from oracle import exact

pytestmark = pytest.mark.gpu

P8 = [F(x, 100) for x in [5, 10, 15, 20, 5, 25, 10, 10]]
Q8 = [F(x, 100) for x in [30, 5, 5, 10, 25, 5, 15, 5]]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(parent, tok, tl, sp, qr, seed):
    import tree_speculative_verification_attn_amd as tv
    from tests.gpu_util import to_dev
    n, N = tok.shape
    par = to_dev(np.tile(parent.astype(np.int32), (n, 1)))
    anc = torch.zeros((n, N), dtype=torch.int64, device="cuda:0")
    child = torch.zeros((n, N + 1), dtype=torch.int64, device="cuda:0")
    depth = torch.zeros((n, N), dtype=torch.int32, device="cuda:0")
    st = torch.zeros((n,), dtype=torch.int32, device="cuda:0")
    tv.tree_build_mask(par, anc, child, depth, st)
    acc = torch.empty((n, N), dtype=torch.int32, device="cuda:0")
    num = torch.empty((n,), dtype=torch.int32, device="cuda:0")
    bonus = torch.empty((n,), dtype=torch.int32, device="cuda:0")
    ws = torch.zeros(tv.tree_verify_workspace(n, N, tl.shape[2]), dtype=torch.uint8, device="cuda:0")  # zero before first use
    tok_d = to_dev(tok.astype(np.int32))
    tv.tree_verify_mss(to_dev(tl), to_dev(sp), to_dev(qr), tok_d, child, st, seed, 0, acc, num, bonus,
                       None, ws)
    torch.cuda.synchronize()
    assert int((st != 0).sum()) == 0
    first = torch.where(num > 0, torch.gather(tok_d, 1, acc[:, :1].clamp(min=0).long()).squeeze(1), bonus)
    return first.cpu().numpy(), num.cpu().numpy()


def test_tv_iid_children_million():
    n = 1_000_000
    p = np.array([float(x) for x in P8])
    q = np.array([float(x) for x in Q8])
    print("[case] TV iid star3 V=8 n=1e6", flush=True)
    parent, tok, tl, sp, qr = synth.iid_tree_batch(4242, n, p, q, "star3")
    first, num = _run(parent, tok, tl, sp, qr, seed=99)
    hist = np.bincount(first, minlength=8) / n
    tv_ = exact.tv(hist, P8)
    print(f"TV(first token, P_LLM) = {tv_:.2e}; accept rate {np.mean(num > 0):.3f}")
    assert tv_ < 5e-3
    # acceptance probability agrees with the exact enumeration
    acc_exact = float(exact.accept_prob_first_level(P8, Q8, 3))
    assert abs(np.mean(num > 0) - acc_exact) < 3e-3


def test_fixed_tree_matches_enumeration():
    n = 400_000
    p = [F(3, 10), F(3, 10), F(4, 10)]
    q = [F(6, 10), F(3, 10), F(1, 10)]
    print("[case] TV fixed top-2 V=3", flush=True)
    tl = np.broadcast_to(np.log(np.array([0.3, 0.3, 0.4])).astype(np.float32), (n, 3, 3)).copy()
    sp = np.broadcast_to(np.array([0.6, 0.3, 0.1], dtype=np.float32), (n, 1, 3)).copy()
    tok = np.tile(np.array([0, 1], dtype=np.int32), (n, 1))
    qr = np.zeros((n, 2), dtype=np.int32)
    first, _ = _run(np.array([-1, -1]), tok, tl, sp, qr, seed=5)
    hist = np.bincount(first, minlength=3) / n
    want = exact.node_output_dist(p, [(0, q), (1, q)])
    assert exact.tv(hist, want) < 5e-3
    assert exact.tv(hist, p) > 0.04          # and it is not P_LLM (fixed tree)
