"""tree_verify_mss_noalloc, whose workspace is the library's fixed device
array, against tree_verify_mss with a caller's workspace.

Two calls in a row through the C-ABI, the second on a smaller input (fewer
requests, a smaller vocabulary, another tree), each on the sliced walk
(V > 16384) that exchanges values through the workspace: every output of the
fixed-scratch call must equal the workspace call's bit for bit (the same
kernels on the same inputs), and both must match the oracle exactly or at a
near tie of its walk.  A third call after a call that timed out checks that
the shared array is left zero by a walk that gave up.  Requests skipped
upstream keep their status in every call."""
import os

import numpy as np
import pytest
import torch

import synth
import tree_speculative_verification_attn_amd as tv
from oracle import verify as o_verify
from tests.gpu_util import DEV, DeviceRun, compare_mss

pytestmark = pytest.mark.gpu


def _case(*a):
    print("[case]", *a, flush=True)


def _noalloc(run):
    """The fixed-scratch call on run's inputs, from the status the masks left."""
    w = run.w
    out = dict(acc=torch.full((w.B, w.N), -7, dtype=torch.int32, device=DEV),
               num=torch.full((w.B,), -7, dtype=torch.int32, device=DEV),
               bonus=torch.full((w.B,), -7, dtype=torch.int32, device=DEV),
               rounds=torch.full((w.B,), -7, dtype=torch.int32, device=DEV),
               status=run.status.clone())
    tv.tree_verify_mss_noalloc(run.tl, run.sp, run.qr, run.token, run.child, out["status"], w.seed, w.offset,
                               out["acc"], out["num"], out["bonus"], out["rounds"])
    return out


def _check_pair(w, skipped):
    run = DeviceRun(w).mask()
    for b in skipped:
        run.status[b] = 1                  # skipped upstream: keeps its own status
    na = _noalloc(run)                      # fixed scratch first, then the caller's workspace
    run.mss()
    torch.cuda.synchronize()
    for k, ref in (("acc", run.m_acc), ("num", run.m_num), ("bonus", run.m_bonus), ("rounds", run.m_rounds),
                   ("status", run.status)):
        assert torch.equal(na[k], ref), f"{k} differs from tree_verify_mss"
    st = run.status.cpu().numpy()
    assert all(st[b] == 1 for b in skipped)
    status_in = [1 if b in skipped else 0 for b in range(w.B)]
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, status_in, w.seed,
                              w.offset)
    exact, excused, bad = compare_mss(run, ref)
    assert not bad, f"requests {bad} differ from the oracle"
    assert exact + excused == w.B
    return run


def test_noalloc_matches_workspace_call_twice():
    _case("noalloc: B=24 V=40000 (first), then B=5 V=20000 (smaller)")
    _check_pair(synth.make_workload(2, B=24, L=40, H=2, V=40000), skipped=[3])
    _check_pair(synth.make_workload(3, seed=7, B=5, L=24, H=2, V=20000), skipped=[0])


def test_noalloc_after_a_timed_out_walk():
    _case("noalloc: timed-out walk, then a normal call on the same array")
    w = synth.make_workload(2, B=6, L=40, H=2, V=40000)
    run = DeviceRun(w).mask()
    os.environ["TREEVERIFY_WALK_WAIT_POLLS"] = "0"
    try:
        timed = _noalloc(run)
        torch.cuda.synchronize()
    finally:
        del os.environ["TREEVERIFY_WALK_WAIT_POLLS"]
    assert np.all(timed["status"].cpu().numpy() == 9)
    assert np.all(timed["num"].cpu().numpy() == -1)
    _check_pair(w, skipped=[])


def test_noalloc_rejects_more_than_the_scratch():
    _case("noalloc: oversize request count")
    B, N, V = 1261, 4, 32000
    assert tv.tree_verify_workspace(B, N, V) > tv.TV_NOALLOC_SCRATCH_BYTES
    tl = torch.zeros((B, N + 1, V), dtype=torch.float32, device=DEV)
    sp = torch.zeros((B, 1, V), dtype=torch.float32, device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    with pytest.raises(tv.TreeVerifyError, match="fixed scratch"):
        tv.tree_verify_mss_noalloc(tl, sp, torch.zeros((B, N), **i32), torch.zeros((B, N), **i32),
                                   torch.zeros((B, N + 1), dtype=torch.int64, device=DEV),
                                   torch.zeros((B,), **i32), 1, 0, torch.zeros((B, N), **i32),
                                   torch.zeros((B,), **i32), torch.zeros((B,), **i32), torch.zeros((B,), **i32))
