"""The sliced walk's time-out path, forced from the host.

Workgroups of a sliced walk (V > 16384) exchange values through the
workspace, and every wait for another workgroup is bounded.  The bound is
read from TREEVERIFY_WALK_WAIT_POLLS at each call; 0 makes every wait give
up at its first look, so every request times out at its first exchange
without any kernel hanging.  Checked: each request reports TV_REQ_TIMEOUT
with the outputs of a skipped request (num_accepted, bonus and rounds -1, no
accepted node), the fused MSS + commit moves nothing and leaves the prefix
lengths alone, the workspace is left all zero, and the next call with the
normal bound on the same workspace matches the oracle exactly."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import verify as o_verify
from tests.gpu_util import DeviceRun, compare_mss

pytestmark = pytest.mark.gpu

TIMEOUT = 9


def _case(*a):
    print("[case]", *a, flush=True)


@pytest.fixture
def no_wait():
    os.environ["TREEVERIFY_WALK_WAIT_POLLS"] = "0"
    yield
    del os.environ["TREEVERIFY_WALK_WAIT_POLLS"]


def _raw(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("mode", ["greedy", "mss", "naive", "mss_commit"])
def test_walk_times_out_cleanly(mode, no_wait):
    _case("walk timeout", mode)
    w = synth.make_workload(2, B=4, L=40, H=2, V=40000)
    run = DeviceRun(w).mask()
    run.status[1] = 1                          # skipped upstream: keeps its own status
    k0, v0, pl0 = _raw(run.k), _raw(run.v), run.pl.cpu().numpy()
    getattr(run, mode)()
    torch.cuda.synchronize()
    st = run.status.cpu().numpy()
    assert list(st) == [TIMEOUT, 1, TIMEOUT, TIMEOUT]
    pre = "n" if mode == "naive" else ("g" if mode == "greedy" else "m")
    acc, num, bonus = (getattr(run, f"{pre}_{x}").cpu().numpy() for x in ("acc", "num", "bonus"))
    assert np.all(num == -1) and np.all(bonus == -1) and np.all(acc == -1)
    if pre == "m":
        assert np.all(run.m_rounds.cpu().numpy() == -1)
    assert int(run.ws_v.count_nonzero()) == 0, "workspace not left zero"
    if mode == "mss_commit":
        assert np.array_equal(run.pl.cpu().numpy(), pl0)
        assert np.array_equal(_raw(run.k), k0) and np.array_equal(_raw(run.v), v0)


def test_normal_bound_after_timeouts():
    """After timed-out calls, the same workspace serves a normal call."""
    w = synth.make_workload(2, B=4, L=40, H=2, V=40000)
    run = DeviceRun(w).mask()
    os.environ["TREEVERIFY_WALK_WAIT_POLLS"] = "0"
    try:
        run.mss()
        torch.cuda.synchronize()
    finally:
        del os.environ["TREEVERIFY_WALK_WAIT_POLLS"]
    assert list(run.status.cpu().numpy()) == [TIMEOUT] * 4
    run.status.zero_()
    run.mss()
    torch.cuda.synchronize()
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B, w.seed, w.offset)
    exact, excused, bad = compare_mss(run, ref)
    assert not bad and exact + excused == w.B
    assert int(run.ws_v.count_nonzero()) == 0


def test_commit_without_every_report_times_out():
    """The fused MSS + commit grows a request's prefix length only when every
    walking workgroup reports its block of heads moved.  A report of "not
    moved" is planted from the host for requests 0 and 2 (the reports word is
    word 6 of the request's 256-byte line at the start of the workspace), so
    workgroup 0 of those requests gives up once the count is complete, while
    requests 1 and 3 commit as usual.  Checked: the planted requests report
    TV_REQ_TIMEOUT with a skipped request's outputs and their prefix lengths
    unchanged; every row of the caches is either as before or as the normal
    call leaves it; the other requests equal the normal call; the workspace is
    left all zero."""
    _case("commit reports incomplete")
    w = synth.make_workload(2, B=4, L=40, H=5, V=40000)
    ref = DeviceRun(w).mask()
    ref.mss_commit()
    run = DeviceRun(w).mask()
    torch.cuda.synchronize()
    k0, v0, pl0 = _raw(run.k), _raw(run.v), run.pl.cpu().numpy()
    words = run._ws_verify().view(torch.int32)
    for b in (0, 2):
        words[b * 64 + 6] = 0x10000
    run.mss_commit()
    torch.cuda.synchronize()
    st_ref = ref.status.cpu().numpy()
    assert list(st_ref) == [0] * 4
    assert list(run.status.cpu().numpy()) == [TIMEOUT, 0, TIMEOUT, 0]
    pl_ref = ref.pl.cpu().numpy()
    assert (pl_ref[[0, 2]] > pl0[[0, 2]]).any(), "the case should grow a planted request's prefix"
    assert np.array_equal(run.pl.cpu().numpy(), [pl0[0], pl_ref[1], pl0[2], pl_ref[3]])
    for name in ("m_num", "m_bonus", "m_rounds"):
        got, exp = getattr(run, name).cpu().numpy(), getattr(ref, name).cpu().numpy()
        assert np.all(got[[0, 2]] == -1) and np.array_equal(got[[1, 3]], exp[[1, 3]]), name
    acc, acc_ref = run.m_acc.cpu().numpy(), ref.m_acc.cpu().numpy()
    assert np.all(acc[[0, 2]] == -1) and np.array_equal(acc[[1, 3]], acc_ref[[1, 3]])
    for got, pre, exp in ((_raw(run.k), k0, _raw(ref.k)), (_raw(run.v), v0, _raw(ref.v))):
        same_pre = np.all(got == pre, axis=(2, 3))
        same_ref = np.all(got == exp, axis=(2, 3))
        assert np.all(same_pre | same_ref), "a (block, head) slab is neither as before nor committed"
    assert int(run.ws_v.count_nonzero()) == 0, "workspace not left zero"
