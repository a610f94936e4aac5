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
