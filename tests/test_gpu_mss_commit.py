"""tree_verify_mss_commit against tree_verify_mss followed by
kv_commit_accepted: every output, the status codes, the prefix lengths and
the whole K/V caches must be identical bit for bit (the fused call promises
exactly the results of the two calls in sequence), on both walk kernels
(one workgroup per request up to V = 16384, sliced above), bf16 and fp32
caches, and the status paths of both halves.  The MSS results are also
checked against the oracle, and the compaction against the oracle's."""
import numpy as np
import pytest
import torch

import synth
from oracle import commit as o_commit
from oracle import verify as o_verify
from tests.gpu_util import DeviceRun, compare_mss

pytestmark = pytest.mark.gpu


def _case(*a):
    print("[case]", *a, flush=True)


def _raw(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _run_both(w, mutate=None, seed=None, offset=None):
    seq = DeviceRun(w).mask()
    fus = DeviceRun(w).mask()
    if mutate:
        mutate(seq)
        mutate(fus)
    torch.cuda.synchronize()
    st_mask = seq.status.cpu().numpy().copy()
    seq.mss(seed, offset)
    torch.cuda.synchronize()
    st_verify = seq.status.cpu().numpy().copy()
    seq.commit(seq.m_acc, seq.m_num)
    fus.mss_commit(seed, offset)
    torch.cuda.synchronize()
    for name in ("m_acc", "m_num", "m_bonus", "m_rounds", "status", "pl"):
        a, b = getattr(seq, name).cpu().numpy(), getattr(fus, name).cpu().numpy()
        assert np.array_equal(a, b), (name, a, b)
    assert np.array_equal(_raw(seq.k), _raw(fus.k)) and np.array_equal(_raw(seq.v), _raw(fus.v))
    return seq, fus, st_mask, st_verify


def _oracle_commit(w, fus, st_verify, k0, v0, bt, pl0):
    acc, num = fus.m_acc.cpu().numpy(), fus.m_num.cpu().numpy()
    k_ref, v_ref, pl_ref, st_ref = o_commit.kv_commit(k0, v0, bt, pl0, acc, num, st_verify, w.N)
    assert np.array_equal(fus.pl.cpu().numpy(), pl_ref)
    assert np.array_equal(fus.status.cpu().numpy(), st_ref)
    kr = k_ref.view(np.int16) if k_ref.dtype == np.uint16 else k_ref
    vr = v_ref.view(np.int16) if v_ref.dtype == np.uint16 else v_ref
    assert np.array_equal(_raw(fus.k), kr) and np.array_equal(_raw(fus.v), vr)


CASES = {
    # one workgroup per request (V <= 16384)
    "row_c2_bf16": (2, dict(B=3, L=100, H=4, V=3000)),
    "row_c5_f32_d64": (5, dict(B=2, L=301, H=2, D=64, V=1000, dtype="f32")),
    "row_c1_tiny": (1, dict()),
    "row_c4_scalar_loads": (4, dict(B=2, H=2, V=4097)),
    # several workgroups per request (V > 16384)
    "sliced_c2_bf16": (2, dict(B=3, L=20, H=2, V=40000)),
    "sliced_c4_scalar_loads": (4, dict(B=2, H=2, V=33001)),
    "sliced_c3_f32": (3, dict(B=2, L=40, H=2, V=20000, dtype="f32")),
    # the walking workgroups share the move by head: 13 heads over the 40
    # workgroups of a request (most move none), and 37 heads over 10 (uneven
    # blocks; 40 requests do not fit one workgroup per CU)
    "sliced_heads_fewer_than_groups": (2, dict(B=3, L=30, H=13, V=40000)),
    "sliced_heads_uneven_blocks": (2, dict(B=40, L=20, H=37, V=40000)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_sequential(name):
    cfg, kw = CASES[name]
    _case("mss_commit", name)
    w = synth.make_workload(cfg, **kw)
    seq, fus, st_mask, st_verify = _run_both(w)
    # the MSS half against the oracle, the commit half against the oracle's
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B, w.seed,
                              w.offset)
    exact, excused, bad = compare_mss(fus, ref)
    assert not bad, bad
    _oracle_commit(w, fus, st_verify, w.k_cache, w.v_cache, w.block_table, w.prefix_len)
    print(f"{name}: accepted {fus.m_num.cpu().numpy().tolist()}, MSS exact {exact}, near-tie {excused}")


@pytest.mark.parametrize("kernel_V", [3000, 40000])
def test_fused_status_paths(kernel_V):
    # request 0 ok; 1 a bad block in its tree range; 2 prefix too long for
    # the table; 3 a NaN in the root row (verify fails, commit skips); 4
    # already failed before the call
    _case("mss_commit status paths", kernel_V)
    w = synth.make_workload(2, B=5, L=40, H=2, V=kernel_V)
    L0 = w.prefix_len.copy()

    def mutate(run):
        bt = run.bt.cpu().numpy()
        bt[1, (int(L0[1]) + 1) // 16] = w.num_blocks + 3
        run.bt.copy_(torch.from_numpy(bt))
        pl = run.pl.cpu().numpy()
        pl[2] = w.max_blocks * 16 - w.N + 1
        run.pl.copy_(torch.from_numpy(pl))
        run.tl[3, 0, 7] = float("nan")
        run.status[4] = 3

    seq, fus, st_mask, st_verify = _run_both(w, mutate)
    st = fus.status.cpu().numpy()
    assert st[1] == 7 and st[2] == 6 and st[3] == 4 and st[4] == 3, st
    assert st[0] == 0
    bt = seq.bt.cpu().numpy()
    pl_in = L0.copy()
    pl_in[2] = w.max_blocks * 16 - w.N + 1
    _oracle_commit(w, fus, st_verify, w.k_cache, w.v_cache, bt, pl_in)


def test_fused_repeated_offsets():
    # several calls in a row on one workspace (left zeroed by each call), each
    # compacting the next tree; every call equals the two-call sequence
    _case("mss_commit repeated")
    w = synth.make_workload(2, B=4, L=60, H=2, V=40000)
    for off in range(3):
        _run_both(w, offset=w.offset + off)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fused_full_config(cfg):
    """The step's verify launch at full size: identical to the two calls, the
    MSS results equal to the oracle's (or differing only at a near tie of its
    walk), and the whole K/V caches equal to the oracle's compaction."""
    _case(f"mss_commit full config {cfg}")
    w = synth.make_config(cfg)
    seq, fus, st_mask, st_verify = _run_both(w)
    print(f"config {cfg}: accepted {fus.m_num.cpu().numpy().tolist()}")
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, st_mask, w.seed,
                              w.offset)
    exact, excused, bad = compare_mss(fus, ref)
    assert not bad, f"requests {bad} differ from the oracle"
    print(f"config {cfg}: {exact} exact, {excused} at a near tie")
    del seq
    _oracle_commit(w, fus, st_verify, w.k_cache, w.v_cache, w.block_table, w.prefix_len)
