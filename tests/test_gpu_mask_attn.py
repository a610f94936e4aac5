"""tree_mask_attn_verify against tree_build_mask followed by tree_attn_verify:
the masks, depths, status codes and outputs must be identical bit for bit
(the call promises the results of the two calls in sequence, and the
attention sums every chunk in a fixed order), both where it is one kernel
(bf16, one chunk per (request, head)) and where it runs the two (fp32, split
chunk plans).  Outputs are also checked against the oracle, masks against the
oracle's tree builder."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import DeviceRun, o_attn, o_tree, out_to_f64, to_dev, u64
import tree_speculative_verification_attn_amd as tv

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-2), "f32": (1e-5, 1e-5)}

CASES = {
    "c1_tiny": dict(cfg=1),
    "c2_small": dict(cfg=2, B=2, L=100, H=4, V=64),
    "c2_small_d64": dict(cfg=2, B=2, L=70, H=4, D=64, V=64),
    "c3_small": dict(cfg=3, B=3, L=77, H=3, V=64),
    "c4_small": dict(cfg=4, B=3, H=2, V=64),
    "c5_split": dict(cfg=5, B=1, L=1500, H=2, V=64),            # several chunks: two kernels
    "c2_small_f32": dict(cfg=2, B=2, L=100, H=3, V=64, dtype="f32"),
}


def _case(*a):
    print("[case]", *a, flush=True)


def _raw(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _both(w, mutate=None, stale=-99):
    seq = DeviceRun(w)
    fus = DeviceRun(w)
    for r in (seq, fus):
        r.status.fill_(stale)                  # the mask stage writes every status
        r.anc.fill_(-1)
        r.child.fill_(-1)
        r.depth.fill_(-1)
        if mutate:
            mutate(r)
    seq.mask().attn()
    fus.mask_attn()
    torch.cuda.synchronize()
    return seq, fus


def _same(seq, fus):
    assert torch.equal(seq.status, fus.status), (seq.status, fus.status)
    assert torch.equal(seq.anc, fus.anc)
    assert torch.equal(seq.child, fus.child)
    assert torch.equal(seq.depth, fus.depth)
    ok = seq.status.cpu().numpy() == 0         # (a bad block id leaves the output unspecified)
    assert np.array_equal(_raw(seq.out)[ok], _raw(fus.out)[ok])
    zero = np.isin(seq.status.cpu().numpy(), (1, 6))
    assert np.all(out_to_f64(fus.out)[zero] == 0)


def _oracle(run, pairs=None):
    w = run.w
    anc, child, depth, st = o_tree.build_mask_batch(w.parent)
    B, N = w.B, w.N
    assert np.array_equal(u64(run.anc), np.array(anc, dtype=np.uint64).reshape(B, N))
    assert np.array_equal(u64(run.child), np.array(child, dtype=np.uint64).reshape(B, N + 1))
    assert np.array_equal(run.depth.cpu().numpy(), np.array(depth).reshape(B, N))
    ref, rst = o_attn.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len, anc, st,
                                     w.dtype, w.scale, pairs=pairs)
    assert list(run.status.cpu().numpy()) == rst
    got = out_to_f64(run.out)
    atol, rtol = TOL[w.dtype]
    for b, h in (pairs if pairs is not None else [(b, h) for b in range(B) for h in range(w.H)]):
        err = np.abs(got[b, :, h] - ref[b, :, h])
        assert not (err > atol + rtol * np.abs(ref[b, :, h])).any(), (b, h, float(err.max()))


def _kernels(w):
    code = tv.TV_BF16 if w.dtype == "bf16" else tv.TV_F32
    one = w.dtype == "bf16" and tv.tree_attn_verify_workspace(code, w.B, w.N, w.H, w.D, w.max_blocks) == 0
    return "one kernel" if one else "two kernels"


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_sequential(name):
    kw = dict(CASES[name])
    w = synth.make_workload(kw.pop("cfg"), **kw)
    _case("mask+attn", name, _kernels(w))
    seq, fus = _both(w)
    _same(seq, fus)
    _oracle(fus)


def test_fused_tree_shapes():
    # one node, a 64-node chain, padding slots, a star, prefix 0 and ragged prefixes
    trees = (("parents", [-1]), ("parents", [-1] + list(range(63))), ("parents", [-1, -2, 0, -2]),
             ("parents", [-1] * 64), ("expand_trunc", (4, 4, 2, 1, 1), 64))
    for L in (0, 15, 129):
        for tree_ in trees:
            _case("mask+attn tree", L, tree_[0], len(tree_[1]) if tree_[0] == "parents" else tree_[1])
            w = synth.make_workload(dict(name="t", B=2, H=2, D=128, V=128, dtype="bf16", tree=tree_, L=L,
                                         sig_t=1.0, sig_s=1.0), 91)
            seq, fus = _both(w)
            _same(seq, fus)
            _oracle(fus)


def test_fused_status_paths():
    w = synth.make_workload(2, B=5, L=40, H=3, V=64)
    par = w.parent.copy()
    par[0, 3] = 7                          # a parent after its child: malformed
    par[3, 0] = -3
    w.parent = par
    pl = w.prefix_len.copy()
    pl[1] = w.max_blocks * 16              # no room for the tree
    pl[4] = 10                             # a shorter prefix: its last table entry is not needed
    bt = w.block_table.copy()
    bt[2, 1] = w.num_blocks + 5            # a bad block id the call needs
    assert (10 + w.N - 1) // 16 < w.max_blocks - 1
    bt[4, w.max_blocks - 1] = -7           # ... and one it does not need
    def mutate(r):
        r.pl = to_dev(pl)
        r.bt = to_dev(bt)
    _case("mask+attn status", "malformed, capacity, bad block, unused bad block")
    seq, fus = _both(w, mutate)
    assert list(fus.status.cpu().numpy()) == [1, 6, 7, 1, 0]
    _same(seq, fus)
    # a malformed tree with no room for it still reports the malformed tree
    pl2 = pl.copy()
    pl2[0] = w.max_blocks * 16
    _case("mask+attn status", "malformed and over capacity")
    seq, fus = _both(w, lambda r: setattr(r, "pl", to_dev(pl2)))
    assert fus.status.cpu().numpy()[0] == 1
    _same(seq, fus)


def test_fused_empty_tree():
    w = synth.make_workload(dict(name="e", B=3, H=2, D=128, V=50, dtype="bf16", tree=("parents", []), L=10,
                                 sig_t=1.0, sig_s=1.0), 3)
    _case("mask+attn", "N = 0")
    run = DeviceRun(w)
    run.status.fill_(-99)
    run.child.fill_(-1)
    run.mask_attn()
    torch.cuda.synchronize()
    assert run.status.cpu().numpy().tolist() == [0, 0, 0]
    assert run.child.cpu().numpy().tolist() == [[0], [0], [0]]


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fused_full_config(cfg):
    """The step's attention launch at full size: the same results as the two
    calls, the same bits on repeated calls, masks equal to the oracle's,
    sampled (request, head) outputs within the bar of the oracle."""
    w = synth.make_config(cfg)
    _case(f"mask+attn full config {cfg}", _kernels(w))
    if cfg in (2, 4):
        assert _kernels(w) == "one kernel"
    seq, fus = _both(w)
    _same(seq, fus)
    first = _raw(fus.out)
    for _ in range(3):                       # repeated calls: the same bits
        fus.mask_attn()
        torch.cuda.synchronize()
        assert np.array_equal(_raw(fus.out), first)
    rng = np.random.default_rng(100 + cfg)
    pairs = {(b, int(rng.integers(w.H))) for b in range(w.B)}      # every request once
    pairs |= {(0, 0), (w.B - 1, w.H - 1)}
    _oracle(fus, pairs=sorted(pairs))
