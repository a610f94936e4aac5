"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.

Bars: masks, accepted paths, bonus tokens, rounds, status and KV compaction
bit-exact; MSS decisions may differ only for requests whose oracle trace has a
near tie (|u - ratio| < 1e-6, or an inverse-CDF boundary within 1e-6 of the
total mass), counted and printed; attention per element within
2e-2 + 2e-2*|ref| for bf16 and 1e-5 + 1e-5*|ref| for fp32.
"""
import numpy as np
import pytest
import torch

import synth
from tests.golden.load import read_mask_fixture

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_util import (DeviceRun, compare_mss, compare_naive, o_attn, o_commit, o_tree, o_verify,
                                out_to_f64, to_dev, u64)

TOL = {"bf16": (2e-2, 2e-2), "f32": (1e-5, 1e-5)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL = {
    "c1_tiny": dict(cfg=1),
    "c2_small": dict(cfg=2, B=2, L=100, H=4, V=3000),
    "c2_small_f32": dict(cfg=2, B=2, L=100, H=3, V=3000, dtype="f32"),
    "c2_small_d64": dict(cfg=2, B=2, L=70, H=4, D=64, V=3000),
    "c3_small": dict(cfg=3, B=3, L=77, H=3, V=5003),
    "c4_small": dict(cfg=4, B=3, H=2, V=4000),
    "c5_small": dict(cfg=5, B=1, L=1500, H=2, V=2000),
    "c5_small_f32_d64": dict(cfg=5, B=2, L=301, H=2, D=64, V=1000, dtype="f32"),
}


def _small(name):
    kw = dict(SMALL[name])
    cfg = kw.pop("cfg")
    return synth.make_workload(cfg, **kw)


def _print_case(*a):
    print("[case]", *a, flush=True)


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------
def _mask_case(parent_2d):
    B, N = parent_2d.shape
    p = to_dev(parent_2d.astype(np.int32))
    anc = torch.zeros((B, N), dtype=torch.int64, device="cuda:0")
    child = torch.zeros((B, N + 1), dtype=torch.int64, device="cuda:0")
    depth = torch.zeros((B, N), dtype=torch.int32, device="cuda:0")
    st = torch.full((B,), -5, dtype=torch.int32, device="cuda:0")
    import tree_speculative_verification_attn_amd as tv
    tv.tree_build_mask(p, anc, child, depth, st)
    torch.cuda.synchronize()
    ra, rc, rd, rs = o_tree.build_mask_batch(parent_2d)
    assert np.array_equal(u64(anc), np.array(ra, dtype=np.uint64).reshape(B, N))
    assert np.array_equal(u64(child), np.array(rc, dtype=np.uint64).reshape(B, N + 1))
    assert np.array_equal(depth.cpu().numpy(), np.array(rd).reshape(B, N))
    assert np.array_equal(st.cpu().numpy(), np.array(rs))


def test_mask_golden_and_random():
    _print_case("mask golden")
    for fx in ("p3_tree_mask.txt", "fig3_tree.txt"):
        parent, _ = read_mask_fixture(fx)
        _mask_case(np.array([parent]))
    rng = np.random.default_rng(5)
    for n in (1, 2, 17, 63, 64):
        par = np.array([[-1] + [int(rng.integers(-1, i)) for i in range(1, n)] for _ in range(37)])
        _mask_case(par)
    # chains, stars, padding slots, malformed rows mixed in one batch
    rows = [[-1] + list(range(63)), [-1] * 64, [0] + [-1] * 63, [-1, 1] + [-1] * 62,
            [-1, 0, 5] + [-1] * 61, [-3] + [-1] * 63, [-1, -2, 0] + [-2] * 61,
            [-2, 0] + [-1] * 62, [-2] * 64]
    _mask_case(np.array(rows))


def test_mask_all_configs():
    for cfg in (1, 2, 3, 4, 5):
        _print_case("mask config", cfg)
        w = synth.make_workload(cfg, B=4 if cfg != 1 else 1, L=10, H=1, V=64)
        _mask_case(w.parent)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _check_attn(run, pairs=None):
    w = run.w
    anc, _, _, st = o_tree.build_mask_batch(w.parent)
    ref, rst = o_attn.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len, anc, st,
                                     w.dtype, w.scale, pairs=pairs)
    got = out_to_f64(run.out)
    sel = pairs if pairs is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    atol, rtol = TOL[w.dtype]
    worst = 0.0
    for b, h in sel:
        r = ref[b, :, h]
        g = got[b, :, h]
        err = np.abs(g - r)
        worst = max(worst, float(err.max()))
        bad = err > atol + rtol * np.abs(r)
        assert not bad.any(), (b, h, float(err.max()), np.argwhere(bad)[:5])
    assert list(run.status.cpu().numpy()) == rst
    return worst


@pytest.mark.parametrize("name", list(SMALL))
def test_attention_small(name):
    _print_case("attention", name)
    w = _small(name)
    run = DeviceRun(w).mask().attn()
    torch.cuda.synchronize()
    worst = _check_attn(run)
    print(f"{name}: max abs err {worst:.3e}")


def test_attention_edge_shapes():
    # prefix 0, one node, ragged prefix that is not a multiple of 16 or 32
    for kw in (dict(L=0), dict(L=1), dict(L=15), dict(L=33), dict(L=129)):
        for tree_ in (("parents", [-1]), ("parents", [-1, 0, 0, 1, -1]),
                      ("expand_trunc", (4, 4, 2, 1, 1), 64), ("parents", [-1, -2, 0, -2])):
            for dt in ("bf16", "f32"):
                _print_case("attention edge", kw, tree_, dt)
                w = synth.make_workload(dict(name="e", B=2, H=2, D=128, V=50, dtype=dt, tree=tree_,
                                             sig_t=1.0, sig_s=1.0, **kw), 77)
                run = DeviceRun(w).mask().attn()
                torch.cuda.synchronize()
                _check_attn(run)


def test_attention_status_paths():
    w = synth.make_workload(2, B=3, L=40, H=2, V=100)
    _print_case("attention status")
    run = DeviceRun(w).mask()
    # request 0 malformed upstream, request 1 over capacity, request 2 fine
    run.status[0] = 1
    pl = w.prefix_len.copy()
    pl[1] = w.max_blocks * 16
    run.pl = to_dev(pl)
    run.attn()
    torch.cuda.synchronize()
    st = run.status.cpu().numpy()
    assert list(st) == [1, 6, 0]
    out = out_to_f64(run.out)
    assert np.all(out[0] == 0)
    # request 2 matches the oracle
    w2 = w
    anc, _, _, _ = o_tree.build_mask_batch(w2.parent)
    ref, _ = o_attn.tree_attention(w2.q, w2.k_cache, w2.v_cache, w2.block_table, w2.prefix_len, anc,
                                   [0, 0, 0], w2.dtype, w2.scale, pairs=[(2, 0), (2, 1)])
    np.testing.assert_allclose(out[2], ref[2], atol=2e-2, rtol=2e-2)
    # a bad block id is reported as status 7
    bt = w.block_table.copy()
    bt[2, 0] = w.num_blocks + 5
    run2 = DeviceRun(w).mask()
    run2.bt = to_dev(bt)
    run2.attn()
    torch.cuda.synchronize()
    assert run2.status.cpu().numpy()[2] == 7


@pytest.mark.parametrize("B,H,D", [(40, 2, 128), (70, 2, 128), (40, 24, 128), (70, 12, 128), (300, 3, 128),
                                   (256, 3, 128), (64, 24, 64)])
@pytest.mark.parametrize("fused", [False, True])
def test_attention_ragged_order(B, H, D, fused):
    """Ragged prefixes in one batch (B on both sides of 64), with equal
    lengths, an empty prefix, the longest prefix repeated, a request skipped
    upstream and one past the cache's capacity; every (request, head) output
    is checked.  On a 256-CU device, 40 x 24, 70 x 12 and 256 x 3 (request,
    head) items at head dim 128, and 64 x 24 at head dim 64 (two default
    workgroups per CU there), are at least three rounds of workgroups, which
    runs the single-group kernel that takes requests longest first (ties by
    index; 256 requests is the most it ranks); 300 requests are more than it
    ranks, and the others fewer items."""
    _print_case("attention ragged order", B, H, D, "fused" if fused else "plain")
    w = synth.make_workload(dict(name="ragged", B=B, H=H, D=D, V=50, dtype="bf16", tree=("expand", (2, 2, 1)),
                                 L=("uniform", 0, 300), sig_t=1.0, sig_s=1.0), 91)
    pl = w.prefix_len.copy()
    pl[3] = pl[7] = pl[11] = pl[5]          # ties: rank by request index
    pl[10] = 0
    pl[12] = pl.max()
    pl[20] = w.max_blocks * 16              # past the table: TV_REQ_KV_CAPACITY
    w.prefix_len = pl
    run = DeviceRun(w)
    anc, _, _, st0 = o_tree.build_mask_batch(w.parent)
    st_in = list(st0)
    if fused:
        run.mask_attn()
    else:
        run.mask()
        run.status[2] = 1                   # skipped upstream
        st_in[2] = 1
        run.attn()
    torch.cuda.synchronize()
    ref, rst = o_attn.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len, anc, st_in,
                                     w.dtype, w.scale)
    assert list(run.status.cpu().numpy()) == rst
    got = out_to_f64(run.out)
    atol, rtol = TOL[w.dtype]
    for b in range(B):
        if rst[b] != 0:
            if rst[b] == 1:
                assert np.all(got[b] == 0)
            continue
        err = np.abs(got[b] - ref[b])
        assert not (err > atol + rtol * np.abs(ref[b])).any(), (b, float(err.max()))


# ----------------------------------------------------------------------------
# greedy / MSS
# ----------------------------------------------------------------------------
def _check_greedy(run):
    w = run.w
    ref = o_verify.verify_greedy(w.parent, w.token, w.target_logits, [0] * w.B)
    assert np.array_equal(run.g_acc.cpu().numpy(), ref["accepted"])
    assert np.array_equal(run.g_num.cpu().numpy(), ref["num_accepted"])
    assert np.array_equal(run.g_bonus.cpu().numpy(), ref["bonus"])
    assert np.array_equal(run.status.cpu().numpy(), ref["status"])


def _check_mss(run, label):
    w = run.w
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B,
                              w.seed, w.offset)
    exact, excused, bad = compare_mss(run, ref)
    print(f"{label}: MSS exact {exact}, near-tie {excused}, unexcused {len(bad)}; "
          f"accepted {run.m_num.cpu().numpy().tolist()}")
    assert not bad, (bad, run.m_num.cpu().numpy()[bad], ref["num_accepted"][bad])
    return ref


@pytest.mark.parametrize("name", list(SMALL))
def test_verify_small(name):
    _print_case("verify", name)
    w = _small(name)
    run = DeviceRun(w).mask().greedy()
    torch.cuda.synchronize()
    _check_greedy(run)
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    _check_mss(run, name)


def test_greedy_forced_paths():
    # logits make the LLM's choice equal a chosen child at every level
    w = synth.make_workload(1)
    tl = w.target_logits.copy()
    path = [0, 1, 2]        # learning -> algorithm -> is
    for d, node in enumerate(path):
        row = 0 if d == 0 else path[d - 1] + 1
        tl[0, row, :] = 0
        tl[0, row, w.token[0, node]] = 5.0
    tl[0, path[-1] + 1, :] = 0
    tl[0, path[-1] + 1, 7] = 5.0
    w.target_logits = tl
    run = DeviceRun(w).mask().greedy()
    torch.cuda.synchronize()
    assert run.g_num.cpu().numpy()[0] == 3 and run.g_bonus.cpu().numpy()[0] == 7
    _check_greedy(run)


def test_verify_status_paths():
    w = synth.make_workload(2, B=6, L=20, H=1, V=500)
    tok = w.token.copy()
    qr = w.q_row.copy()
    tl = w.target_logits.copy()
    sp = w.ssm_probs.copy()
    tok[1, 3] = w.V                 # bad token
    qr[2, 5] = w.R                  # bad q row
    tl[3, 0, 17] = np.nan           # the root row is always visited
    tl[4, 0, :] = -np.inf           # no finite value in a visited row
    tl[5, 0, :5] = -np.inf          # masked entries are fine
    w.token, w.q_row, w.target_logits, w.ssm_probs = tok, qr, tl, sp
    _print_case("verify status")
    run = DeviceRun(w).mask()
    run.status[0] = 1               # upstream fault
    run.greedy()
    torch.cuda.synchronize()
    st_g = run.status.cpu().numpy().copy()
    ref_g = o_verify.verify_greedy(w.parent, w.token, w.target_logits, [1, 0, 0, 0, 0, 0])
    assert list(st_g) == list(ref_g["status"])
    assert np.array_equal(run.g_num.cpu().numpy(), ref_g["num_accepted"])
    run = DeviceRun(w).mask()
    run.status[0] = 1
    run.mss()
    torch.cuda.synchronize()
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row,
                              [1, 0, 0, 0, 0, 0], w.seed)
    assert list(run.status.cpu().numpy()) == list(ref["status"])
    assert list(run.status.cpu().numpy())[:5] == [1, 2, 3, 4, 4]
    exact, excused, bad = compare_mss(run, ref)
    assert not bad


def test_mss_q_row_problems():
    # a negative draft probability on a tested child, and a NaN in a row read in full
    w = synth.make_workload(1)
    base_run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    sp = w.ssm_probs.copy()
    sp[0, :, :] = np.where(sp[0] > 0, sp[0], 0)
    sp[0, 0, 5] = np.nan            # row 0 proposes the root's children
    w.ssm_probs = sp
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0], w.seed)
    exact, excused, bad = compare_mss(run, ref)
    assert not bad
    assert base_run.status.cpu().numpy()[0] == 0


def test_mss_offsets_and_determinism():
    w = _small("c2_small")
    a = DeviceRun(w).mask().mss(offset=3)
    b = DeviceRun(w).mask().mss(offset=3)
    torch.cuda.synchronize()
    for x, y in ((a.m_acc, b.m_acc), (a.m_bonus, b.m_bonus), (a.m_rounds, b.m_rounds)):
        assert torch.equal(x, y)
    ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B,
                              w.seed, 3)
    exact, excused, bad = compare_mss(a, ref)
    assert not bad


def test_empty_tree_verify():
    w = synth.make_workload(dict(name="e", B=3, H=1, D=64, L=5, V=300, dtype="f32",
                                 tree=("parents", []), sig_t=2.0, sig_s=1.0), 3)
    run = DeviceRun(w).mask().greedy()
    torch.cuda.synchronize()
    _check_greedy(run)
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    _check_mss(run, "empty tree")


@pytest.mark.parametrize("V", [8, 2048, 4097, 8193, 12000, 16384])
def test_verify_row_vocab(V):
    # vocabularies up to 16384 entries: one workgroup per request, 8, 16 or 32
    # registers per row per thread; 4097 and 8193 take scalar loads
    for cfg, kw in ((2, dict(B=3, L=20, H=1)), (4, dict(B=2, H=1))):
        w = synth.make_workload(cfg, V=V, **kw)
        _print_case("verify row", cfg, V)
        run = DeviceRun(w).mask().greedy()
        torch.cuda.synchronize()
        _check_greedy(run)
        run = DeviceRun(w).mask().mss()
        torch.cuda.synchronize()
        _check_mss(run, f"row cfg{cfg} V={V}")


@pytest.mark.parametrize("V", [16385, 40000, 33001, 70001])
def test_verify_sliced_vocab(V):
    # vocabularies above 16384 entries take the kernel that splits a row over
    # several workgroups (2048 entries each); 16385, 33001 and 70001 have
    # ragged tails and take scalar loads
    for cfg, kw in ((2, dict(B=3, L=20, H=1)), (4, dict(B=2, H=1))):
        w = synth.make_workload(cfg, V=V, **kw)
        _print_case("verify sliced", cfg, V)
        run = DeviceRun(w).mask().greedy()
        torch.cuda.synchronize()
        _check_greedy(run)
        run = DeviceRun(w).mask().mss()
        torch.cuda.synchronize()
        _check_mss(run, f"sliced cfg{cfg} V={V}")
        assert int(run.ws_v.count_nonzero()) == 0


@pytest.mark.parametrize("B,V", [(6, 40000), (12, 40000), (24, 40000), (40, 40000), (24, 40001), (12, 33001)])
def test_verify_slice_widths(B, V):
    # The sliced MSS and naive walks pick 4, 8 or 16 entries per thread per
    # call (greedy keeps 8): on a 256-CU device, B = 6, 12 and 24 at
    # V = 40000 take 4, 8 and 16 (each the smallest width that gives every
    # workgroup a CU of its own) and B = 40 takes 16 over two launches.
    # V = 40001 and 33001 take the scalar loads.
    w = synth.make_workload(2, B=B, L=20, H=1, V=V)
    _print_case("verify slice widths", B, V)
    run = DeviceRun(w).mask().greedy()
    torch.cuda.synchronize()
    _check_greedy(run)
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    _check_mss(run, f"slice widths B={B} V={V}")
    assert int(run.ws_v.count_nonzero()) == 0
    # MSS with the compaction: the same path, and the prefix grown by it
    fused = DeviceRun(w).mask().mss_commit()
    torch.cuda.synchronize()
    for name in ("m_acc", "m_num", "m_bonus", "m_rounds", "status"):
        assert torch.equal(getattr(fused, name), getattr(run, name)), name
    num = run.m_num.cpu().numpy()
    assert np.array_equal(fused.pl.cpu().numpy(), w.prefix_len + np.maximum(num, 0))
    run = DeviceRun(w).mask().naive()
    torch.cuda.synchronize()
    ref = o_verify.verify_naive(w.parent, w.token, w.target_logits, [0] * w.B, w.seed, w.offset)
    exact, excused, bad = compare_naive(run, ref)
    assert not bad, bad
    assert int(run.ws_v.count_nonzero()) == 0


def test_verify_largest_vocabulary():
    # V = 2^20, the largest vocabulary the boundary accepts: 512 workgroups
    # of 8 entries per thread (greedy) or 256 of 16 (MSS, naive) per request,
    # one request per launch
    w = synth.make_workload(2, B=2, L=20, H=1, V=1 << 20)
    _print_case("verify largest vocabulary", w.V)
    run = DeviceRun(w).mask().greedy()
    torch.cuda.synchronize()
    _check_greedy(run)
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    _check_mss(run, "V = 2^20")
    assert int(run.ws_v.count_nonzero()) == 0
    run = DeviceRun(w).mask().naive()
    torch.cuda.synchronize()
    ref = o_verify.verify_naive(w.parent, w.token, w.target_logits, [0] * w.B, w.seed, w.offset)
    exact, excused, bad = compare_naive(run, ref)
    assert not bad, bad


@pytest.mark.parametrize("B", [6, 24])
def test_verify_rows_with_empty_slices(B):
    # Rows whose entries are -inf over whole workgroup slices (as top-k or
    # top-p filtering leaves them): such a slice has no argmax, and its
    # missing index must not be read as a NaN or +inf flag.  B = 6 takes 4
    # entries per thread (1024-entry slices), B = 24 takes 16 (4096).
    w = synth.make_workload(2, B=B, L=20, H=1, V=40000, seed=5)
    w.token = (w.token % 4096).astype(w.token.dtype)     # tokens below 4096 stay finite
    tl = w.target_logits.copy()
    tl[:, :, 4096:12288] = -np.inf            # several whole slices at any width
    tl[:, :, 20480:36864] = -np.inf
    w.target_logits = tl
    _print_case("verify rows with empty slices", B)
    run = DeviceRun(w).mask().greedy()
    torch.cuda.synchronize()
    _check_greedy(run)
    assert (run.status.cpu().numpy() == 0).all()
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    _check_mss(run, f"empty slices B={B}")
    assert (run.status.cpu().numpy() == 0).all()
    run = DeviceRun(w).mask().naive()
    torch.cuda.synchronize()
    ref = o_verify.verify_naive(w.parent, w.token, w.target_logits, [0] * w.B, w.seed, w.offset)
    exact, excused, bad = compare_naive(run, ref)
    assert not bad, bad


@pytest.mark.parametrize("V", [5003, 40003])
def test_verify_workspace_reuse(V):
    # one workspace for every call, left all zero after each; V = 5003 takes
    # one workgroup per request (ragged tail, scalar loads), V = 40003 splits
    # rows over 20 workgroups that exchange through the workspace
    w = synth.make_workload(3, B=3, L=77, H=3, V=V)
    run = DeviceRun(w).mask()
    outs = []
    for rep in range(3):
        _print_case("verify workspace reuse", rep)
        run.greedy().mss(offset=w.offset + rep % 2)
        torch.cuda.synchronize()
        assert int(run.ws_v.count_nonzero()) == 0
        outs.append([t.cpu().numpy().copy() for t in (run.g_acc, run.g_bonus, run.m_acc, run.m_num,
                                                      run.m_bonus, run.m_rounds)])
    for x, y in zip(outs[0], outs[2]):
        assert np.array_equal(x, y)
    _check_greedy(run)
    _check_mss(run, "workspace reuse")


@pytest.mark.parametrize("V", [12000, 40000])
def test_verify_many_requests(V):
    # 200 requests with a 7-node tree: one workgroup each (V = 12000), or 20
    # workgroups each, more than the device holds at once, so the requests
    # go out in several launches (V = 40000)
    w = synth.make_workload(dict(name="many", B=200, H=1, D=64, L=3, V=V, dtype="f32",
                                 tree=("parents", [-1, 0, 0, 1, -1, 4, 5]), sig_t=2.0, sig_s=1.0), 11)
    _print_case("verify many requests", w.B, w.V)
    run = DeviceRun(w).mask().greedy().mss()
    torch.cuda.synchronize()
    _check_greedy(run)
    ref = _check_mss(run, "many requests")
    assert int(run.ws_v.count_nonzero()) == 0
    assert (ref["status"] == 0).all()


@pytest.mark.parametrize("name", list(SMALL))
def test_naive_small(name):
    _print_case("naive", name)
    w = _small(name)
    run = DeviceRun(w).mask().naive()
    torch.cuda.synchronize()
    ref = o_verify.verify_naive(w.parent, w.token, w.target_logits, [0] * w.B, w.seed, w.offset)
    ex, excused, bad = compare_naive(run, ref)
    print(f"{name}: naive exact {ex}, near-tie {excused}")
    assert not bad


@pytest.mark.parametrize("V", [8, 4097, 16384, 16385, 40000, 33001])
def test_naive_both_kernels(V):
    # one workgroup per request up to V = 16384, sliced rows above; peaked
    # target rows make the draws hit tree tokens, so walks go deep
    for cfg, kw in ((2, dict(B=3, L=20, H=1)), (4, dict(B=2, H=1))):
        w = synth.make_workload(cfg, V=V, **kw)
        tl = w.target_logits.copy()
        for b in range(w.B):
            for i in range(w.N):         # node i's row favours its first child's token
                kids = [c for c in range(w.N) if w.parent[b, c] == i]
                if kids:
                    tl[b, i + 1, w.token[b, kids[0]]] += 12.0
            roots = [c for c in range(w.N) if w.parent[b, c] == -1]
            tl[b, 0, w.token[b, roots[0]]] += 12.0
        w.target_logits = tl
        _print_case("naive", cfg, V)
        run = DeviceRun(w).mask().naive(offset=7)
        torch.cuda.synchronize()
        ref = o_verify.verify_naive(w.parent, w.token, w.target_logits, [0] * w.B, w.seed, 7)
        ex, excused, bad = compare_naive(run, ref)
        print(f"naive cfg{cfg} V={V}: exact {ex}, near-tie {excused}, accepted {run.n_num.cpu().numpy().tolist()}")
        assert not bad
        assert int(run.n_num.max()) >= 2
        assert int(run.ws_v.count_nonzero()) == 0


def test_naive_status_and_rejection_rate():
    w = synth.make_workload(2, B=6, L=20, H=1, V=500)
    tok = w.token.copy()
    tl = w.target_logits.copy()
    tok[1, 3] = w.V                 # bad token
    tl[3, 0, 17] = np.nan
    tl[4, 0, :] = -np.inf
    w.token, w.target_logits = tok, tl
    run = DeviceRun(w).mask()
    run.status[0] = 1
    run.naive()
    torch.cuda.synchronize()
    ref = o_verify.verify_naive(w.parent, w.token, w.target_logits, [1, 0, 0, 0, 0, 0], w.seed, w.offset)
    assert list(run.status.cpu().numpy()) == list(ref["status"])
    ex, excused, bad = compare_naive(run, ref)
    assert not bad
    # Theorem 4.3's naive comparator: root rejection rate 1 - (mass of the
    # distinct root-child tokens), over many requests with their own streams
    from tests.test_gpu_distribution import P8, Q8
    p = np.array([float(x) for x in P8])
    q = np.array([float(x) for x in Q8])
    parent, tok, tl, sp, qr = synth.iid_tree_batch(4243, 200_000, p, q, "star3")
    n = tok.shape[0]
    par = torch.from_numpy(np.tile(parent, (n, 1))).cuda()
    anc = torch.zeros((n, 3), dtype=torch.int64, device="cuda:0")
    child = torch.zeros((n, 4), dtype=torch.int64, device="cuda:0")
    depth = torch.zeros((n, 3), dtype=torch.int32, device="cuda:0")
    st = torch.zeros((n,), dtype=torch.int32, device="cuda:0")
    import tree_speculative_verification_attn_amd as tv
    tv.tree_build_mask(par, anc, child, depth, st)
    acc = torch.empty((n, 3), dtype=torch.int32, device="cuda:0")
    num = torch.empty((n,), dtype=torch.int32, device="cuda:0")
    bonus = torch.empty((n,), dtype=torch.int32, device="cuda:0")
    ws = torch.zeros(tv.tree_verify_workspace(n, 3, 8), dtype=torch.uint8, device="cuda:0")
    tv.tree_verify_naive(torch.from_numpy(tl).cuda(), torch.from_numpy(tok).cuda(), child, st, 3, 0,
                         acc, num, bonus, ws)
    torch.cuda.synchronize()
    num = num.cpu().numpy()
    want = np.mean([o_verify.naive_reject_prob(p, row) for row in tok])
    got = np.mean(num == 0)
    print(f"naive root rejection {got:.4f}, closed form {want:.4f}")
    assert abs(got - want) < 4 * np.sqrt(want * (1 - want) / n)


# ----------------------------------------------------------------------------
# KV compaction
# ----------------------------------------------------------------------------
def _slots(cache, bt, b, slots):
    blk = bt[b, np.asarray(slots) // 16]
    return cache[blk, :, np.asarray(slots) % 16]


def _check_commit(run, w, acc, num, st_in, k_before, v_before):
    k_ref, v_ref, pl_ref, st_ref = o_commit.kv_commit(k_before, v_before, w.block_table, w.prefix_len,
                                                      acc, num, st_in, w.N)
    assert np.array_equal(run.pl.cpu().numpy(), pl_ref)
    assert np.array_equal(run.status.cpu().numpy(), st_ref)
    kg = run.k.view(torch.int16).cpu().numpy() if run.k.dtype == torch.bfloat16 else run.k.cpu().numpy()
    vg = run.v.view(torch.int16).cpu().numpy() if run.v.dtype == torch.bfloat16 else run.v.cpu().numpy()
    kr = k_ref.view(np.int16) if k_ref.dtype == np.uint16 else k_ref
    vr = v_ref.view(np.int16) if v_ref.dtype == np.uint16 else v_ref
    assert np.array_equal(kg, kr) and np.array_equal(vg, vr)


@pytest.mark.parametrize("name", ["c1_tiny", "c2_small", "c3_small", "c5_small", "c5_small_f32_d64"])
def test_commit_small(name):
    _print_case("commit", name)
    w = _small(name)
    run = DeviceRun(w).mask().mss()
    torch.cuda.synchronize()
    acc = run.m_acc.cpu().numpy()
    num = run.m_num.cpu().numpy()
    st_in = run.status.cpu().numpy().copy()
    run.commit(run.m_acc, run.m_num)
    torch.cuda.synchronize()
    _check_commit(run, w, acc, num, st_in, w.k_cache, w.v_cache)


def test_commit_hazard_and_errors():
    # path (1,2,4) overlaps sources and destinations; bad ids and capacity
    w = synth.make_workload(dict(name="h", B=5, H=3, D=128, L=29, V=40, dtype="bf16",
                                 tree=("parents", [-1, -1, 1, 2, 2, 3, 0]), sig_t=1.0, sig_s=1.0), 9)
    acc = np.full((5, 7), -1, dtype=np.int32)
    num = np.array([3, 2, 3, 0, -1], dtype=np.int32)
    acc[0, :3] = [1, 2, 4]
    acc[1, :2] = [6, 0]
    acc[2, :3] = [1, 2, 7]          # 7 >= N: bad accepted list
    run = DeviceRun(w).mask()
    torch.cuda.synchronize()
    st_in = run.status.cpu().numpy().copy()
    run.commit(to_dev(acc), to_dev(num))
    torch.cuda.synchronize()
    _check_commit(run, w, acc, num, st_in, w.k_cache, w.v_cache)
    assert run.status.cpu().numpy()[2] == 8


# ----------------------------------------------------------------------------
# full-size configurations (sampled attention outputs)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_config(cfg):
    _print_case("full config", cfg, "generate")
    w = synth.make_config(cfg)
    _print_case("full config", cfg, "mask+attn")
    run = DeviceRun(w).mask().attn()
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    # every request once (prefix lengths are ragged), at a random head, plus the corners
    pairs = [(b, int(rng.integers(w.H))) for b in range(w.B)]
    pairs += [(0, 0), (w.B - 1, w.H - 1)]
    worst = _check_attn(run, pairs=pairs)
    print(f"config {cfg}: attention max abs err {worst:.3e} over {len(pairs)} (b,h) pairs")
    _print_case("full config", cfg, "greedy")
    run.greedy()
    torch.cuda.synchronize()
    _check_greedy(run)
    _print_case("full config", cfg, "mss")
    run.mss()
    torch.cuda.synchronize()
    _check_mss(run, f"config {cfg}")
    _print_case("full config", cfg, "commit")
    acc = run.m_acc.cpu().numpy()
    num = run.m_num.cpu().numpy()
    L = w.prefix_len
    before_k = {}
    for b in range(w.B):
        if num[b] > 0:
            before_k[b] = (_slots(w.k_cache, w.block_table, b, L[b] + acc[b, : num[b]]),
                           _slots(w.v_cache, w.block_table, b, L[b] + acc[b, : num[b]]))
    run.commit(run.m_acc, run.m_num)
    torch.cuda.synchronize()
    assert np.array_equal(run.pl.cpu().numpy(), L + np.maximum(num, 0))
    kd = run.k.view(torch.int16) if run.k.dtype == torch.bfloat16 else run.k
    vd = run.v.view(torch.int16) if run.v.dtype == torch.bfloat16 else run.v
    for b, (kk, vv) in before_k.items():
        slots = L[b] + np.arange(num[b])
        blk = torch.from_numpy(w.block_table[b, slots // 16].astype(np.int64)).to("cuda:0")
        off = torch.from_numpy((slots % 16).astype(np.int64)).to("cuda:0")
        kg = kd[blk, :, off].cpu().numpy()
        vg = vd[blk, :, off].cpu().numpy()
        kr = kk.view(np.int16) if kk.dtype == np.uint16 else kk
        vr = vv.view(np.int16) if vv.dtype == np.uint16 else vv
        assert np.array_equal(kg, kr) and np.array_equal(vg, vr)
