"""Sampling transforms on the GPU (tree_logits_transform) against the oracle
(oracle/sampling.py), and verification of transformed rows.

Bars: the kept set exactly, except at a tie that rounding may settle either
way (counted): the oracle's top-p cut within 4e-6 (relative to the kept mass)
of a cumulative mass, or its k-th and (k+1)-th scaled logits within fp32
rounding of each other; kept scaled logits within 2.5e-7 relative of the
oracle's exact l / T (the device forms fp32(l * fp32(1/T)), at most two
roundings; exact at T = 1); probabilities within 1e-5 relative.  MSS on
transformed rows follows the MSS parity bar; and with i.i.d. drafted children
it samples the transformed target distribution (Theorem 4.2 for the sampling
distributions, as the wiki's implementation sketch applies it)."""
import numpy as np
import pytest
import torch

import synth
from oracle import exact, sampling

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


COMBOS = [(1.0, 0, 1.0), (0.7, 0, 1.0), (1.0, 50, 1.0), (1.0, 0, 0.9), (0.8, 40, 0.95),
          (1.3, 1, 1.0), (1.0, 3, 0.5), (2.0, 0, 0.3), (0.5, 1000, 0.99)]


def _rows(V, n, seed, ties):
    rng = np.random.default_rng(seed)
    r = rng.normal(0, 2.0, (n, V)).astype(np.float32)
    if ties:
        r = np.round(r * 4) / 4
    r[rng.random((n, V)) < 0.05] = -np.inf
    r[:, 0] = rng.normal(0, 2.0, n)               # at least one finite entry
    return r.astype(np.float32)


def _check_rows(rows, T, k, p, label):
    import tree_speculative_verification_attn_amd as tv
    dev = torch.from_numpy(rows).cuda()
    lg = torch.empty_like(dev)
    pr = torch.empty_like(dev)
    tv.tree_logits_transform(dev, lg, T, k, p, tv.TV_OUT_LOGITS)
    tv.tree_logits_transform(dev, pr, T, k, p, tv.TV_OUT_PROBS)
    torch.cuda.synchronize()
    lg, pr = lg.cpu().numpy(), pr.cpu().numpy()
    near = 0
    for i, row in enumerate(rows):
        keep = sampling.kept_in_rank_order(row, T, k, p)
        if keep is None:
            assert np.isnan(lg[i]).all() and np.isnan(pr[i]).all(), label
            continue
        got = set(np.nonzero(np.isfinite(lg[i]))[0].tolist())
        assert set(np.nonzero(pr[i] > 0)[0].tolist()) <= got, label      # tiny masses may round to 0
        if got != set(keep):
            m = sampling.top_p_margin(row, T, k, p)
            tie_k = sampling.rounding_tie_at_topk(row, T, k)
            assert m < 4e-6 or tie_k, (label, i, sorted(got ^ set(keep))[:10], m)
            near += 1
            continue
        ref_l = sampling.transform_row(row, T, k, p, "logits")
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(lg[i]), fin), label
        if T == 1.0:
            assert np.array_equal(lg[i][fin].astype(np.float64), ref_l[fin]), label
        else:
            np.testing.assert_allclose(lg[i][fin].astype(np.float64), ref_l[fin], rtol=2.5e-7, atol=3e-45,
                                       err_msg=label)
        ref_p = sampling.transform_row(row, T, k, p, "probs")
        np.testing.assert_allclose(pr[i], ref_p, rtol=1e-5, atol=1e-12, err_msg=label)
    return near


@pytest.mark.parametrize("V", [1, 7, 300, 2048, 5003, 32000, 36864, 40000, 100003])
def test_transform_matches_oracle(V):
    n = 4 if V > 50000 else 8
    near = 0
    for c, (T, k, p) in enumerate(COMBOS):
        for ties in (False, True):
            print(f"[case] transform V={V} T={T} k={k} p={p} ties={ties}", flush=True)
            near += _check_rows(_rows(V, n, 1000 * V + 10 * c + ties, ties), T, k, p, f"V={V} {T} {k} {p}")
    print(f"V={V}: {near} rows with a cut at a rounding-level tie")


def test_transform_fallback_paths():
    # Rows that defeat the short paths of the row-resident kernel: every entry
    # tied (the list above the top-k bound overflows), a few distinct values
    # (thousands tied at the top), and 600 entries tied at the maximum (a list
    # too long for the ranking search but short enough to list).
    rng = np.random.default_rng(11)
    V = 32000
    rows = np.empty((4, V), dtype=np.float32)
    rows[0] = 0.5
    rows[1] = rng.integers(0, 3, V).astype(np.float32)
    rows[2] = rng.normal(0, 1.0, V).astype(np.float32)
    rows[2, rng.choice(V, 600, replace=False)] = 9.0
    rows[3] = rng.normal(0, 1.0, V).astype(np.float32)
    rows[3, rng.choice(V, 3000, replace=False)] = -np.inf
    for T, k, p in ((0.8, 50, 0.9), (1.0, 200, 1.0), (1.0, 0, 0.5), (1.1, 250, 0.7), (1.0, 7, 1.0)):
        print(f"[case] transform fallbacks T={T} k={k} p={p}", flush=True)
        _check_rows(rows, T, k, p, f"fallback {T} {k} {p}")
        _check_rows(rows[:, :6000].copy(), T, k, p, f"fallback V=6000 {T} {k} {p}")


def test_transform_special_rows_in_place_and_errors():
    import tree_speculative_verification_attn_amd as tv
    rows = np.zeros((6, 9), dtype=np.float32)
    rows[1, 3] = np.nan
    rows[2, 5] = np.inf
    rows[3, :] = -np.inf
    rows[4, :] = 1.5                                # all tied: index order decides
    rows[5, :] = [3.0e38, 1, 2, 3, 4, 5, 6, 7, 8]   # overflows at T = 0.5
    for T, k, p in ((1.0, 4, 1.0), (0.5, 0, 0.6), (1.0, 0, 0.34)):
        _check_rows(rows, T, k, p, f"special {T} {k} {p}")
    # in place
    dev = torch.from_numpy(rows[4:5].copy()).cuda()
    tv.tree_logits_transform(dev, dev, 1.0, 4, 1.0, tv.TV_OUT_PROBS)
    torch.cuda.synchronize()
    np.testing.assert_allclose(dev.cpu().numpy()[0], [0.25] * 4 + [0.0] * 5)
    x = torch.zeros((2, 5), device="cuda:0")
    for kw in (dict(temperature=0.0), dict(top_p=0.0), dict(top_p=1.5), dict(top_k=-1), dict(kind=2)):
        with pytest.raises(tv.TreeVerifyError):
            tv.tree_logits_transform(x, x, **kw)


def test_mss_on_transformed_rows():
    import tree_speculative_verification_attn_amd as tv
    from oracle import verify as o_verify
    from tests.gpu_util import DeviceRun, compare_mss
    for V, (T, k, p) in ((3000, (0.8, 40, 0.9)), (40000, (1.2, 0, 0.8))):
        w = synth.make_workload(2, B=4, L=20, H=1, V=V)
        print(f"[case] MSS on transformed rows V={V}", flush=True)
        with np.errstate(divide="ignore"):
            logq = np.log(w.ssm_probs).astype(np.float32)
        run = DeviceRun(w).mask()
        tv.tree_logits_transform(run.tl, run.tl, T, k, p, tv.TV_OUT_LOGITS)
        lq = torch.from_numpy(logq).cuda()
        tv.tree_logits_transform(lq, run.sp, T, k, p, tv.TV_OUT_PROBS)
        run.mss()
        torch.cuda.synchronize()
        w.target_logits = sampling.transform(w.target_logits, T, k, p, "logits").astype(np.float32)
        w.ssm_probs = sampling.transform(logq, T, k, p, "probs").astype(np.float32)
        ref = o_verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B,
                                  w.seed, w.offset)
        ex, excused, bad = compare_mss(run, ref)
        print(f"V={V}: MSS exact {ex}, near-tie {excused}")
        assert not bad


def test_transformed_distribution_is_sampled():
    """i.i.d. children from the transformed draft distribution, transformed
    target rows: the first emitted token follows the transformed target."""
    import tree_speculative_verification_attn_amd as tv
    from tests.test_gpu_distribution import P8, Q8, _run
    T, k, p = 0.7, 6, 0.85
    lp = np.log(np.array([float(x) for x in P8])).astype(np.float32)
    lq = np.log(np.array([float(x) for x in Q8])).astype(np.float32)
    p_t = sampling.transform_row(lp, T, k, p, "probs")
    q_t = sampling.transform_row(lq, T, k, p, "probs")
    n = 1_000_000
    print("[case] transformed TV iid star3 V=8 n=1e6", flush=True)
    parent, tok, _, _, qr = synth.iid_tree_batch(777, n, p_t, q_t, "star3")
    tl = torch.from_numpy(np.broadcast_to(lp, (n, 4, 8)).copy()).cuda()
    tv.tree_logits_transform(tl, tl, T, k, p, tv.TV_OUT_LOGITS)
    sp = torch.from_numpy(lq[None, None, :].copy()).cuda()
    tv.tree_logits_transform(sp, sp, T, k, p, tv.TV_OUT_PROBS)
    sp = sp.expand(n, 1, 8).contiguous()
    first, num = _run(parent, tok, tl.cpu().numpy(), sp.cpu().numpy(), qr, seed=31)
    hist = np.bincount(first, minlength=8) / n
    tv_ = 0.5 * np.abs(hist - p_t).sum()
    print(f"TV(first token, transformed P_LLM) = {tv_:.2e}; accept rate {np.mean(num > 0):.3f}")
    assert tv_ < 5e-3
    assert 0.5 * np.abs(hist - np.array([float(x) for x in P8])).sum() > 0.05   # not the raw target
