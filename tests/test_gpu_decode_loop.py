"""The toy speculative decoding loop end to end on the GPU (masks, tree
attention, verification and KV compaction through the library):

- greedy speculative decoding emits what plain greedy decoding of the same
  target emits (a difference is allowed only where plain decoding's two best
  logits are within 1e-4, a tie that rounding may break either way);
- stochastic speculative decoding with i.i.d. drafted children samples the
  target's own distribution: the first two emitted tokens of many runs
  against the exact two-token probabilities (SpecInfer summary, Theorem 4.2);
- after decoding, the cache holds exactly the K/V of the committed tokens at
  their positions, and the prefix length counts them."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _setup(V, seed=0, noise=1.0, n_ssm=1, dtype=torch.float32):
    from tree_speculative_verification_attn_amd import decode_loop as dl
    model = dl.ToyTarget(V, seed=seed, dtype=dtype)
    drafter = dl.BigramDrafter(model, n_ssm=n_ssm, noise=noise, seed=seed + 1)
    return dl, model, drafter


@pytest.mark.parametrize("tree", [("expand", (3, 2, 1)), ("merge", 4)])
def test_greedy_matches_plain(tree):
    print(f"[case] loop greedy {tree}", flush=True)
    dl, model, drafter = _setup(64, seed=3, noise=0.5, n_ssm=3)
    B, T = 16, 40
    prompt = torch.randint(0, 64, (B, 5), generator=torch.Generator().manual_seed(7)).cuda()
    dec = dl.SpecDecoder(model, drafter, B, mode="greedy", tree=tree)
    dec.prefill(prompt)
    got = np.array(dec.generate(T))
    want, margin = dl.plain_greedy(model, prompt, T)
    excused = 0
    for b in range(B):
        diff = np.nonzero(got[b] != want[b])[0]
        if diff.size:
            t = int(diff[0])
            assert margin[b, t] < 1e-4, (b, t, got[b, :t + 1], want[b, :t + 1], margin[b, t])
            excused += 1
    tokens_per_iter = (dec.accepted_total + B * dec.iters) / (B * dec.iters)
    print(f"greedy {tree}: {dec.iters} iterations, {dec.accepted_total} accepted, "
          f"{tokens_per_iter:.2f} tokens per request per iteration, {excused} near-tie divergences")
    assert dec.accepted_total > 0 and excused <= 1


def test_mss_samples_target_distribution():
    print("[case] loop MSS distribution", flush=True)
    dl, model, drafter = _setup(8, seed=11, noise=1.0)
    prompt_row = torch.tensor([1, 5, 2])
    exact = dl.continuation_probs(model, prompt_row.cuda(), 2)       # [V][V]
    counts = np.zeros((8, 8))
    n = 0
    for rep in range(4):
        B = 8192
        dec = dl.SpecDecoder(model, drafter, B, mode="mss", tree=("expand", (2, 2)), seed=100 + rep,
                             draft_seed=200 + rep)
        dec.prefill(prompt_row[None, :].repeat(B, 1).cuda())
        out = np.array(dec.generate(2))
        np.add.at(counts, (out[:, 0], out[:, 1]), 1)
        n += B
    emp = counts / n
    tv = 0.5 * np.abs(emp - exact).sum()
    # the same statistic for n draws from the exact distribution itself
    rng = np.random.default_rng(0)
    ref = [0.5 * np.abs(rng.multinomial(n, exact.ravel()) / n - exact.ravel()).sum() for _ in range(20)]
    print(f"MSS loop: TV {tv:.4f} over {n} runs; TV of exact draws {np.mean(ref):.4f} "
          f"(max {np.max(ref):.4f})")
    assert tv < 2.0 * max(ref)
    # and the drafter alone is far from the target: the test can tell them apart
    q1 = drafter.tables[0][2].cpu().numpy()
    assert 0.5 * np.abs(q1 - exact.sum(1)).sum() > 5 * max(ref)


def test_naive_is_unbiased_and_mss_accepts_more():
    """Naive sampling (draw, then look for the token; the drawn token is
    emitted on a miss) also samples the target, and MSS accepts more tokens
    per iteration on the same trees (Theorem 4.3, Table 3's comparison)."""
    print("[case] loop naive vs MSS", flush=True)
    dl, model, drafter = _setup(8, seed=11, noise=1.0)
    prompt_row = torch.tensor([1, 5, 2])
    exact = dl.continuation_probs(model, prompt_row.cuda(), 2)
    per_iter = {}
    for mode in ("naive", "mss"):
        counts = np.zeros((8, 8))
        n = acc = iters = 0
        for rep in range(2):
            B = 8192
            dec = dl.SpecDecoder(model, drafter, B, mode=mode, tree=("expand", (2, 2)), seed=300 + rep,
                                 draft_seed=400 + rep)
            dec.prefill(prompt_row[None, :].repeat(B, 1).cuda())
            out = np.array(dec.generate(2))
            np.add.at(counts, (out[:, 0], out[:, 1]), 1)
            n += B
            acc += dec.accepted_total
            iters += dec.iters * B
        tv_ = 0.5 * np.abs(counts / n - exact).sum()
        per_iter[mode] = (acc + iters) / iters
        print(f"{mode}: TV {tv_:.4f}, {per_iter[mode]:.3f} tokens per request per iteration")
        assert tv_ < 0.025
    assert per_iter["mss"] > per_iter["naive"]


@pytest.mark.parametrize("mode,dtype", [("mss", torch.float32), ("greedy", torch.bfloat16)])
def test_cache_holds_committed_tokens(mode, dtype):
    print(f"[case] loop cache {mode} {dtype}", flush=True)
    dl, model, drafter = _setup(32, seed=5, noise=0.7, n_ssm=2, dtype=dtype)
    B = 6
    prompt = torch.randint(0, 32, (B, 4), generator=torch.Generator().manual_seed(1)).cuda()
    dec = dl.SpecDecoder(model, drafter, B, mode=mode, tree=("merge", 3) if mode == "greedy" else ("expand", (2, 2)))
    dec.prefill(prompt)
    dec.generate(20)
    st = dec.state
    pl = st.prefix_len.cpu().numpy()
    for b in range(B):
        seq = prompt[b].tolist() + dec.out[b][:-1]       # the last bonus is still pending
        assert pl[b] == len(seq)
        toks = torch.tensor(seq, device="cuda:0")[None, :]
        pos = torch.arange(len(seq), device="cuda:0")[None, :]
        _, k, v = model.qkv(model.embed(toks, pos))
        slots = torch.arange(len(seq), device="cuda:0")
        blk = st.block_table[b, slots // 16].long()
        kc = st.k[blk, :, slots % 16, :]
        vc = st.v[blk, :, slots % 16, :]
        tol = 1e-4 if dtype == torch.float32 else 2e-2
        assert torch.allclose(kc.float(), k[0].float(), atol=tol, rtol=tol)
        assert torch.allclose(vc.float(), v[0].float(), atol=tol, rtol=tol)
