"""The whole verification step captured in a HIP graph: every replay must
match the eager step bit for bit, the attention output included (chunks of
a few and of more than 100 stages of 32 keys: each group sums a fixed set of
stages in a fixed order).

The step is tree_build_mask -> tree_attn_verify -> tree_verify_greedy ->
tree_verify_mss -> kv_commit_accepted on one seeded workload, either as five
calls or as the benchmark's three (tree_mask_attn_verify, tree_verify_greedy,
tree_verify_mss_commit).  Between
replays the test restores the KV cache and prefix lengths (which the commit
changes) with eager copies, runs unrelated eager work, and synchronizes, so a
graph node that depends on state left by an earlier replay would show up as
a mismatch.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tree_speculative_verification_attn_amd as tv
    from tests.gpu_util import to_dev


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _state(w):
    bf = w.dtype == "bf16"
    s = dict(q=to_dev(w.q, bf), k=to_dev(w.k_cache, bf), v=to_dev(w.v_cache, bf), bt=to_dev(w.block_table),
             pl=to_dev(w.prefix_len), parent=to_dev(w.parent), token=to_dev(w.token),
             tl=to_dev(w.target_logits), sp=to_dev(w.ssm_probs), qr=to_dev(w.q_row))
    B, N = w.B, w.N
    dev = "cuda:0"
    s.update(anc=torch.zeros((B, N), dtype=torch.int64, device=dev),
             child=torch.zeros((B, N + 1), dtype=torch.int64, device=dev),
             depth=torch.zeros((B, N), dtype=torch.int32, device=dev),
             status=torch.zeros((B,), dtype=torch.int32, device=dev),
             out=torch.zeros_like(s["q"]))
    for name in ("g_acc", "m_acc"):
        s[name] = torch.zeros((B, N), dtype=torch.int32, device=dev)
    for name in ("g_num", "g_bonus", "m_num", "m_bonus", "m_rounds"):
        s[name] = torch.zeros((B,), dtype=torch.int32, device=dev)
    code = tv.TV_BF16 if bf else tv.TV_F32
    n_a = tv.tree_attn_verify_workspace(code, B, N, w.H, w.D, w.max_blocks)
    s["ws_a"] = torch.zeros(max(n_a, 1), dtype=torch.uint8, device=dev) if n_a else None
    s["ws_v"] = torch.zeros(tv.tree_verify_workspace(B, N, w.V), dtype=torch.uint8, device=dev)
    return s


def _step(s, w, fused):
    if fused:
        tv.tree_mask_attn_verify(s["q"], s["k"], s["v"], s["bt"], s["pl"], s["parent"], s["anc"], s["child"],
                                 s["depth"], s["status"], s["out"], s["ws_a"], scale=w.scale)
        tv.tree_verify_greedy(s["tl"], s["token"], s["child"], s["status"], s["g_acc"], s["g_num"], s["g_bonus"],
                              s["ws_v"])
        tv.tree_verify_mss_commit(s["tl"], s["sp"], s["qr"], s["token"], s["child"], s["status"], w.seed, w.offset,
                                  s["m_acc"], s["m_num"], s["m_bonus"], s["m_rounds"], s["ws_v"], s["k"], s["v"],
                                  s["bt"], s["pl"])
        return
    tv.tree_build_mask(s["parent"], s["anc"], s["child"], s["depth"], s["status"])
    tv.tree_attn_verify(s["q"], s["k"], s["v"], s["bt"], s["pl"], s["anc"], s["status"], s["out"], s["ws_a"],
                        scale=w.scale)
    tv.tree_verify_greedy(s["tl"], s["token"], s["child"], s["status"], s["g_acc"], s["g_num"], s["g_bonus"],
                          s["ws_v"])
    tv.tree_verify_mss(s["tl"], s["sp"], s["qr"], s["token"], s["child"], s["status"], w.seed, w.offset,
                       s["m_acc"], s["m_num"], s["m_bonus"], s["m_rounds"], s["ws_v"])
    tv.kv_commit_accepted(s["k"], s["v"], s["bt"], s["pl"], s["m_acc"], s["m_num"], s["status"])


OUTS = ("anc", "child", "depth", "status", "out", "g_acc", "g_num", "g_bonus", "m_acc", "m_num", "m_bonus",
        "m_rounds", "pl", "k", "v")


def _same(name, got, ref, w):
    return torch.equal(got, ref)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("cfg,kw", [(2, dict(B=4, L=300, H=8, V=32000)),
                                    (3, dict(B=3, L=77, H=3, V=50272)),
                                    (4, dict(B=6, H=2, V=20000)),
                                    # 960 (request, head) items: the single-group attention
                                    # kernel that ranks requests by prefix length
                                    (4, dict(B=40, H=24, V=20000))])
def test_graph_replay_matches_eager(cfg, kw, fused):
    w = synth.make_workload(cfg, **kw)
    print("[case] graph replay", cfg, kw, "three launches" if fused else "five calls", flush=True)
    s = _state(w)
    k0, v0, pl0 = s["k"].clone(), s["v"].clone(), s["pl"].clone()

    def restore():
        s["k"].copy_(k0)
        s["v"].copy_(v0)
        s["pl"].copy_(pl0)
        s["status"].zero_()

    _step(s, w, fused)                       # eager reference
    torch.cuda.synchronize()
    ref = {n: s[n].clone() for n in OUTS}
    assert int((ref["status"] != 0).sum()) == 0

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(s, w, fused)
    for rep in range(4):
        restore()
        for n in OUTS[4:12]:
            s[n].fill_(-7)                   # stale outputs must be overwritten
        junk = torch.randn(1 << 20, device="cuda:0").sum()     # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for n in OUTS:
            assert _same(n, s[n], ref[n], w), (rep, n)
        assert int(s["ws_v"].count_nonzero()) == 0
