"""Per-sequence layout on the GPU: every root-to-leaf path run as a chain of
its own through tree_attn_verify gives, at each chain node, the tree output of
the node it copies, and the oracle's attention over the same chains (causal
attention along each path over its prefix) gives the same outputs; both
within the attention bar of the parity tests: 2e-2 + 2e-2*|ref| for bf16,
1e-5 + 1e-5*|ref| for fp32."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-2), "f32": (1e-5, 1e-5)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _host(t):
    """Device tensor -> numpy array in the oracle's input form (bf16 as bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _attn(tv, q, k, v, bt, pl, parent, dtype, scale, H, D):
    S, N = parent.shape
    anc = torch.zeros((S, N), dtype=torch.int64, device="cuda:0")
    child = torch.zeros((S, N + 1), dtype=torch.int64, device="cuda:0")
    depth = torch.zeros((S, N), dtype=torch.int32, device="cuda:0")
    st = torch.zeros((S,), dtype=torch.int32, device="cuda:0")
    tv.tree_build_mask(parent, anc, child, depth, st)
    code = tv.TV_BF16 if dtype == "bf16" else tv.TV_F32
    n = tv.tree_attn_verify_workspace(code, S, N, H, D, bt.shape[1])
    ws = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(q)
    tv.tree_attn_verify(q, k, v, bt, pl, anc, st, out, ws if n else None, scale=scale)
    torch.cuda.synchronize()
    assert (st.cpu().numpy() == 0).all()
    return out


@pytest.mark.parametrize("cfg,kw", [(2, dict(B=2, L=100, H=4, V=64)),
                                    (3, dict(B=3, L=77, H=3, V=64)),
                                    (4, dict(B=3, H=2, V=64)),
                                    (5, dict(B=2, L=301, H=2, D=64, V=64, dtype="f32"))])
def test_paths_match_tree(cfg, kw):
    import tree_speculative_verification_attn_amd as tv
    from tree_speculative_verification_attn_amd import per_sequence
    from tests.gpu_util import DeviceRun, out_to_f64
    w = synth.make_workload(cfg, **kw)
    print(f"[case] per-sequence cfg{cfg}", flush=True)
    run = DeviceRun(w).mask().attn()
    torch.cuda.synchronize()
    tree_out = out_to_f64(run.out)
    sb = per_sequence.build(w.parent, w.prefix_len, run.q, run.k, run.v, run.bt)
    assert sb.S == sum(len(per_sequence.leaf_paths(w.parent[b])) for b in range(w.B))
    seq_out = out_to_f64(_attn(tv, sb.q, sb.k_cache, sb.v_cache, sb.block_table, sb.prefix_len,
                               sb.parent, w.dtype, w.scale, w.H, w.D))
    atol, rtol = TOL[w.dtype]
    for s, (b, path) in enumerate(sb.paths):
        got = seq_out[s, :len(path)]
        ref = tree_out[b, path]
        bad = np.abs(got - ref) > atol + rtol * np.abs(ref)
        assert not bad.any(), (s, b, path, float(np.abs(got - ref).max()))
    # the chains against the oracle, every chain node and head
    from oracle import attention as o_attn
    from oracle import tree as o_tree
    par = sb.parent.cpu().numpy()
    anc_o, _, _, st_o = o_tree.build_mask_batch(par)
    ref_seq, st_ref = o_attn.tree_attention(_host(sb.q), _host(sb.k_cache), _host(sb.v_cache),
                                            sb.block_table.cpu().numpy(), sb.prefix_len.cpu().numpy(), anc_o,
                                            st_o, w.dtype, w.scale)
    assert all(x == 0 for x in st_ref)
    for s, (b, path) in enumerate(sb.paths):
        got = seq_out[s, :len(path)]
        ref = ref_seq[s, :len(path)]
        bad = np.abs(got - ref) > atol + rtol * np.abs(ref)
        assert not bad.any(), ("oracle", s, b, path, float(np.abs(got - ref).max()))
