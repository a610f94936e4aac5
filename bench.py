"""Benchmark of one tree-verification step on one MI355X.

A step is the whole verification path over one batch of synthetic input:
tree_build_mask -> tree_attn_verify -> tree_verify_greedy -> tree_verify_mss
-> kv_commit_accepted, in three launches: tree_mask_attn_verify (the masks
and the attention, with the results of the first two calls),
tree_verify_greedy, and tree_verify_mss_commit (the results of the last two).

The headline workload is the LLaMA-65B-shaped layer, the largest of the
five that runs on one GPU (bf16, 32 requests x 64 heads x 128 dims, ragged
prefixes of 512..4096 tokens in a paged cache, random 64-node trees, fp32
logits over a 32000-token vocabulary).  The LLaMA-7B, OPT-30B and
long-context layers are measured the same way and reported beside it, and so
is one GPU's share of the LLaMA-65B layer under 8-way tensor parallelism
over heads (8 of the 64 heads, every request).

Inputs stay resident in HBM.  The timed loop rotates over several copies of
the inputs whose total exceeds twice the 256 MB Infinity Cache, so each step
reads from HBM.  The commit grows each copy's prefix lengths; the timed
graphs hold one step per copy and then one copy that restores every copy's
prefix lengths, so each step sees the same workload.

Prints ONE JSON line (rank 0, N = 1): throughput in verified tree tokens/s
(B * N tree nodes per step), the roofline of the dominant kernel (attention,
HBM-bound) from HIP events recorded on the launch stream, the other
workloads, and the CPU oracle timed on a bounded sample of the same workload
on one host core and on all of the host's cores given to this GPU; the
oracle also replays the step's MSS call, and the line reports how many
requests match it exactly and how many differ only at a near tie.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree tokens/s + achieved HBM GB/s (% peak), tree_attn + MSS verify"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=None, help="workload id 1..5 (default 4 = LLaMA-65B layer)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="measure the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU sample time per leg")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + steps eager steps and exit (for counter collection)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run 5 device-to-device copies of this many MiB (counter calibration)")
    ap.add_argument("--compare-sequence", action="store_true",
                    help="only time tree against per-path attention on workloads 2..5, one JSON line each")
    return ap.parse_args()


def attn_bytes(w):
    """Algorithmic HBM bytes of one tree_attn_verify launch: every prefix and
    tree K/V row once, Q read once, O written once."""
    esz = 2 if w.dtype == "bf16" else 4
    kv = int(np.sum(w.prefix_len.astype(np.int64) + w.N)) * w.H * w.D * esz * 2
    qo = 2 * w.B * w.N * w.H * w.D * esz
    return kv + qo


def mask_bytes(w):
    """Algorithmic bytes of the mask part of tree_mask_attn_verify: parents
    read, ancestor and child masks, depths and status written, once each."""
    return w.B * w.N * 4 + w.B * w.N * 8 + w.B * (w.N + 1) * 8 + w.B * w.N * 4 + w.B * 4


def logit_bytes(w):
    """Algorithmic bytes of one verify call: every target row read once."""
    return w.B * (w.N + 1) * w.V * 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this benchmark measures one GPU; attention shards by head and verification by request)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mb or args.compare_sequence:
        import torch
        if args.copy_calibration_mb:
            copy_calibration(torch, args.copy_calibration_mb)
        else:
            compare_sequence_all(torch, [args.config] if args.config else [2, 3, 4, 5])
        return

    import synth
    w = synth.make_config(args.config or 4)
    note(f"built {w.name}")
    # The CPU oracle runs first, while no GPU context exists in this process,
    # so its all-cores leg can fork worker processes.
    cpu = None
    if not args.no_cpu and not args.profile_only:
        cpu = cpu_baseline(w, args.cpu_seconds)
        note("timed the CPU oracle")

    import torch
    import tree_speculative_verification_attn_amd as tv
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    res = run_workload(torch, tv, w, args, full=True)
    if res is None:                       # --profile-only
        return
    note(f"measured {w.name}")
    replays = {w.name: (w, res.pop("_mss_out"))} if cpu is not None else {}
    res.pop("_mss_out", None)
    if not args.no_others and args.config is None:
        others = {}
        for c in (2, 3, 5):
            wc = synth.make_config(c)
            others[wc.name] = run_workload(torch, tv, wc, args, full=False)
            out = others[wc.name].pop("_mss_out")
            if cpu is not None:
                replays[wc.name] = (wc, out)
            note(f"measured {wc.name}")
            del wc
            torch.cuda.empty_cache()
        # one GPU's share of the LLaMA-65B layer under 8-way tensor
        # parallelism over heads: every request, 8 of the 64 heads
        wc = synth.make_workload(4, H=8)
        others["llama65b_layer_tp8_shard"] = run_workload(torch, tv, wc, args, full=False)
        others["llama65b_layer_tp8_shard"].pop("_mss_out")
        note("measured llama65b_layer_tp8_shard")
        del wc
        torch.cuda.empty_cache()
        res["other_workloads"] = others
    res["roofline"]["measured_copy_ceiling_GBps"] = copy_ceiling(torch)
    res["roofline"]["frac_of_copy_ceiling"] = round(res["roofline"]["achieved"] /
                                                    res["roofline"]["measured_copy_ceiling_GBps"], 4)
    if cpu is not None:
        for leg in ("one_core", "all_cores"):
            cpu[leg]["gpu_over_cpu"] = round(res["value"] / cpu[leg]["value"], 1)
        # the oracle replays each workload's MSS call (after every GPU timing)
        cpu["mss_replay"] = {name: mss_replay(wr, out) for name, (wr, out) in replays.items()}
        res["cpu_baseline"] = cpu
    print(json.dumps(res))


def note(msg):
    """Progress on stderr; the JSON line alone goes to stdout."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def run_workload(torch, tv, w, args, full):
    """Time the step and its launches on one workload.  full: the headline
    line (with the verify variants, every entry point, tree against per-path
    attention, and the MSS outputs the oracle replays); otherwise a summary."""
    from synth.device import to_dev

    dev = "cuda:0"
    bf = w.dtype == "bf16"
    B, N, H, D, V, R = w.B, w.N, w.H, w.D, w.V, w.R
    step_bytes = w.k_cache.nbytes * 2 + w.target_logits.nbytes + w.ssm_probs.nbytes
    n_copies = max(2, int(np.ceil(2 * MALL_BYTES / max(1, step_bytes))) + 1)

    copies = []
    for _ in range(n_copies):
        copies.append(dict(q=to_dev(w.q, bf), k=to_dev(w.k_cache, bf), v=to_dev(w.v_cache, bf),
                           tl=to_dev(w.target_logits), sp=to_dev(w.ssm_probs)))
    bt = to_dev(w.block_table)
    pl0 = to_dev(w.prefix_len)
    pl0_all = pl0.repeat(n_copies, 1)
    pl_all = pl0_all.clone()                  # row c: prefix lengths of input copy c
    for c, cp in enumerate(copies):
        cp["pl"] = pl_all[c]
    parent = to_dev(w.parent)
    token = to_dev(w.token)
    qr = to_dev(w.q_row)
    anc = torch.zeros((B, N), dtype=torch.int64, device=dev)
    child = torch.zeros((B, N + 1), dtype=torch.int64, device=dev)
    depth = torch.zeros((B, N), dtype=torch.int32, device=dev)
    status = torch.zeros((B,), dtype=torch.int32, device=dev)
    out = torch.empty_like(copies[0]["q"])
    code = tv.TV_BF16 if bf else tv.TV_F32
    ws_a = tv.tree_attn_verify_workspace(code, B, N, H, D, w.max_blocks)
    ws_attn = torch.zeros(max(ws_a, 1), dtype=torch.uint8, device=dev) if ws_a else None
    ws_v = torch.zeros(tv.tree_verify_workspace(B, N, V), dtype=torch.uint8, device=dev)   # zero once; calls leave it zero
    g_acc = torch.empty((B, N), dtype=torch.int32, device=dev)
    g_num = torch.empty((B,), dtype=torch.int32, device=dev)
    g_bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    m_acc = torch.empty((B, N), dtype=torch.int32, device=dev)
    m_num = torch.empty((B,), dtype=torch.int32, device=dev)
    m_bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    m_rounds = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None, restore=True):
        c = copies[i % n_copies]
        cur = torch.cuda.current_stream()              # the capture stream inside a graph
        if restore:
            c["pl"].copy_(pl0)                         # the last commit on this copy grew it
        if ev: ev[0].record(cur)
        # the masks and the attention, in one launch
        tv.tree_mask_attn_verify(c["q"], c["k"], c["v"], bt, c["pl"], parent, anc, child, depth, status, out,
                                 ws_attn, scale=w.scale)
        if ev: ev[1].record(cur)
        tv.tree_verify_greedy(c["tl"], token, child, status, g_acc, g_num, g_bonus, ws_v)
        if ev: ev[2].record(cur)
        # MSS and the compaction of its path, in one launch
        tv.tree_verify_mss_commit(c["tl"], c["sp"], qr, token, child, status, w.seed, w.offset + i, m_acc,
                                  m_num, m_bonus, m_rounds, ws_v, c["k"], c["v"], bt, c["pl"])
        if ev: ev[3].record(cur)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.profile_only:
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        print(f"ran {args.warmup} + {args.steps} eager steps of {w.name}")
        return None

    # Eager pass with HIP events between the calls: per-call times on the
    # launch stream (the attention figure feeds the roofline).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    names = ["mask_attn", "greedy", "mss_commit"]
    comp = {n: float(np.mean([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(args.steps)]))
            for k, n in enumerate(names)}
    assert int((status != 0).sum()) == 0, "a request failed during the benchmark"

    # The timed loop: a HIP graph holds one step per input copy and then one
    # copy restoring every copy's prefix lengths; steps left over run from
    # one-step graphs that restore their own copy first.
    cycle, singles = None, []
    if not args.eager:
        cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cycle):
            for c in range(n_copies):
                step(c, restore=False)
            pl_all.copy_(pl0_all)
        for c in range(n_copies):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                step(c)
            singles.append(gph)
        cycle.replay()
        for gph in singles:
            gph.replay()
        pl_all.copy_(pl0_all)
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if cycle is not None:
        i = 0
        while i + n_copies <= args.steps:
            cycle.replay()
            i += n_copies
        for j in range(i, args.steps):
            singles[j % n_copies].replay()
    else:
        for i in range(args.steps):
            step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    acc_tokens = float(np.mean(np.maximum(m_num.cpu().numpy(), 0) + 1))
    assert int((status != 0).sum()) == 0, "a request failed during the benchmark"

    # Device time per launch of the dominant call (and of MSS): a graph of
    # back-to-back calls over the rotating input copies, timed with HIP
    # events on the stream the graph runs on.
    def per_call_ms(call, reps=10, use=None):
        use = copies if use is None else use
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for c in use * 2:
                call(c)
        gph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            gph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * 2 * len(use))

    pl_all.copy_(pl0_all)
    # the step's attention launch (masks built in the kernel), and the
    # attention alone for the comparison with per-path attention
    t_attn = per_call_ms(lambda c: tv.tree_mask_attn_verify(c["q"], c["k"], c["v"], bt, pl0, parent, anc, child,
                                                            depth, status, out, ws_attn, scale=w.scale))
    t_attn_only = per_call_ms(lambda c: tv.tree_attn_verify(c["q"], c["k"], c["v"], bt, pl0, anc, status, out,
                                                            ws_attn, scale=w.scale))
    # the same launch on one input copy over and over: warm caches (labelled,
    # not the roofline figure; the 256 MB Infinity Cache holds small workloads)
    t_attn_warm = per_call_ms(lambda c: tv.tree_mask_attn_verify(c["q"], c["k"], c["v"], bt, pl0, parent, anc,
                                                                 child, depth, status, out, ws_attn, scale=w.scale),
                              use=copies[:1])
    t_mss = per_call_ms(lambda c: tv.tree_verify_mss(c["tl"], c["sp"], qr, token, child, status, w.seed, w.offset,
                                                     m_acc, m_num, m_bonus, m_rounds, ws_v))
    assert int((status != 0).sum()) == 0, "a request failed during the benchmark"
    t_greedy = per_call_ms(lambda c: tv.tree_verify_greedy(c["tl"], token, child, status, g_acc, g_num, g_bonus, ws_v))
    a_bytes = attn_bytes(w) + mask_bytes(w)
    l_bytes = logit_bytes(w)
    attn_gbs = a_bytes / (t_attn * 1e-3) / 1e9
    mss_gbs = l_bytes / (t_mss * 1e-3) / 1e9
    value = B * N / (ms_per_step * 1e-3)

    # the MSS call the oracle replays: input copy 0, the workload's own
    # Philox key and offset, every request live
    st0 = torch.zeros((B,), dtype=torch.int32, device=dev)
    tv.tree_verify_mss(copies[0]["tl"], copies[0]["sp"], qr, token, child, st0, w.seed, w.offset, m_acc, m_num,
                       m_bonus, m_rounds, ws_v)
    torch.cuda.synchronize()
    mss_out = {k: t.cpu().numpy() for k, t in (("accepted", m_acc), ("num_accepted", m_num), ("bonus", m_bonus),
                                               ("rounds", m_rounds), ("status", st0))}
    if not full:
        del copies
        return {"workload": f"{w.name}: B={B} H={H} D={D} L={_lens(w)} N={N} V={V}",
                "ms_per_step": round(ms_per_step, 5), "verified_tree_tokens_per_s": round(value, 1),
                "attention": {"kernel": "tree_mask_attn_verify", "ms_per_launch": round(t_attn, 5),
                              "achieved_GBps": round(attn_gbs, 1), "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                              "algorithmic_bytes": a_bytes,
                              "tree_attn_verify_ms_per_launch": round(t_attn_only, 5),
                              "warm_cache_ms_per_launch": round(t_attn_warm, 5)},
                "mss": {"ms_per_launch": round(t_mss, 5), "achieved_GBps_on_logit_bytes": round(mss_gbs, 1),
                        "frac": round(mss_gbs / HBM_PEAK_GBS, 4), "logit_bytes": l_bytes},
                "greedy_ms_per_launch": round(t_greedy, 5),
                "tree_attn_plus_mss_tokens_per_s": round(B * N / ((t_attn + t_mss) * 1e-3), 1),
                "input_copies_rotated": n_copies, "_mss_out": mss_out}

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded NumPy; page-shaped, no model weights)",
        "config": {"workload": f"{w.name}: B={B} H={H} D={D} L={_lens(w)} N={N} V={V}",
                   "tree": str(w.meta.get("tree")), "batch": B, "tree_nodes": N,
                   "prefix_len_min": int(w.prefix_len.min()), "prefix_len_max": int(w.prefix_len.max()),
                   "prefix_len_mean": round(float(w.prefix_len.mean()), 2), "vocab": V,
                   "input_copies_rotated": n_copies},
        "roofline": {"bound": "hbm", "kernel": "tree_mask_attn_verify", "achieved": round(attn_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name), "algorithmic_bytes": a_bytes,
                     "ms_per_launch": round(t_attn, 5),
                     "tree_attn_verify_ms_per_launch": round(t_attn_only, 5),
                     "warm_cache_ms_per_launch": round(t_attn_warm, 5)},
        "eager_components_ms": {k: round(v, 5) for k, v in comp.items()},
        "launch": "eager" if args.eager else f"hip_graph_per_{n_copies}_steps",
        "eager_ms_per_step": round(eager_ms, 5),
        "mss": {"ms_per_launch": round(t_mss, 5), "achieved_GBps_on_logit_bytes": round(mss_gbs, 1),
                "frac": round(mss_gbs / HBM_PEAK_GBS, 4), "logit_bytes": l_bytes,
                "tree_attn_plus_mss_tokens_per_s": round(B * N / ((t_attn + t_mss) * 1e-3), 1),
                "mean_tokens_emitted_per_request": round(acc_tokens, 3)},
    }
    variants = verify_variants(torch, tv, w, copies, per_call_ms, qr, token, child, status, ws_v, t_mss, t_greedy)
    res["verify_variants"] = variants
    res["per_call_ms"] = per_call_table(torch, tv, w, copies, per_call_ms, pl0, parent, anc, child, depth, status,
                                        token, qr, bt, m_acc, m_num, m_bonus, m_rounds, ws_v, t_attn, t_attn_only,
                                        t_mss, variants)
    res["tree_vs_sequence"] = tree_vs_sequence(torch, tv, w, copies, bt, t_attn_only, stream)
    res["_mss_out"] = mss_out
    del copies
    torch.cuda.empty_cache()
    return res


def _lens(w):
    lo, hi = int(w.prefix_len.min()), int(w.prefix_len.max())
    return str(hi) if lo == hi else f"{lo}..{hi}"


def verify_variants(torch, tv, w, copies, per_call_ms, qr, token, child, status, ws_v, t_mss, t_greedy):
    """The Table 3 analogue on this synthetic workload (SpecInfer summary,
    Theorem 4.3 and Table 3: MSS against naive sampling, tokens per step), the
    greedy rule beside them, and the cost of a sampling transform of every
    target row (temperature 0.8, top-k 50, top-p 0.9)."""
    dev = "cuda:0"
    B, N = w.B, w.N
    acc = torch.empty((B, N), dtype=torch.int32, device=dev)
    num = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    rounds = torch.empty((B,), dtype=torch.int32, device=dev)
    reps = 64
    tokens = {"mss": 0.0, "naive": 0.0, "greedy": 0.0}
    for i in range(reps):                 # fresh random streams: offsets 1000 + i
        c = copies[i % len(copies)]
        tv.tree_verify_mss(c["tl"], c["sp"], qr, token, child, status, w.seed, 1000 + i, acc, num, bonus,
                           rounds, ws_v)
        tokens["mss"] += float((num.clamp(min=0) + 1).float().mean())
        tv.tree_verify_naive(c["tl"], token, child, status, w.seed, 1000 + i, acc, num, bonus, ws_v)
        tokens["naive"] += float((num.clamp(min=0) + 1).float().mean())
    tv.tree_verify_greedy(copies[0]["tl"], token, child, status, acc, num, bonus, ws_v)
    tokens["greedy"] = float((num.clamp(min=0) + 1).float().mean()) * reps
    t_naive = per_call_ms(lambda c: tv.tree_verify_naive(c["tl"], token, child, status, w.seed, w.offset,
                                                         acc, num, bonus, ws_v))
    scratch = torch.empty_like(copies[0]["tl"])
    t_tf = per_call_ms(lambda c: tv.tree_logits_transform(c["tl"], scratch, 0.8, 50, 0.9, tv.TV_OUT_LOGITS))
    assert int((status != 0).sum()) == 0, "a request failed in the verify variants"
    return {"tokens_per_step": {k: round(v / reps, 4) for k, v in tokens.items()},
            "mss_over_naive": round(tokens["mss"] / tokens["naive"], 4),
            "ms_per_launch": {"mss": round(t_mss, 5), "naive": round(t_naive, 5), "greedy": round(t_greedy, 5)},
            "sampling_transform_ms": round(t_tf, 5),
            "sampling_transform": f"tree_logits_transform of all {B * (N + 1)} target rows, T 0.8, top-k 50, top-p 0.9",
            "note": "synthetic rows (draft = target + noise); tokens per step = accepted + bonus, mean over "
                    f"{reps} random streams"}


def per_call_table(torch, tv, w, copies, per_call_ms, pl0, parent, anc, child, depth, status, token, qr, bt,
                   m_acc, m_num, m_bonus, m_rounds, ws_v, t_attn, t_attn_only, t_mss, variants):
    """Every entry point on this workload, per call, from graphs of
    back-to-back calls over the rotating input copies.  The two calls that
    grow the prefix lengths are timed as (restore + call) minus (restore
    alone), so each call sees the same lengths; kv_commit_accepted moves the
    path of the benchmark's last MSS call."""
    t_mask = per_call_ms(lambda c: tv.tree_build_mask(parent, anc, child, depth, status))
    t_restore = per_call_ms(lambda c: c["pl"].copy_(pl0))
    t_commit = per_call_ms(lambda c: (c["pl"].copy_(pl0),
                                      tv.kv_commit_accepted(c["k"], c["v"], bt, c["pl"], m_acc, m_num, status)))
    acc = torch.empty_like(m_acc)
    num = torch.empty_like(m_num)
    bonus = torch.empty_like(m_bonus)
    rounds = torch.empty_like(m_rounds)
    t_mss_commit = per_call_ms(lambda c: (c["pl"].copy_(pl0),
                                          tv.tree_verify_mss_commit(c["tl"], c["sp"], qr, token, child, status, w.seed,
                                                                    w.offset, acc, num, bonus, rounds, ws_v, c["k"],
                                                                    c["v"], bt, c["pl"])))
    for cp in copies:
        cp["pl"].copy_(pl0)
    assert int((status != 0).sum()) == 0, "a request failed in the per-call timings"
    ml = variants["ms_per_launch"]
    return {"tree_build_mask": round(t_mask, 5), "tree_attn_verify": round(t_attn_only, 5),
            "tree_mask_attn_verify": round(t_attn, 5), "tree_verify_greedy": ml["greedy"],
            "tree_verify_mss": round(t_mss, 5), "tree_verify_naive": ml["naive"],
            "kv_commit_accepted": round(t_commit - t_restore, 5),
            "tree_verify_mss_commit": round(t_mss_commit - t_restore, 5),
            "tree_logits_transform": variants["sampling_transform_ms"],
            "prefix_len_restore": round(t_restore, 5)}


def compare_sequence_all(torch, cfgs):
    """Tree against per-path attention on the given workloads (one JSON line each)."""
    import synth
    import tree_speculative_verification_attn_amd as tv
    from synth.device import to_dev
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    for cfg in cfgs:
        w = synth.make_config(cfg)
        bf = w.dtype == "bf16"
        n_copies = max(2, int(np.ceil(2 * MALL_BYTES / max(1, w.k_cache.nbytes * 2))) + 1)
        copies = [dict(q=to_dev(w.q, bf), k=to_dev(w.k_cache, bf), v=to_dev(w.v_cache, bf))
                  for _ in range(n_copies)]
        bt, pl = to_dev(w.block_table), to_dev(w.prefix_len)
        anc = torch.zeros((w.B, w.N), dtype=torch.int64, device=dev)
        child = torch.zeros((w.B, w.N + 1), dtype=torch.int64, device=dev)
        depth = torch.zeros((w.B, w.N), dtype=torch.int32, device=dev)
        st = torch.zeros((w.B,), dtype=torch.int32, device=dev)
        tv.tree_build_mask(to_dev(w.parent), anc, child, depth, st)
        code = tv.TV_BF16 if bf else tv.TV_F32
        n = tv.tree_attn_verify_workspace(code, w.B, w.N, w.H, w.D, w.max_blocks)
        ws = torch.zeros(n, dtype=torch.uint8, device=dev) if n else None
        out = torch.empty_like(copies[0]["q"])

        def call(c):
            tv.tree_attn_verify(c["q"], c["k"], c["v"], bt, pl, anc, st, out, ws, scale=w.scale)

        for c in copies:
            call(c)
        torch.cuda.synchronize()
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for c in copies * 2:
                call(c)
        gph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            gph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t_tree = e0.elapsed_time(e1) / (5 * 2 * n_copies)
        assert int((st != 0).sum()) == 0
        del gph
        r = tree_vs_sequence(torch, tv, w, copies, bt, t_tree, stream, reps=5)
        r["workload"] = f"{w.name}: B={w.B} H={w.H} D={w.D} N={w.N} L_max={int(w.prefix_len.max())}"
        print(json.dumps(r), flush=True)
        del copies, ws, out
        torch.cuda.empty_cache()


def tree_vs_sequence(torch, tv, w, copies, bt, t_tree, stream, reps=10):
    """Tree attention against sequence-based verification of the same tree
    (SpecInfer summary, "Evaluation", Figure 11): every root-to-leaf path as a
    chain of its own over the same prefix blocks, through the same attention
    kernel, timed like the tree call (a graph of back-to-back calls over the
    rotating input copies)."""
    from tree_speculative_verification_attn_amd import per_sequence
    dev = "cuda:0"
    sbs = [per_sequence.build(w.parent, w.prefix_len, c["q"], c["k"], c["v"], bt) for c in copies]
    S, N2 = sbs[0].S, sbs[0].N
    anc = torch.zeros((S, N2), dtype=torch.int64, device=dev)
    child = torch.zeros((S, N2 + 1), dtype=torch.int64, device=dev)
    depth = torch.zeros((S, N2), dtype=torch.int32, device=dev)
    st = torch.zeros((S,), dtype=torch.int32, device=dev)
    tv.tree_build_mask(sbs[0].parent, anc, child, depth, st)
    code = tv.TV_BF16 if w.dtype == "bf16" else tv.TV_F32
    n = tv.tree_attn_verify_workspace(code, S, N2, w.H, w.D, sbs[0].block_table.shape[1])
    ws = torch.zeros(n, dtype=torch.uint8, device=dev) if n else None
    out = torch.empty_like(sbs[0].q)

    def call(sb):
        tv.tree_attn_verify(sb.q, sb.k_cache, sb.v_cache, sb.block_table, sb.prefix_len, anc, st, out, ws,
                            scale=w.scale)

    for sb in sbs:
        call(sb)
    torch.cuda.synchronize()
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        for sb in sbs * 2:
            call(sb)
    gph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        gph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t_seq = e0.elapsed_time(e1) / (reps * 2 * len(sbs))
    assert int((st != 0).sum()) == 0, "a per-path request failed"
    esz = 2 if w.dtype == "bf16" else 4
    tree_kv = int(np.sum(w.prefix_len.astype(np.int64) + w.N)) * w.H * w.D * esz * 2
    return {"paths": S, "longest_path": N2, "tree_ms": round(t_tree, 5), "sequence_ms": round(t_seq, 5),
            "tree_speedup": round(t_seq / t_tree, 3), "tree_kv_bytes": tree_kv,
            "sequence_kv_bytes": sbs[0].kv_bytes,
            "kernel": "tree_attn_verify for both; paths share the physical prefix blocks"}


def copy_ceiling(torch, mib=1024, reps=20):
    """GB/s of a plain device-to-device copy of `mib` MiB (bytes read plus
    bytes written over the time), timed with HIP events on the current
    stream: the practical HBM ceiling the roofline fraction is read against."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def copy_calibration(torch, mib):
    """Five plain device-to-device copies of `mib` MiB: the reference that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB 5 times")


ATTN_SOURCES = ("tree_speculative_verification_attn_amd/csrc/attn.hip",
                "tree_speculative_verification_attn_amd/csrc/tv_common.h",
                "tree_speculative_verification_attn_amd/csrc/tree_mask.h")


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per attention launch of the step from the committed counter
    summary of this workload, or None when there is none or the attention
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"tree_attn_verify_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("attn_source_sha256") != attn_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


_CPU = {}          # the workload and its masks, inherited by forked workers


def _cpu_init():
    import threadpoolctl
    _CPU["limit"] = threadpoolctl.threadpool_limits(1)


def _cpu_attn(pairs):
    from oracle import attention
    w, anc, st = _CPU["w"], _CPU["anc"], _CPU["st"]
    t = time.perf_counter()
    for b, h in pairs:
        attention.tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len, anc, st,
                                 w.dtype, w.scale, pairs=[(b, h)])
    return time.perf_counter() - t


def _cpu_verify(reqs):
    from oracle import verify
    w = _CPU["w"]
    t = time.perf_counter()
    for r in reqs:
        verify.verify_greedy(w.parent[r:r + 1], w.token[r:r + 1], w.target_logits[r:r + 1], [0])
        verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B,
                          w.seed, w.offset, requests=[r])
    return time.perf_counter() - t


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers and clock (a virtual machine may report only a brand)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                       # the first processor's block is enough
                key, _, val = line.partition(":")
                info[key.strip()] = val.strip()
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    if "cpu MHz" in info:
        ids.append(f"{float(info['cpu MHz']):.0f} MHz")
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(w, budget_s):
    """The float64 oracle on a bounded sample of the same workload, scaled to
    one whole step, on one core and on all the cores this process may use (at
    most 16, one worker process per core, each with one BLAS thread).
    Attention is timed on (request, head) pairs drawn at random, verification
    (greedy + MSS) on requests taken in turn; each leg spends about budget_s
    seconds of wall time."""
    import multiprocessing

    import threadpoolctl

    from oracle import tree

    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads by default)"
            for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    anc, child, depth, st = tree.build_mask_batch(w.parent)
    _CPU.update(w=w, anc=anc, st=st)
    rng = np.random.default_rng(0)
    pair_stream = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4096)]

    # one core
    with threadpoolctl.threadpool_limits(1):
        t = time.perf_counter()
        tree.build_mask_batch(w.parent)
        t_mask = time.perf_counter() - t
        n_pairs, t_attn = 0, 0.0
        while t_attn < budget_s * 0.65 and n_pairs < len(pair_stream):
            t_attn += _cpu_attn(pair_stream[n_pairs:n_pairs + 1])
            n_pairs += 1
        n_reqs, t_ver = 0, 0.0
        while t_ver < budget_s * 0.35:
            t_ver += _cpu_verify([n_reqs % w.B])
            n_reqs += 1
    step1 = t_mask + t_attn / n_pairs * (w.B * w.H) + t_ver / n_reqs * w.B
    one = {"value": round(w.B * w.N / step1, 3), "unit": "verified tree tokens/s", "cores": 1,
           "step_s": round(step1, 3),
           "sample": f"{n_pairs} (request, head) pairs of {w.B * w.H} drawn at random, greedy + MSS on "
                     f"{n_reqs} requests of {w.B} in turn, masks for all requests; "
                     f"{t_mask + t_attn + t_ver:.1f} s of work"}

    # all cores: the same units spread over worker processes
    cores = min(16, len(os.sched_getaffinity(0)))
    per_pair, per_req = t_attn / n_pairs, t_ver / n_reqs
    k_pairs = max(cores, int(budget_s * 0.65 * cores / per_pair))
    k_reqs = max(cores, int(budget_s * 0.35 * cores / per_req))
    while len(pair_stream) < n_pairs + k_pairs:
        pair_stream.append((int(rng.integers(w.B)), int(rng.integers(w.H))))
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(cores, initializer=_cpu_init) as pool:
        pool.map(_cpu_attn, [pair_stream[i:i + 1] for i in range(cores)])       # workers up
        chunks = [pair_stream[n_pairs + i:n_pairs + k_pairs:cores] for i in range(cores)]
        t = time.perf_counter()
        pool.map(_cpu_attn, chunks, chunksize=1)
        wall_attn = time.perf_counter() - t
        reqs = [(n_reqs + i) % w.B for i in range(k_reqs)]
        t = time.perf_counter()
        pool.map(_cpu_verify, [reqs[i::cores] for i in range(cores)], chunksize=1)
        wall_ver = time.perf_counter() - t
    stepn = t_mask + wall_attn / k_pairs * (w.B * w.H) + wall_ver / k_reqs * w.B
    alln = {"value": round(w.B * w.N / stepn, 3), "unit": "verified tree tokens/s", "cores": cores,
            "step_s": round(stepn, 3),
            "sample": f"{k_pairs} (request, head) pairs and {k_reqs} requests over {cores} worker processes "
                      f"(one BLAS thread each), {wall_attn + wall_ver:.1f} s wall; masks as one core"}
    return {"value": alln["value"], "unit": "verified tree tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 NumPy oracle of {w.name}, scaled from a bounded sample to one full step; "
                      f"all-cores leg: {alln['sample']}",
            "one_core": one, "all_cores": alln, "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(), "cpus_usable": len(os.sched_getaffinity(0)),
            "blas": "; ".join(blas) or "none found"}


NEAR_TIE = 1e-6


def mss_replay(w, dev_out):
    """The oracle's MSS walk of every request of the step's MSS call (the
    workload's key and offset) against the device's outputs.  A request
    counts as a near tie when it differs and the oracle's walk with one
    decision of margin below 1e-6 taken the other way gives the device's
    result; anything else is a mismatch."""
    from oracle import verify
    t = time.perf_counter()
    ref = verify.verify_mss(w.parent, w.token, w.target_logits, w.ssm_probs, w.q_row, [0] * w.B, w.seed, w.offset)
    exact = near = 0
    bad = []
    for b in range(w.B):
        def same(r, b=b):
            return (dev_out["num_accepted"][b] == r["num_accepted"][b] and dev_out["bonus"][b] == r["bonus"][b]
                    and dev_out["rounds"][b] == r["rounds"][b] and dev_out["status"][b] == r["status"][b]
                    and np.array_equal(dev_out["accepted"][b], r["accepted"][b]))
        if same(ref):
            exact += 1
            continue
        margins = [m for _, m in ref["traces"][b] if m is not None]
        if any(m < NEAR_TIE and same(ref["redo"](b, k)) for k, m in enumerate(margins)):
            near += 1
        else:
            bad.append(b)
    return {"requests": w.B, "exact": exact, "near_tie": near, "mismatch": len(bad), "mismatched_requests": bad,
            "oracle_s": round(time.perf_counter() - t, 2)}


if __name__ == "__main__":
    main()
