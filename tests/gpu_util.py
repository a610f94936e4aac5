"""Helpers for GPU tests: move a synthetic workload to the device, run each
verification step through the C-ABI binding, and compare with the oracle."""
import numpy as np
import torch

import tree_speculative_verification_attn_amd as tv
from oracle import attention as o_attn
from oracle import commit as o_commit
from oracle import tree as o_tree
from oracle import verify as o_verify
from synth.device import DEV, to_dev


def u64(t):
    """int64 device tensor holding uint64 bit patterns -> numpy uint64."""
    return t.cpu().numpy().view(np.uint64)


class DeviceRun:
    """One workload on the device plus the outputs of each call."""

    def __init__(self, w):
        self.w = w
        bf = w.dtype == "bf16"
        self.q = to_dev(w.q, bf)
        self.k = to_dev(w.k_cache, bf)
        self.v = to_dev(w.v_cache, bf)
        self.bt = to_dev(w.block_table)
        self.pl = to_dev(w.prefix_len)
        self.parent = to_dev(w.parent)
        self.token = to_dev(w.token)
        self.tl = to_dev(w.target_logits)
        self.sp = to_dev(w.ssm_probs)
        self.qr = to_dev(w.q_row)
        B, N = w.B, w.N
        self.anc = torch.zeros((B, N), dtype=torch.int64, device=DEV)
        self.child = torch.zeros((B, N + 1), dtype=torch.int64, device=DEV)
        self.depth = torch.zeros((B, N), dtype=torch.int32, device=DEV)
        self.status = torch.full((B,), -99, dtype=torch.int32, device=DEV)

    def mask(self):
        tv.tree_build_mask(self.parent, self.anc, self.child, self.depth, self.status)
        return self

    def attn(self):
        w = self.w
        code = tv.TV_BF16 if w.dtype == "bf16" else tv.TV_F32
        ws = tv.tree_attn_verify_workspace(code, w.B, w.N, w.H, w.D, w.max_blocks)
        self.ws_attn = torch.zeros(max(ws, 1), dtype=torch.uint8, device=DEV)   # counters start at 0
        self.out = torch.empty_like(self.q)
        tv.tree_attn_verify(self.q, self.k, self.v, self.bt, self.pl, self.anc, self.status, self.out,
                            self.ws_attn if ws else None, scale=w.scale)
        return self

    def mask_attn(self):
        """tree_mask_attn_verify: the masks and the attention in one call."""
        w = self.w
        code = tv.TV_BF16 if w.dtype == "bf16" else tv.TV_F32
        ws = tv.tree_attn_verify_workspace(code, w.B, w.N, w.H, w.D, w.max_blocks)
        self.ws_attn = torch.zeros(max(ws, 1), dtype=torch.uint8, device=DEV)
        self.out = torch.empty_like(self.q)
        tv.tree_mask_attn_verify(self.q, self.k, self.v, self.bt, self.pl, self.parent, self.anc, self.child,
                                 self.depth, self.status, self.out, self.ws_attn if ws else None, scale=w.scale)
        return self

    def _ws_verify(self):
        """One verify workspace for every verify call of this run: zeroed once
        at allocation, and each completed call leaves it zeroed again."""
        if getattr(self, "ws_v", None) is None:
            w = self.w
            n = tv.tree_verify_workspace(w.B, w.N, w.V)
            self.ws_v = torch.zeros(max(n, 1), dtype=torch.uint8, device=DEV)
        return self.ws_v

    def greedy(self):
        w = self.w
        self.g_acc = torch.empty((w.B, w.N), dtype=torch.int32, device=DEV)
        self.g_num = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.g_bonus = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        tv.tree_verify_greedy(self.tl, self.token, self.child, self.status, self.g_acc, self.g_num,
                              self.g_bonus, self._ws_verify())
        return self

    def mss(self, seed=None, offset=None):
        w = self.w
        self.m_acc = torch.empty((w.B, w.N), dtype=torch.int32, device=DEV)
        self.m_num = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.m_bonus = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.m_rounds = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        tv.tree_verify_mss(self.tl, self.sp, self.qr, self.token, self.child, self.status,
                           w.seed if seed is None else seed, w.offset if offset is None else offset,
                           self.m_acc, self.m_num, self.m_bonus, self.m_rounds, self._ws_verify())
        return self

    def mss_commit(self, seed=None, offset=None):
        """tree_verify_mss and the commit of its path in one call."""
        w = self.w
        self.m_acc = torch.empty((w.B, w.N), dtype=torch.int32, device=DEV)
        self.m_num = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.m_bonus = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.m_rounds = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        tv.tree_verify_mss_commit(self.tl, self.sp, self.qr, self.token, self.child, self.status,
                                  w.seed if seed is None else seed, w.offset if offset is None else offset,
                                  self.m_acc, self.m_num, self.m_bonus, self.m_rounds, self._ws_verify(),
                                  self.k, self.v, self.bt, self.pl)
        return self

    def mss_multi(self, prop_node, prop_row, seed=None, offset=None):
        """MSS over proposal lists (numpy [B][S] int arrays)."""
        w = self.w
        self.m_acc = torch.empty((w.B, w.N), dtype=torch.int32, device=DEV)
        self.m_num = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.m_bonus = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.m_rounds = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        tv.tree_verify_mss_multi(self.tl, self.sp, to_dev(np.asarray(prop_node, dtype=np.int32)),
                                 to_dev(np.asarray(prop_row, dtype=np.int32)), self.token, self.child, self.status,
                                 w.seed if seed is None else seed, w.offset if offset is None else offset,
                                 self.m_acc, self.m_num, self.m_bonus, self.m_rounds, self._ws_verify())
        return self

    def naive(self, seed=None, offset=None):
        w = self.w
        self.n_acc = torch.empty((w.B, w.N), dtype=torch.int32, device=DEV)
        self.n_num = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        self.n_bonus = torch.empty((w.B,), dtype=torch.int32, device=DEV)
        tv.tree_verify_naive(self.tl, self.token, self.child, self.status,
                             w.seed if seed is None else seed, w.offset if offset is None else offset,
                             self.n_acc, self.n_num, self.n_bonus, self._ws_verify())
        return self

    def commit(self, accepted, num_accepted):
        tv.kv_commit_accepted(self.k, self.v, self.bt, self.pl, accepted, num_accepted, self.status)
        return self


def bf16_tol_check(got, ref, atol, rtol):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    return int(bad.sum()), float(err.max()) if err.size else 0.0


def out_to_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


NEAR_TIE = 1e-6


def _near_tie_excused(ref, b, same):
    """True iff the oracle's walk of request b, with one of its near-tie
    decisions (margin < 1e-6) taken the other way, gives the device's result
    (`same` compares one request of an oracle result with the device's).
    Everything before the flipped decision is the oracle's own walk, so the
    device's result then first departs from the oracle at that near tie."""
    margins = [m for _, m in ref["traces"][b] if m is not None]
    for k, m in enumerate(margins):
        if m < NEAR_TIE and same(ref["redo"](b, k)):
            return True
    return False


def compare_mss(run, ref):
    """Compare GPU MSS outputs with the oracle.  A request may differ only
    where its first divergent decision is a near tie of the oracle's walk
    (|u - ratio| < 1e-6, or a draw within 1e-6 of a cumulative-sum boundary):
    the oracle's walk with that one decision flipped must give the device's
    result.  Returns (n_exact, n_near_tie_excused, list of unexcused request
    ids)."""
    acc = run.m_acc.cpu().numpy()
    num = run.m_num.cpu().numpy()
    bonus = run.m_bonus.cpu().numpy()
    rounds = run.m_rounds.cpu().numpy()
    st = run.status.cpu().numpy()
    exact = excused = 0
    bad = []
    for b in range(len(num)):
        def same(r, b=b):
            return (num[b] == r["num_accepted"][b] and bonus[b] == r["bonus"][b]
                    and rounds[b] == r["rounds"][b] and st[b] == r["status"][b]
                    and np.array_equal(acc[b], r["accepted"][b]))
        if same(ref):
            exact += 1
        elif _near_tie_excused(ref, b, same):
            excused += 1
        else:
            bad.append(b)
    return exact, excused, bad


def compare_naive(run, ref):
    """Naive verification against the oracle: exact, except requests whose
    first divergent draw is within 1e-6 of a cumulative-mass boundary (as
    compare_mss).  Returns (n_exact, n_near_tie_excused, list of unexcused
    request ids)."""
    acc, num, bonus, st = (t.cpu().numpy() for t in (run.n_acc, run.n_num, run.n_bonus, run.status))
    exact = excused = 0
    bad = []
    for b in range(len(num)):
        def same(r, b=b):
            return (num[b] == r["num_accepted"][b] and bonus[b] == r["bonus"][b] and st[b] == r["status"][b]
                    and np.array_equal(acc[b], r["accepted"][b]))
        if same(ref):
            exact += 1
        elif _near_tie_excused(ref, b, same):
            excused += 1
        else:
            bad.append(b)
    return exact, excused, bad


def oracle_masks(w):
    return o_tree.build_mask_batch(w.parent)


__all__ = ["DeviceRun", "to_dev", "u64", "compare_mss", "compare_naive", "bf16_tol_check", "out_to_f64", "oracle_masks",
           "o_attn", "o_commit", "o_tree", "o_verify", "DEV"]
