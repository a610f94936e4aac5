"""Sampling transforms applied before verification (oracle side, float64).
Test infrastructure: only tests, smoke() and the benchmark's CPU baseline use
this package.

Source: wiki concept page "Speculative decoding", "Implementation sketch": the
lossless acceptance rule holds for any sampling distribution, so temperature,
top-k and top-p are applied to both the target's and the draft's distribution
before the rule.

The page names the transforms without defining them; the readings here are
the usual definitions:
  * temperature T > 0: p(x) proportional to exp(l(x) / T);
  * top-k, k > 0: keep the k largest logits, ties going to the lower index;
    k = 0, or k at least the number of finite entries, keeps every finite one;
  * top-p, 0 < p < 1: of the entries top-k kept, keep the smallest set of
    largest probabilities (ties: lower index first) whose mass reaches p times
    the mass top-k kept; p = 1 keeps them all;
  * order: temperature, then top-k, then top-p (top-k on logits does not
    depend on T);
  * -inf entries have probability 0 and are never kept; a row with a NaN or
    +inf entry, or with no finite entry, becomes all NaN (judged on the scaled
    values below, so a finite logit that the scaling overflows counts too).
Outputs: kind "logits" gives the scaled logits where kept and -inf elsewhere
(a softmax of them is the transformed distribution); kind "probs" gives the
normalised kept probabilities and 0 elsewhere.

Precision reading: the scaled logit is l / T, exact in float64 (l is an fp32
row, so the quotient is exact up to float64 rounding); ranks, masses and
outputs are taken from it.  The output is an fp32 row, so a scaled value
beyond the fp32 range acts as its fp32 rounding would: above it, +inf (the
row is invalid); below minus it, -inf (the entry has probability 0 and is
never kept).  A device that rounds the scaled logits to fp32 can then differ
from this only at rounding-level ties: two entries whose fp32 scaled values
coincide at the top-k cut, or a top-p target within rounding of a cumulative
mass.
"""
import numpy as np


FP32_MAX = float(np.finfo(np.float32).max)
FP32_HALF_ULP_AT_MAX = 2.0 ** 103          # values below FP32_MAX + this round to FP32_MAX


def scaled(logits_row, temperature):
    """l / T in float64; non-finite entries pass through, and values beyond
    the fp32 range become the infinity fp32 rounding would give."""
    l = np.asarray(logits_row, dtype=np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        x = l / float(temperature)
    lim = FP32_MAX + FP32_HALF_ULP_AT_MAX
    x = np.where(np.isfinite(x) & (x >= lim), np.inf, x)
    x = np.where(np.isfinite(x) & (x <= -lim), -np.inf, x)
    return x


def rounding_tie_at_topk(logits_row, temperature, top_k):
    """True when the k-th and (k+1)-th ranked scaled logits are within fp32
    rounding of each other (relative 2^-22): the cut is then a tie that a
    device rounding the scaled values to fp32 may settle either way."""
    if top_k <= 0:
        return False
    l = scaled(logits_row, temperature)
    fin = np.sort(l[np.isfinite(l)])[::-1]
    if len(fin) <= top_k:
        return False
    a, b = fin[top_k - 1], fin[top_k]
    return abs(a - b) <= 2.0 ** -22 * max(abs(a), abs(b))


def kept_in_rank_order(logits_row, temperature=1.0, top_k=0, top_p=1.0):
    """The kept entries, largest first (ties: lower index first), or None for
    an invalid row."""
    l = scaled(logits_row, temperature)
    if np.isnan(l).any() or np.isposinf(l).any() or not np.isfinite(l).any():
        return None
    order = sorted(np.nonzero(np.isfinite(l))[0].tolist(), key=lambda x: (-l[x], x))
    if top_k > 0:
        order = order[:top_k]
    if top_p < 1.0:
        mass = np.exp(l[order] - l[order[0]])
        target = top_p * mass.sum()
        csum = np.cumsum(mass)
        reach = np.nonzero(csum >= target)[0]
        order = order[: int(reach[0]) + 1 if len(reach) else len(order)]
    return order


def transform_row(logits_row, temperature=1.0, top_k=0, top_p=1.0, kind="logits"):
    """One transformed row (float64)."""
    raw = np.asarray(logits_row, dtype=np.float32)
    keep = kept_in_rank_order(raw, temperature, top_k, top_p)
    if keep is None:
        return np.full(raw.shape, np.nan)
    keep = np.asarray(keep, dtype=np.int64)
    l = scaled(raw, temperature)
    if kind == "logits":
        out = np.full(raw.shape, -np.inf)
        out[keep] = l[keep]
        return out
    e = np.exp(l[keep] - l[keep].max())
    out = np.zeros(raw.shape)
    out[keep] = e / e.sum()
    return out


def transform(rows, temperature=1.0, top_k=0, top_p=1.0, kind="logits"):
    """transform_row over the last axis of an array of rows."""
    rows = np.asarray(rows)
    flat = rows.reshape(-1, rows.shape[-1])
    out = np.stack([transform_row(r, temperature, top_k, top_p, kind) for r in flat])
    return out.reshape(rows.shape)


def top_p_margin(logits_row, temperature, top_k, top_p):
    """Distance, relative to the kept mass, of the top-p target to the nearest
    cumulative mass in rank order (rounding can move the cut when it is tiny)."""
    keep = kept_in_rank_order(logits_row, temperature, top_k, 1.0)
    if keep is None or top_p >= 1.0:
        return np.inf
    l = scaled(logits_row, temperature)
    mass = np.exp(l[keep] - l[keep[0]])
    csum = np.cumsum(mass)
    return float(np.min(np.abs(csum - top_p * csum[-1])) / csum[-1])
