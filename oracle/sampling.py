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

Precision reading: the rows are fp32, so the scaled logit is the fp32 product
l' = fp32(l * fp32(1 / T)) (exact for T = 1), and ranks, masses and outputs
are taken from l'.  A consumer of the "logits" output then sees exactly these
fp32 values.
"""
import numpy as np


def scaled(logits_row, temperature):
    """l' = fp32(l * fp32(1/T)) as float64 (non-finite entries pass through)."""
    l32 = np.asarray(logits_row, dtype=np.float32)
    inv = np.float32(1.0) / np.float32(temperature)
    with np.errstate(invalid="ignore", over="ignore"):
        return (l32 * inv).astype(np.float32).astype(np.float64)


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
