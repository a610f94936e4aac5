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
    +inf entry, or with no finite entry, becomes all NaN.
Outputs: kind "logits" gives l / T where kept and -inf elsewhere (a softmax of
it is the transformed distribution); kind "probs" gives the normalised kept
probabilities and 0 elsewhere.
"""
import numpy as np


def _f64(logits_row):
    return np.asarray(logits_row, dtype=np.float32).astype(np.float64)


def kept_in_rank_order(logits_row, temperature=1.0, top_k=0, top_p=1.0):
    """The kept entries, largest first (ties: lower index first), or None for
    an invalid row."""
    l = _f64(logits_row)
    if np.isnan(l).any() or np.isposinf(l).any() or not np.isfinite(l).any():
        return None
    order = sorted(np.nonzero(np.isfinite(l))[0].tolist(), key=lambda x: (-l[x], x))
    if top_k > 0:
        order = order[:top_k]
    if top_p < 1.0:
        mass = np.exp((l[order] - l[order[0]]) / temperature)
        target = top_p * mass.sum()
        csum = np.cumsum(mass)
        reach = np.nonzero(csum >= target)[0]
        order = order[: int(reach[0]) + 1 if len(reach) else len(order)]
    return order


def transform_row(logits_row, temperature=1.0, top_k=0, top_p=1.0, kind="logits"):
    """One transformed row (float64)."""
    l = _f64(logits_row)
    keep = kept_in_rank_order(l, temperature, top_k, top_p)
    if keep is None:
        return np.full(l.shape, np.nan)
    keep = np.asarray(keep, dtype=np.int64)
    if kind == "logits":
        out = np.full(l.shape, -np.inf)
        out[keep] = l[keep] / temperature
        return out
    e = np.exp((l[keep] - l[keep].max()) / temperature)
    out = np.zeros(l.shape)
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
    l = _f64(logits_row)
    keep = kept_in_rank_order(l, temperature, top_k, 1.0)
    if keep is None or top_p >= 1.0:
        return np.inf
    mass = np.exp((l[keep] - l[keep[0]]) / temperature)
    csum = np.cumsum(mass)
    return float(np.min(np.abs(csum - top_p * csum[-1])) / csum[-1])
