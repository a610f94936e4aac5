"""Keep only the accepted path's KV entries (oracle side).

Sources: SpecInfer summary, "KV-cache for verified tokens" (after
verification only the accepted tokens keep their cache entries; rejected
ones are discarded); wiki concept page "Speculative decoding",
"Implementation sketch" step 4 and "KV-cache rollback" (the accepted path's
entries are compacted into contiguous slots).

For request b with prefix length L and accepted node ids a_0..a_{k-1}: the
entry of logical slot L + a_j moves to slot L + j for every head (K and V),
then L grows by k.  Reads all use the pre-call cache contents.  Requests with
nonzero status or num_accepted < 0 are left alone.
"""
import numpy as np

from .status import ST_OK, ST_KV_CAPACITY, ST_BAD_BLOCK, ST_BAD_ACCEPTED

BLOCK = 16


def commit_status(block_table_row, L, N, num_blocks, accepted_row, k):
    if L < 0 or L + N > len(block_table_row) * BLOCK:
        return ST_KV_CAPACITY
    # the blocks holding the tree slots L .. L+N-1 (the only ones the move touches)
    if N > 0 and any(not (0 <= int(block_table_row[j]) < num_blocks)
                     for j in range(L // BLOCK, (L + N - 1) // BLOCK + 1)):
        return ST_BAD_BLOCK
    if k > N or any(not (0 <= int(accepted_row[j]) < N) for j in range(k)):
        return ST_BAD_ACCEPTED
    return ST_OK


def kv_commit(k_cache, v_cache, block_table, prefix_len, accepted, num_accepted, status, N):
    """Return (k_new, v_new, prefix_len_new, status_new); inputs are not modified."""
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    pl = np.array(prefix_len, dtype=np.int64).copy()
    st = [int(s) for s in status]
    nb = k_cache.shape[0]
    for b in range(len(pl)):
        k = int(num_accepted[b])
        if st[b] != ST_OK or k < 0:
            continue
        L = int(pl[b])
        s = commit_status(block_table[b], L, N, nb, accepted[b], k)
        if s != ST_OK:
            st[b] = s
            continue
        for j in range(k):
            src = L + int(accepted[b][j])
            dst = L + j
            sb, so = int(block_table[b][src // BLOCK]), src % BLOCK
            db, do = int(block_table[b][dst // BLOCK]), dst % BLOCK
            k_new[db, :, do, :] = k_cache[sb, :, so, :]
            v_new[db, :, do, :] = v_cache[sb, :, so, :]
        pl[b] = L + k
    return k_new, v_new, pl, np.array(st)
