"""Philox4x32-10 in plain Python integers (oracle side).

Definition: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC'11, section 3 (the Philox S-P network).  A 128-bit counter
(c0, c1, c2, c3) and a 64-bit key (k0, k1) go through 10 rounds.  One round:
    (hi0, lo0) = 0xD2511F53 * c0      (64-bit product split in halves)
    (hi1, lo1) = 0xCD9E8D57 * c2
    c' = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
and between rounds the key advances by the Weyl constants
(0x9E3779B9, 0xBB67AE85) modulo 2^32.

The verifier draws its random words from this generator with
    key     = (seed mod 2^32, seed >> 32)
    counter = (64 * node_slot + round, request, offset mod 2^32, offset >> 32)
where node_slot is 0 for the root and i + 1 for tree node i, and round counts
the ratio tests made at that node.  Word 0 picks a child, word 1 is the accept
uniform, word 2 (of round 0 at the node where the walk stops) is the uniform of
the final sample.
"""
MASK32 = 0xFFFFFFFF
_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85


def philox4x32_10(counter, key):
    """Return the four 32-bit output words for a 4-word counter and 2-word key."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & MASK32
            k1 = (k1 + _W1) & MASK32
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return c0, c1, c2, c3


def words(seed, offset, request, node_slot, rnd):
    """Random words used at (request, node_slot, round)."""
    key = (seed & MASK32, (seed >> 32) & MASK32)
    ctr = ((64 * node_slot + rnd) & MASK32, request & MASK32,
           offset & MASK32, (offset >> 32) & MASK32)
    return philox4x32_10(ctr, key)


def unit_open0(word):
    """Uniform in (0, 1]: the top 24 bits plus one, times 2^-24 (exact in fp32)."""
    return ((int(word) >> 8) + 1) * 2.0 ** -24


def pick_index(word, m):
    """Uniform integer in [0, m) by multiply-shift of the top 24 bits."""
    return ((int(word) >> 8) * int(m)) >> 24
