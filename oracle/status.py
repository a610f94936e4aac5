"""Per-request status codes of the verification step (oracle's own copy)."""
ST_OK = 0
ST_BAD_PARENT = 1      # parent[i] not in {-1} U [0, i), or more than 64 nodes
ST_BAD_TOKEN = 2       # a speculated token outside [0, V)
ST_BAD_QROW = 3        # a draft-row index outside [0, R)
ST_NONFINITE = 4       # non-finite target logit, or unusable draft probability
ST_KV_CAPACITY = 6     # prefix_len < 0 or prefix_len + N beyond the block table
ST_BAD_BLOCK = 7       # a block-table entry outside [0, num_blocks)
ST_BAD_ACCEPTED = 8    # accepted list not a valid node list of length <= N
