/*
 * treeverify.h - tree-based speculative verification on AMD MI355X (gfx950).
 *
 * One verification step of tree-based speculative inference, as the SpecInfer
 * paper describes it ("SpecInfer: Accelerating Large Language Model Serving
 * with Tree-based Speculative Inference and Verification", arXiv 2305.09781):
 * the target model scores every node of a token tree in one pass with tree
 * attention over a shared KV cache, the tree is verified greedily or by
 * multi-step speculative sampling (MSS), and the KV entries of the accepted
 * path are kept in contiguous cache slots.
 *
 * Conventions shared by every entry point
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, frees nothing and keeps no state between calls (it
 *    caches, per device, only what the device reports about itself: its
 *    compute unit count and the occupancy of its kernels).  The one
 *    exception is tree_verify_mss_noalloc, whose workspace is a fixed
 *    device array of the library.
 *  - Every call is asynchronous on `stream` (0 = the null stream).
 *  - The return value reports host-checkable problems only: bad sizes or
 *    dtypes, null pointers, a workspace that is too small, a failed launch.
 *    On a non-OK return nothing has been launched.
 *  - Data-dependent problems are reported per request in `status[b]`
 *    (TV_REQ_* codes).  tree_build_mask writes it; later calls read it, skip a
 *    request whose status is nonzero, and may set it (only from 0) when they
 *    find a problem of their own.  Outputs of a skipped request are filled as
 *    stated per call.
 *  - A tree has N <= 64 nodes in an order where every parent precedes its
 *    children (DFS preorder in practice).  The tree root is NOT a node: it is
 *    the end of the verified prefix, whose K/V is already cached; parent[i] =
 *    -1 marks a child of the root.  parent[i] = -2 marks an unused padding
 *    slot, so that trees of different sizes share one [B][N] batch: it is
 *    nobody's child, has no ancestors and no children, and its outputs are
 *    never read.
 *  - Row r of a per-request logits array is the target model's output for a
 *    context: r = 0 is the root (the verified prefix), r = 1 + i is node i.
 *  - The paged KV cache stores head h of logical slot t of request b at
 *    k_cache[block_table[b][t / block_size]][h][t % block_size][0..D-1].
 *    Slots 0..L_b-1 hold the verified prefix (L_b = prefix_len[b]); the
 *    caller writes the K/V of tree node i at slot L_b + i before attention.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_EINVAL = 1,      /* a size, a null pointer or an unsupported shape */
  TV_ETOOBIG = 2,     /* N > 64 */
  TV_EDTYPE = 3,      /* unknown tv_dtype */
  TV_EWORKSPACE = 4,  /* workspace smaller than the *_workspace() size */
  TV_EHIP = 5,        /* a HIP launch failed */
  TV_ESCRATCH = 6     /* the call needs more than the library's fixed scratch
                         (tree_verify_mss_noalloc) */
} tv_status;

/* Bytes of the fixed device array tree_verify_mss_noalloc uses as workspace. */
#define TV_NOALLOC_SCRATCH_BYTES (4u << 20)

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Per-request status codes written to status[b]. */
enum {
  TV_REQ_OK = 0,
  TV_REQ_BAD_PARENT = 1,    /* parent[i] not in {-2, -1} U [0, i), or the parent
                               is a padding slot */
  TV_REQ_BAD_TOKEN = 2,     /* token[i] not in [0, V) */
  TV_REQ_BAD_QROW = 3,      /* q_row[i] not in [0, R) */
  TV_REQ_NONFINITE = 4,     /* a visited logits row holds NaN or +inf or no finite
                               value, or a draft probability the walk reads is
                               NaN, infinite or negative */
  TV_REQ_KV_CAPACITY = 6,   /* prefix_len < 0 or prefix_len + N > max_blocks * block_size */
  TV_REQ_BAD_BLOCK = 7,     /* a block_table entry the call needs is outside [0, num_blocks) */
  TV_REQ_BAD_ACCEPTED = 8,  /* num_accepted > N or an accepted id outside [0, N) */
  TV_REQ_TIMEOUT = 9        /* a wait inside a call ran out: the workgroups of
                               a sliced verify walk did not meet within the
                               wait bound (they were not all resident), or an
                               attention group barrier did; the request's
                               outputs are as for a skipped request */
};

/*
 * tree_build_mask - topology-aware causal mask of every tree.
 * Defines: SpecInfer summary, section "Tree-based Parallel Decoding:
 * Topology-Aware Causal Mask" (TreeMask equation): node u attends node v iff
 * v is an ancestor of u or v = u; the verified prefix is visible to all.
 *
 *   parent [B][N] int32     parent node of each node, -1 = child of the root,
 *                           -2 = padding slot
 *   anc    [B][N] uint64    out: bit j set iff node j is node i or an ancestor
 *                           (0 for a padding slot)
 *   child  [B][N+1] uint64  out: child[b][0] = children of the root,
 *                           child[b][u+1] = children of node u (bit j = node j)
 *   depth  [B][N] int32     out: nodes on the root-to-i path (1 for root children,
 *                           0 for a padding slot)
 *   status [B] int32        out: TV_REQ_OK, or TV_REQ_BAD_PARENT (then anc,
 *                           child and depth of that request are all zero)
 * Errors: TV_EINVAL if B < 0, N < 0 or a needed pointer is null; TV_ETOOBIG if
 * N > 64.  B = 0 launches nothing.
 */
tv_status tree_build_mask(int B, int N, const int32_t* parent, uint64_t* anc,
                          uint64_t* child, int32_t* depth, int32_t* status,
                          hipStream_t stream);

/*
 * tree_attn_verify - tree attention for every node, head and request.
 * Defines: SpecInfer summary, Definition 4.1 (TreeAttention(u) =
 * Attention(S_u)), Equations 1-4 (scores Q K^T / sqrt(d), mask, softmax,
 * times V) and the TreeMask equation; "KV-cache for verified tokens" (tree K/V
 * live in the same cache, after the verified prefix).
 *
 * For request b, node i, head h: softmax over keys t in
 *   {0..L_b-1} U {L_b + j : bit j of anc[b][i]}
 * of scale * (q . k_t), times v_t, with fp32 accumulation.
 *
 *   dt            TV_F32 or TV_BF16: element type of q, k_cache, v_cache, out
 *   D             head dim, 64 or 128;  scale: usually 1/sqrt(D)
 *   q             [B][N][H][D]
 *   k_cache, v_cache [num_blocks][H][block_size][D]; block_size must be 16
 *   block_table   [B][max_blocks] int32
 *   prefix_len    [B] int32
 *   anc           [B][N] uint64 from tree_build_mask
 *   status        [B] int32 in/out: requests with status != 0 get zero output;
 *                 the call may set TV_REQ_KV_CAPACITY or TV_REQ_BAD_BLOCK
 *                 (then that request's output is unspecified)
 *   out           [B][N][H][D]; every key is summed in an order fixed by
 *                 the shapes and the device (never by timing), so repeated
 *                 calls on the same inputs and device give the same bits
 *   workspace     ws_bytes >= tree_attn_verify_workspace(...) bytes of device
 *                 memory for per-chunk partial results (may be null when that
 *                 size is 0); contents on entry do not matter.  Calls that
 *                 overlap in time must not share a workspace.
 * Errors: TV_EINVAL for N < 0, B < 0, H < 1, D not 64/128, block_size != 16,
 * max_blocks < 1, num_blocks < 1 or null pointers; TV_ETOOBIG for N > 64;
 * TV_EDTYPE; TV_EWORKSPACE.
 */
size_t tree_attn_verify_workspace(tv_dtype dt, int B, int N, int H, int D, int max_blocks);
tv_status tree_attn_verify(tv_dtype dt, int B, int N, int H, int D, float scale,
                           const void* q, const void* k_cache, const void* v_cache,
                           int num_blocks, int block_size, const int32_t* block_table,
                           int max_blocks, const int32_t* prefix_len, const uint64_t* anc,
                           int32_t* status, void* out, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/*
 * tree_mask_attn_verify - tree_build_mask followed by tree_attn_verify, in one
 * launch where it can.
 * Defines: the TreeMask equation and Definition 4.1 with Equations 1-4 of the
 * SpecInfer summary, as for the two calls it stands for.
 *
 * Results (anc, child, depth, status, out) are those of
 *   tree_build_mask(B, N, parent, anc, child, depth, status);
 *   tree_attn_verify(..., prefix_len, anc, status, out, workspace, ...);
 * so status is written, not read: TV_REQ_BAD_PARENT, TV_REQ_KV_CAPACITY,
 * TV_REQ_BAD_BLOCK or TV_REQ_OK (a request that fails a check gets the later
 * call's treatment: zero output for a malformed tree or a prefix past the
 * table, unspecified output for a bad block id).  With bf16 and a chunk plan of
 * one chunk per (request, head) (tree_attn_verify_workspace gives 0) it is one
 * kernel: every workgroup derives its request's masks from parent; otherwise
 * the two kernels run one after the other.  N = 0 only builds the (empty) masks.
 *
 *   parent        [B][N] int32 in; anc [B][N], child [B][N+1] uint64, depth
 *                 [B][N] int32 out, as tree_build_mask
 *   others        as tree_attn_verify (anc is not read)
 * Errors: those of the two calls; every argument is checked before anything
 * is launched, so an error return leaves every buffer unchanged.
 */
tv_status tree_mask_attn_verify(tv_dtype dt, int B, int N, int H, int D, float scale,
                                const void* q, const void* k_cache, const void* v_cache,
                                int num_blocks, int block_size, const int32_t* block_table,
                                int max_blocks, const int32_t* prefix_len, const int32_t* parent,
                                uint64_t* anc, uint64_t* child, int32_t* depth, int32_t* status,
                                void* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * tree_verify_greedy - VerifyGreedy.
 * Defines: SpecInfer summary, section "Token Verification: Greedy Decoding
 * (VerifyGreedy)": from the root, while a child v of the current node u has
 * token O(u), accept v and continue; at the first miss emit O(u).
 * O(u) = lowest index of the maximal fp32 logit of u's row; among children
 * with the same token the lowest node index wins.
 *
 *   target_logits [B][N+1][V] fp32
 *   token         [B][N] int32;   child [B][N+1] uint64 from tree_build_mask
 *   status        [B] in/out (may set TV_REQ_BAD_TOKEN, TV_REQ_NONFINITE,
 *                 TV_REQ_TIMEOUT)
 *   accepted      [B][N] out: accepted node ids in path order, then -1
 *   num_accepted  [B] out: path length (-1 for a request with status != 0)
 *   bonus         [B] out: the emitted target token (-1 if status != 0)
 *   workspace     >= tree_verify_workspace(B, N, V) bytes of device memory
 *                 that is ALL ZERO before its first use; every call that
 *                 completes leaves it all zero again, so one zero fill at
 *                 allocation serves any number of later calls.  It holds the
 *                 counters and values the workgroups of one request exchange.
 *                 Calls that overlap in time must not share a workspace.
 * Work split: up to V = 16384 one workgroup walks a request.  Above, each
 * request is walked by ceil(V / (256 E)) workgroups that exchange values
 * through the workspace and so must be resident at the same time; E = 4, 8 or
 * 16 vocabulary entries per thread (greedy: 8), chosen per call from B, V and
 * the device's compute unit count (one workgroup per compute unit when it
 * fits).  They are started
 * by ordinary launches in batches of requests sized so that every workgroup
 * of a batch fits on the device at once (by the occupancy the device reports
 * for the kernel); that residency is not guaranteed when other work occupies
 * the device's compute units.  Every wait is bounded (2^22 polls, about 0.1 s,
 * or TREEVERIFY_WALK_WAIT_POLLS from the environment): a wait that runs out
 * sets TV_REQ_TIMEOUT for its request instead of hanging, every workgroup
 * still leaves, and the workspace is still left zero.  Workgroup 0 of a
 * request writes all of the request's outputs, so they always come from one
 * decision: a request is either complete or timed out (no bonus from one
 * workgroup beside a status from another).
 * Errors: TV_EINVAL (B, N < 0, V < 1 or V > 2^20, null pointers),
 * TV_ETOOBIG, TV_EWORKSPACE, TV_EHIP (a launch failed, or the device's
 * occupancy query did).
 */
size_t tree_verify_workspace(int B, int N, int V);
tv_status tree_verify_greedy(int B, int N, int V, const float* target_logits,
                             const int32_t* token, const uint64_t* child, int32_t* status,
                             int32_t* accepted, int32_t* num_accepted, int32_t* bonus,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * tree_verify_mss - VerifyStochastic, multi-step speculative sampling.
 * Defines: SpecInfer summary, section "Token Verification: Stochastic
 * Decoding and Multi-Step Speculative Sampling (VerifyStochastic)"; the leaf
 * bonus token and the zero-normaliser guard follow the wiki concept page
 * "Speculative decoding", "Implementation sketch".
 *
 * At node u with untested children U (initially all children), round j:
 *   words (x0,x1,x2,x3) = Philox4x32-10(key = seed, counter =
 *       (64*slot(u) + j, b, offset mod 2^32, offset >> 32)),
 *       slot(root) = 0, slot(node i) = i + 1;
 *   s = the ((x0>>8) * |U| >> 24)-th member of U in ascending node order;
 *   accept s iff ((x1>>8)+1) * 2^-24 <= p(token[s]) / q_s(token[s]) where p is
 *   u's current target distribution (softmax of its row at first) and q_s =
 *   ssm_probs[b][q_row[b][s]] (q = 0: ratio +inf if p > 0, else 0);
 *   on acceptance move to s; on rejection p <- norm(max(0, p - q_s)) (left
 *   unchanged if the normaliser is 0) and drop s from U.
 * When U is empty (all rejected, or a leaf reached by acceptance) the bonus is
 * the smallest x with sum_{y<=x} p(y) >= ((x2>>8)+1) * 2^-24 * sum(p), x2 from
 * round 0 at that node.
 *
 *   target_logits [B][N+1][V] fp32;  ssm_probs [B][R][V] fp32 (used as given)
 *   q_row         [B][N] int32 row of ssm_probs that proposed node i
 *   token, child  as for greedy
 *   status        [B] in/out (may set TV_REQ_BAD_TOKEN, TV_REQ_BAD_QROW,
 *                 TV_REQ_NONFINITE, TV_REQ_TIMEOUT)
 *   accepted, num_accepted, bonus  as for greedy
 *   rounds        [B] out, or null: number of ratio tests (-1 if skipped)
 *   workspace     as for greedy (all zero before first use, left all zero)
 * Errors: as for greedy, plus TV_EINVAL for R < 1.
 */
tv_status tree_verify_mss(int B, int N, int V, int R, const float* target_logits,
                          const float* ssm_probs, const int32_t* q_row, const int32_t* token,
                          const uint64_t* child, int32_t* status, uint64_t seed,
                          uint64_t offset, int32_t* accepted, int32_t* num_accepted,
                          int32_t* bonus, int32_t* rounds, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/*
 * tree_verify_mss_noalloc - tree_verify_mss for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * and harnesses that forbid hipMalloc.  It takes no workspace argument and
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *
 * Arguments, outputs, status codes and results are those of tree_verify_mss;
 * the workspace is a fixed array of TV_NOALLOC_SCRATCH_BYTES bytes of device
 * memory inside the library, one per device, held until the process ends.
 * The first call on a device (with that device current) looks up the
 * array's address and queues a zero fill of it on `stream` ahead of the walk;
 * every completed call leaves it zero again.  Every call on a device shares
 * that device's array: calls that overlap in time on one device (on
 * different streams, or from different threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe.  A first call
 * made while `stream` is being captured also records the fill in the graph,
 * and the next call outside a capture fills again.
 * Errors: those of tree_verify_mss (without TV_EWORKSPACE), TV_ESCRATCH when
 * tree_verify_workspace(B, N, V) exceeds TV_NOALLOC_SCRATCH_BYTES (1260
 * requests at V = 32000, 123 at V = 2^20), TV_EHIP when the array's address
 * cannot be found.
 */
tv_status tree_verify_mss_noalloc(int B, int N, int V, int R, const float* target_logits,
                                  const float* ssm_probs, const int32_t* q_row, const int32_t* token,
                                  const uint64_t* child, int32_t* status, uint64_t seed,
                                  uint64_t offset, int32_t* accepted, int32_t* num_accepted,
                                  int32_t* bonus, int32_t* rounds, hipStream_t stream);

/*
 * kv_commit_accepted - keep only the accepted path's KV entries.
 * Defines: SpecInfer summary, "KV-cache for verified tokens" (only accepted
 * tokens keep their cache entries); wiki concept page "Speculative decoding",
 * "KV-cache rollback" (the accepted path is compacted into contiguous slots).
 *
 * For each request with status 0 and num_accepted k >= 0: for j < k, K and V
 * of slot L + accepted[j] move to slot L + j (all heads; every read sees the
 * cache as it was before the call), then prefix_len[b] = L + k.
 *
 *   k_cache, v_cache in/out, layout as for tree_attn_verify; N = tree size
 *   prefix_len   [B] in/out
 *   accepted     [B][N], num_accepted [B] from a verify call
 *   status       [B] in/out (may set TV_REQ_KV_CAPACITY, TV_REQ_BAD_BLOCK,
 *                TV_REQ_BAD_ACCEPTED; such a request is left unchanged)
 * Errors: TV_EINVAL, TV_ETOOBIG, TV_EDTYPE as for tree_attn_verify.
 */
tv_status kv_commit_accepted(tv_dtype dt, int B, int N, int H, int D, void* k_cache,
                             void* v_cache, int num_blocks, int block_size,
                             const int32_t* block_table, int max_blocks, int32_t* prefix_len,
                             const int32_t* accepted, const int32_t* num_accepted,
                             int32_t* status, hipStream_t stream);

/*
 * tree_verify_mss_multi - VerifyStochastic on a merged token tree, every
 * proposal its own round.
 * Defines: SpecInfer summary, "Token Verification: Stochastic Decoding and
 * Multi-Step Speculative Sampling (VerifyStochastic)" (a child is tested
 * with the distribution of the SSM that proposed it) and "Token Tree Merge"
 * (proposals of the same token share one node).  A node proposed by m SSMs
 * takes part in m rounds, each with its proposer's draft row; accepting any
 * of them enters the node, rejecting one drops only that proposal.  With
 * independent draws, one per SSM, the emitted token then follows P_LLM
 * (Theorem 4.2), which testing a merged node once does not give.
 *
 *   prop_node [B][S] int32  node of proposal slot s, -1 = unused slot
 *   prop_row  [B][S] int32  its proposer's row of ssm_probs
 *   S <= 64 slots per request.  At node u the untested proposals of u's
 *   children are taken in ascending slot order; the random proposal, the
 *   Philox counter, the ratio test, the residual and the final sample are
 *   tree_verify_mss's with "child" read as "proposal" (j counts rounds at u).
 *   With slot s = node s and prop_row = q_row the results equal
 *   tree_verify_mss's.
 * Other arguments, outputs and workspace as tree_verify_mss (q_row is
 * replaced by the proposal lists).  status may also become TV_REQ_BAD_QROW
 * when a used slot names a row outside [0, R) or no node of the tree.
 * Errors: those of tree_verify_mss; TV_ETOOBIG for S > 64; TV_EINVAL for
 * S < 0 or missing proposal arrays.
 */
tv_status tree_verify_mss_multi(int B, int N, int S, int V, int R, const float* target_logits,
                                const float* ssm_probs, const int32_t* prop_node, const int32_t* prop_row,
                                const int32_t* token, const uint64_t* child, int32_t* status,
                                uint64_t seed, uint64_t offset, int32_t* accepted,
                                int32_t* num_accepted, int32_t* bonus, int32_t* rounds,
                                void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * tree_verify_mss_commit - tree_verify_mss, then kv_commit_accepted of the
 * path it accepted, in one launch.
 * Defines: the two operations above (SpecInfer summary, "Token Verification:
 * Stochastic Decoding and Multi-Step Speculative Sampling
 * (VerifyStochastic)" and "KV-cache for verified tokens"): verification
 * decides the accepted path, and only that path keeps its cache entries.
 *
 * The results are exactly those of
 *   tree_verify_mss(B, N, V, R, target_logits, ..., workspace, ws_bytes, stream);
 *   kv_commit_accepted(kv_dtype, B, N, H, D, k_cache, v_cache, num_blocks,
 *                      block_size, block_table, max_blocks, prefix_len,
 *                      accepted, num_accepted, status, stream);
 * on the same arguments (outputs, status codes, cache contents, prefix
 * lengths).  The workgroups that walk a request also move its rows, each a
 * block of heads (all of them when one workgroup walks the request), which
 * saves the second launch and its start-up round trips.  With several
 * workgroups per request, the one that writes the request's outputs decides
 * whether the move is made and grows the prefix length only after every
 * other workgroup has reported its heads moved; if a report does not come
 * within the wait bound, the request ends as TV_REQ_TIMEOUT with its prefix
 * length unchanged, and only then may the K/V rows of its tree's slots
 * [L, L + N) be partly compacted (rows outside them never change).
 * The first 18 arguments are tree_verify_mss's, the rest kv_commit_accepted's
 * (N, B and accepted / num_accepted / status are shared); ownership,
 * workspace rules and errors are the union of theirs.
 */
tv_status tree_verify_mss_commit(int B, int N, int V, int R, const float* target_logits,
                                 const float* ssm_probs, const int32_t* q_row, const int32_t* token,
                                 const uint64_t* child, int32_t* status, uint64_t seed,
                                 uint64_t offset, int32_t* accepted, int32_t* num_accepted,
                                 int32_t* bonus, int32_t* rounds, void* workspace, size_t ws_bytes,
                                 tv_dtype kv_dtype, int H, int D, void* k_cache, void* v_cache,
                                 int num_blocks, int block_size, const int32_t* block_table,
                                 int max_blocks, int32_t* prefix_len, hipStream_t stream);

/* Human-readable name of a tv_status value (static storage). */
/*
 * tree_verify_naive - naive sampling verification (the comparator of
 * SpecInfer's Theorem 4.3; Table 3 compares it with MSS).
 * Defines: SpecInfer summary, "Token Verification" (the naive approach and
 * Theorem 4.3): at the current node u draw x from P_LLM(.|u); if a child of u
 * carries token x, accept the lowest such child and continue from it;
 * otherwise x is the bonus token and the walk stops.  Every emitted token is
 * distributed as P_LLM given the tokens before it, but fewer tokens are
 * accepted than with MSS.  The draw is the inverse-CDF sample of
 * tree_verify_mss's final step with word 2 of round 0 at u's slot.
 *
 * Arguments, outputs, status handling and workspace as tree_verify_greedy,
 * plus seed and offset as tree_verify_mss.  Same errors as tree_verify_greedy.
 */
tv_status tree_verify_naive(int B, int N, int V, const float* target_logits, const int32_t* token,
                            const uint64_t* child, int32_t* status, uint64_t seed, uint64_t offset,
                            int32_t* accepted, int32_t* num_accepted, int32_t* bonus,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * tree_logits_transform - sampling transforms of rows of logits, applied
 * before verification.
 * Defines: wiki concept page "Speculative decoding", "Implementation sketch":
 * the lossless acceptance rule is applied after temperature, top-k and top-p
 * have been applied to both the target's and the draft's distribution.
 *
 *   rows, V        rows of V fp32 logits (V <= 2^20)
 *   in  [rows][V]  fp32 logits (-inf allowed: probability 0)
 *   out [rows][V]  fp32, may be the same array as in
 *   temperature    T > 0; the scaled logit is the fp32 product l * fp32(1/T)
 *   top_k          keep the top_k largest scaled logits (ties: lower index
 *                  first); 0, or at least the number of finite entries, keeps all
 *   top_p          in (0, 1]: then keep the smallest set of largest
 *                  probabilities (ties: lower index first) whose mass reaches
 *                  top_p times the mass top-k kept; 1 keeps all
 *   out_kind       TV_OUT_LOGITS: the scaled logit where kept, -inf elsewhere
 *                  (a softmax of the row is the transformed distribution, so
 *                  it can go straight to tree_verify_greedy / tree_verify_mss);
 *                  TV_OUT_PROBS: the kept probabilities normalised to sum 1, 0
 *                  elsewhere (for draft rows, ssm_probs)
 * A row whose scaled logits hold a NaN or +inf, or no finite value, becomes
 * all NaN (verification then reports TV_REQ_NONFINITE if it reads the row).
 * The kept set is exact: the top-p cut compares sums of per-entry masses held
 * in 2^-32 fixed point, so a cut within about 1e-9 of the target may fall on
 * the other entry than an exact computation.  Work: one workgroup per row.
 * Errors: TV_EINVAL for rows < 0, V outside [1, 2^20], T not finite and > 0,
 * top_k < 0, top_p outside (0, 1], an unknown out_kind or a null pointer;
 * TV_EHIP if the launch fails.  rows = 0 launches nothing.
 */
enum { TV_OUT_LOGITS = 0, TV_OUT_PROBS = 1 };
tv_status tree_logits_transform(int rows, int V, const float* in, float* out, float temperature,
                                int top_k, float top_p, int out_kind, hipStream_t stream);

const char* tv_status_string(tv_status s);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
