// Compaction of a request's accepted path in the paged KV cache, shared by
// kv_commit_accepted and tree_verify_mss_commit.
//
// SpecInfer summary, "KV-cache for verified tokens": after verification only
// the accepted tokens keep their cache entries.  Wiki concept page
// "Speculative decoding", "KV-cache rollback": the accepted path is compacted
// into contiguous slots.  For request b with prefix L and accepted nodes
// a_0..a_{k-1}, slot L + a_j moves to slot L + j (all heads, K and V), then
// the prefix grows by k.  Every read sees the cache as it was before the
// move.
//
// The move is small (k <= tree depth rows per head) and bound by latency: the
// block ids are resolved once into LDS, and the K/V rows of many heads are
// loaded at once.  A destination slot can also be the source of another path
// position (path (1,2,4): slot L+1 is read for j = 0 and written for j = 1),
// so a batch issues all its loads before any of its stores.  Items run in
// the order (head, K or V, path position, 16-byte chunk):
//   * arbitrary ids: batches hold whole heads, and different heads never
//     overlap, so no store of a batch can precede a read of the same row;
//   * ids that grow along the path (a_j > a_{j-1}, as every walk produces:
//     parents precede their children): a destination L + j can only be the
//     source of a position j' < j, which comes earlier in the order (same
//     batch: behind the barrier; earlier batch: its loads completed before
//     its barrier), so batches may be cut anywhere.
#pragma once

#include "tv_common.h"

namespace tv {

struct KvRef {
  int H, D, elem;                // heads, head dim, bytes per element (2 or 4)
  uint8_t* kc;                   // [num_blocks][H][16][D]
  uint8_t* vc;
  int num_blocks;
  const int32_t* block_table;    // [B][max_blocks]
  int max_blocks;
  int32_t* prefix_len;           // [B]
};

// LDS of commit_request (one per workgroup).
struct CommitLds {
  int64_t src[TV_MAX_NODES];     // byte offset of (block, row) of each path source, at head 0
  int64_t dst[TV_MAX_NODES];     //   and of each destination
  int bad;
};

// Largest number of 16-byte chunks one head moves: K and V of up to
// TV_MAX_NODES rows of an fp32 head of dim 128.
constexpr int kMaxHeadChunks = 2 * TV_MAX_NODES * (128 * 4 / 16);
// Blocks that can cover [L, L + N): at most ceil(TV_MAX_NODES / TV_BLOCK) + 1.
constexpr int kMaxTreeBlocks = TV_MAX_NODES / TV_BLOCK + 1;

// Block ids of the blocks covering [L, L + N), for a caller that fetches them
// early (lane i of one wave: block L / 16 + i; 0 past the range or when L is
// out of range).  commit_request then reads them from LDS.
__device__ __forceinline__ int tree_block_id(const KvRef& kv, int b, int N, int L, int i) {
  if (L < 0 || static_cast<int64_t>(L) + N > static_cast<int64_t>(kv.max_blocks) * TV_BLOCK || N <= 0) return 0;
  const int blk_lo = L / TV_BLOCK, nblk = (L + N - 1) / TV_BLOCK - blk_lo + 1;
  return i < nblk ? kv.block_table[static_cast<size_t>(b) * kv.max_blocks + blk_lo + i] : 0;
}

// The move in phases, for callers that overlap its first loads with other
// work (commit_request below strings them together).
struct MovePlan {
  int cpt, per_which, per_head, total, step;
  size_t head_stride;
};

// Checks and block offsets of request b's move (every thread of the
// workgroup calls it; workgroup barriers inside).
//   st        the request's status; anything but TV_REQ_OK is returned as is
//   L, k      prefix length and number of accepted nodes (k < 0: skipped)
//   path      LDS, the k accepted node ids (valid unless ids_bad)
//   ids_bad   the caller found k > N or an id outside [0, N)
//   pre_blk   LDS, the block ids tree_block_id fetched, or nullptr (then
//             they are read here)
// Returns TV_REQ_OK when the move is to be made (plan filled in), else the
// status to store: the input status, TV_REQ_KV_CAPACITY, TV_REQ_BAD_BLOCK or
// TV_REQ_BAD_ACCEPTED in that order of precedence (nothing is written).
template <int NT, int CH, bool MONOTONE>
__device__ int move_prepare(const KvRef& kv, int b, int N, int st, int L, int k, const int* path,
                            bool ids_bad, CommitLds& s, const int* pre_blk, MovePlan& plan) {
  static_assert(MONOTONE || NT * CH >= kMaxHeadChunks, "a batch must hold a whole head");
  if (st != TV_REQ_OK || k < 0) return st == TV_REQ_OK ? -1 : st;
  if (L < 0 || static_cast<int64_t>(L) + N > static_cast<int64_t>(kv.max_blocks) * TV_BLOCK)
    return TV_REQ_KV_CAPACITY;
  const int t = threadIdx.x;
  const int row_bytes = kv.D * kv.elem;
  const size_t head_stride = static_cast<size_t>(TV_BLOCK) * row_bytes;
  const size_t block_stride = static_cast<size_t>(kv.H) * head_stride;
  const int32_t* bt = kv.block_table + static_cast<size_t>(b) * kv.max_blocks;

  if (t == 0) s.bad = 0;
  __syncthreads();
  // every block covering [L, L + N) must be a valid id (these are all the
  // blocks the move can touch); the path's rows are resolved at the same
  // time (only used if the checks pass)
  const int blk_lo = L / TV_BLOCK, nblk = N > 0 ? (L + N - 1) / TV_BLOCK - blk_lo + 1 : 0;
  auto blk_of = [&](int i) { return pre_blk ? pre_blk[i] : bt[blk_lo + i]; };   // i < nblk
  for (int i = t; i < nblk; i += NT) {
    const int blk = blk_of(i);
    if (blk < 0 || blk >= kv.num_blocks) atomicOr(&s.bad, 1);
  }
  if (!ids_bad) {
    for (int j = t; j < k; j += NT) {
      const int src = L + path[j], dst = L + j;
      s.src[j] = static_cast<int64_t>(blk_of(src / TV_BLOCK - blk_lo)) * block_stride + (src % TV_BLOCK) * row_bytes;
      s.dst[j] = static_cast<int64_t>(blk_of(dst / TV_BLOCK - blk_lo)) * block_stride + (dst % TV_BLOCK) * row_bytes;
    }
  }
  __syncthreads();
  if (s.bad) return TV_REQ_BAD_BLOCK;
  if (ids_bad) return TV_REQ_BAD_ACCEPTED;
  plan.cpt = row_bytes / 16;                   // 16-byte chunks per row
  plan.per_which = k * plan.cpt;               // chunks of K (or V) of one head
  plan.per_head = 2 * plan.per_which;
  plan.total = kv.H * plan.per_head;
  plan.step = MONOTONE ? NT * CH : (plan.per_head > 0 ? (NT * CH / plan.per_head) * plan.per_head : NT * CH);
  plan.head_stride = head_stride;
  return TV_REQ_OK;
}

// item -> (head, K or V, path position, chunk): the chunk's address without
// the row's offset, and the path position
__device__ __forceinline__ uint8_t* move_item(const KvRef& kv, const MovePlan& p, int item, int& j) {
  const int hh = item / p.per_head, rem = item - hh * p.per_head;
  const int which = rem / p.per_which, rem2 = rem - which * p.per_which;
  j = rem2 / p.cpt;
  const int ch = rem2 - j * p.cpt;
  return (which ? kv.vc : kv.kc) + hh * p.head_stride + ch * 16;
}

// Loads of the batch starting at item i0.
template <int NT, int CH>
__device__ __forceinline__ void move_load(const KvRef& kv, const MovePlan& p, const CommitLds& s, int i0,
                                          uint4 (&buf)[CH]) {
  const int n = min(p.step, p.total - i0);
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int i = r * NT + static_cast<int>(threadIdx.x);
    // (set on every path: an element assigned only under a condition keeps
    // the whole array in scratch memory)
    buf[r] = make_uint4(0u, 0u, 0u, 0u);
    if (i < n) {
      int j;
      const uint8_t* base = move_item(kv, p, i0 + i, j);
      buf[r] = *reinterpret_cast<const uint4*>(base + s.src[j]);
    }
  }
}

// Stores of the batch starting at i0; every load of the batch, in every
// thread, must have completed (a workgroup barrier after move_load).
template <int NT, int CH>
__device__ __forceinline__ void move_store(const KvRef& kv, const MovePlan& p, const CommitLds& s, int i0,
                                           const uint4 (&buf)[CH]) {
  const int n = min(p.step, p.total - i0);
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int i = r * NT + static_cast<int>(threadIdx.x);
    if (i < n) {
      int j;
      uint8_t* base = move_item(kv, p, i0 + i, j);
      *reinterpret_cast<uint4*>(base + s.dst[j]) = buf[r];
    }
  }
}

// Batches from item i0 on, loads then barrier then stores each (the next
// batch's reads cannot meet this batch's writes, see above).
template <int NT, int CH>
__device__ void move_rest(const KvRef& kv, const MovePlan& p, const CommitLds& s, int i0) {
  for (; i0 < p.total; i0 += p.step) {
    uint4 buf[CH];
    move_load<NT, CH>(kv, p, s, i0, buf);
    __syncthreads();      // every read of this batch precedes every write of it
    move_store<NT, CH>(kv, p, s, i0, buf);
  }
}

// Commits request b's accepted path in one go.  Arguments as move_prepare.
// Returns the request's new status: TV_REQ_OK after the move (prefix_len[b]
// = L + k), else as move_prepare (with nothing written).
template <int NT, int CH, bool MONOTONE>
__device__ int commit_request(const KvRef& kv, int b, int N, int st, int L, int k, const int* path,
                              bool ids_bad, CommitLds& s, const int* pre_blk = nullptr) {
  MovePlan plan;
  const int r = move_prepare<NT, CH, MONOTONE>(kv, b, N, st, L, k, path, ids_bad, s, pre_blk, plan);
  if (r != TV_REQ_OK) return r < 0 ? st : r;
  move_rest<NT, CH>(kv, plan, s, 0);
  if (threadIdx.x == 0) kv.prefix_len[b] = L + k;
  return TV_REQ_OK;
}

}  // namespace tv
