// kv_commit_accepted: keep only the accepted path's KV entries.
//
// SpecInfer summary, "KV-cache for verified tokens": after verification only
// the accepted tokens keep their cache entries.  Wiki concept page
// "Speculative decoding", "KV-cache rollback": the accepted path is compacted
// into contiguous slots.  For request b with prefix L and accepted nodes
// a_0..a_{k-1}, slot L + a_j moves to slot L + j (all heads, K and V), then
// the prefix grows by k.
//
// One workgroup per request.  The move is small (k <= tree depth rows per
// head) and bound by latency, so the kernel keeps the number of dependent
// memory round trips low: the request's checks run in parallel threads, the
// physical rows of the path's sources and destinations are resolved once
// into LDS, and the K/V rows of many heads are loaded at once.  A
// destination slot can also be the source of an earlier path position (path
// (1,2,4): slot L+1 is read for j = 0 and written for j = 1), so every moved
// row of a head is loaded before any of it is stored; batches of loads
// cover whole heads, and different heads never overlap.  The workgroup is
// the only reader of its request's prefix length, so it bumps the length
// itself at the end.
#include "tv_common.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kChunks = 8;                 // 16-byte chunks per thread per batch
constexpr int kBatch = kThreads * kChunks;
// A batch holds at least one whole head: 2 (K, V) * 64 rows * 32 chunks (fp32, D = 128).
static_assert(2 * TV_MAX_NODES * (128 * 4 / 16) <= kBatch, "batch smaller than a head");

template <int kElemBytes>
__global__ __launch_bounds__(kThreads) void kv_commit_kernel(
    int N, int H, int D, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, int num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ num_accepted,
    int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ int s_st, s_k, s_L, s_bad;
  __shared__ int64_t s_src[TV_MAX_NODES], s_dst[TV_MAX_NODES];   // byte offset of (block, row) at head 0

  const int row_bytes = D * kElemBytes;
  const size_t head_stride = static_cast<size_t>(TV_BLOCK) * row_bytes;
  const size_t block_stride = static_cast<size_t>(H) * head_stride;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;

  // first round trip: the request's header and its accepted ids together
  // (a node id is only used once k is known to cover it)
  const int a_t = t < N ? accepted[static_cast<size_t>(b) * N + t] : 0;
  if (t == 0) {
    const int st = status[b];
    const int k = num_accepted[b];
    const int L = prefix_len[b];
    int go = st;
    if (st == TV_REQ_OK) {
      if (k < 0) go = -1;                                   // skipped by the verify call
      else if (L < 0 || static_cast<int64_t>(L) + N > static_cast<int64_t>(max_blocks) * TV_BLOCK)
        go = TV_REQ_KV_CAPACITY;
    }
    s_st = go;
    s_k = k;
    s_L = L;
    s_bad = 0;
  }
  __syncthreads();
  const int go = s_st;
  if (go != TV_REQ_OK) {
    if (t == 0 && go > 0 && go != status[b]) status[b] = go;
    return;
  }
  const int k = s_k, L = s_L;

  // Checks in parallel: every block covering [L, L + N) is a valid id (these
  // are all the blocks the move touches; a bad block takes precedence), the
  // path is no longer than the tree and every accepted id is a node.  The
  // path's source and destination rows are resolved at the same time (only
  // used if the checks pass).
  const int blk_lo = L / TV_BLOCK, nblk = N > 0 ? (L + N - 1) / TV_BLOCK - blk_lo + 1 : 0;
  for (int i = t; i < nblk; i += kThreads) {
    const int blk = bt[blk_lo + i];
    if (blk < 0 || blk >= num_blocks) atomicOr(&s_bad, 1);
  }
  if (k > N) {
    if (t == 0) atomicOr(&s_bad, 2);
  } else if (t < k) {
    const int a = a_t;
    if (a < 0 || a >= N) {
      atomicOr(&s_bad, 2);
    } else {
      const int src = L + a, dst = L + t;
      s_src[t] = static_cast<int64_t>(bt[src / TV_BLOCK]) * block_stride + (src % TV_BLOCK) * row_bytes;
      s_dst[t] = static_cast<int64_t>(bt[dst / TV_BLOCK]) * block_stride + (dst % TV_BLOCK) * row_bytes;
    }
  }
  __syncthreads();
  if (s_bad) {
    if (t == 0) status[b] = (s_bad & 1) ? TV_REQ_BAD_BLOCK : TV_REQ_BAD_ACCEPTED;
    return;
  }

  // ---- the move, in batches of whole heads ----
  const int cpt = row_bytes / 16;                       // 16-byte chunks per row
  const int per_head = 2 * k * cpt;                     // K and V rows of one head
  if (per_head > 0) {
    const int heads_per_batch = max(1, kBatch / per_head);
    for (int h0 = 0; h0 < H; h0 += heads_per_batch) {
      const int nh = min(heads_per_batch, H - h0);
      const int total = nh * per_head;
      uint4 buf[kChunks];
#pragma unroll
      for (int r = 0; r < kChunks; ++r) {
        const int c = t + r * kThreads;
        if (c < total) {
          const int hh = c / per_head, rem = c - hh * per_head;
          const int which = rem / (k * cpt), rem2 = rem - which * k * cpt;
          const int j = rem2 / cpt, ch = rem2 - j * cpt;
          const uint8_t* base = which ? vc : kc;
          buf[r] = *reinterpret_cast<const uint4*>(base + s_src[j] + (h0 + hh) * head_stride + ch * 16);
        }
      }
      __syncthreads();      // every read of these heads precedes every write of them
#pragma unroll
      for (int r = 0; r < kChunks; ++r) {
        const int c = t + r * kThreads;
        if (c < total) {
          const int hh = c / per_head, rem = c - hh * per_head;
          const int which = rem / (k * cpt), rem2 = rem - which * k * cpt;
          const int j = rem2 / cpt, ch = rem2 - j * cpt;
          uint8_t* base = which ? vc : kc;
          *reinterpret_cast<uint4*>(base + s_dst[j] + (h0 + hh) * head_stride + ch * 16) = buf[r];
        }
      }
      // the next batch's heads touch other memory: no barrier before its loads
    }
  }
  if (t == 0) prefix_len[b] = L + k;
}

}  // namespace

extern "C" tv_status kv_commit_accepted(tv_dtype dt, int B, int N, int H, int D, void* k_cache,
                                        void* v_cache, int num_blocks, int block_size,
                                        const int32_t* block_table, int max_blocks,
                                        int32_t* prefix_len, const int32_t* accepted,
                                        const int32_t* num_accepted, int32_t* status,
                                        hipStream_t stream) {
  if (dt != TV_F32 && dt != TV_BF16) return TV_EDTYPE;
  if (B < 0 || N < 0 || H < 1 || (D != 64 && D != 128) || block_size != TV_BLOCK ||
      max_blocks < 1 || num_blocks < 1)
    return TV_EINVAL;
  if (N > TV_MAX_NODES) return TV_ETOOBIG;
  if (B == 0) return TV_OK;
  if (!k_cache || !v_cache || !block_table || !prefix_len || !num_accepted || !status ||
      (N > 0 && !accepted))
    return TV_EINVAL;
  if (dt == TV_BF16)
    hipLaunchKernelGGL(kv_commit_kernel<2>, dim3(B), dim3(kThreads), 0, stream, N, H, D,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_blocks,
                       block_table, max_blocks, prefix_len, accepted, num_accepted, status);
  else
    hipLaunchKernelGGL(kv_commit_kernel<4>, dim3(B), dim3(kThreads), 0, stream, N, H, D,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_blocks,
                       block_table, max_blocks, prefix_len, accepted, num_accepted, status);
  return tv::launch_status();
}
