// kv_commit_accepted: keep only the accepted path's KV entries.
//
// SpecInfer summary, "KV-cache for verified tokens": after verification only
// the accepted tokens keep their cache entries.  Wiki concept page
// "Speculative decoding", "KV-cache rollback": the accepted path is compacted
// into contiguous slots.  For request b with prefix L and accepted nodes
// a_0..a_{k-1}, slot L + a_j moves to slot L + j (all heads, K and V), then
// the prefix grows by k.
//
// A destination slot can also be the source of an earlier path position
// (path (1,2,4): slot L+1 is read for j = 0 and written for j = 1), so each
// workgroup loads every moved entry of its head into registers, waits at a
// barrier, and only then stores.  Different heads never overlap, so heads are
// spread over workgroups; the prefix length is bumped by a second kernel so
// that no workgroup can see a half-updated length.
#include "tv_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunksPerThread = 16;   // 64 tokens * 32 chunks * 2 (K,V) / 256

// Checks shared by both kernels; returns the request's new status (0 = go).
__device__ __forceinline__ int commit_checks(int b, int N, int num_blocks, const int32_t* block_table,
                                             int max_blocks, int L, int k, const int32_t* accepted) {
  if (L < 0 || static_cast<int64_t>(L) + N > static_cast<int64_t>(max_blocks) * TV_BLOCK)
    return TV_REQ_KV_CAPACITY;
  if (N > 0) {
    for (int j = L / TV_BLOCK; j <= (L + N - 1) / TV_BLOCK; ++j) {
      const int blk = block_table[static_cast<size_t>(b) * max_blocks + j];
      if (blk < 0 || blk >= num_blocks) return TV_REQ_BAD_BLOCK;
    }
  }
  if (k > N) return TV_REQ_BAD_ACCEPTED;
  for (int j = 0; j < k; ++j) {
    const int a = accepted[static_cast<size_t>(b) * N + j];
    if (a < 0 || a >= N) return TV_REQ_BAD_ACCEPTED;
  }
  return TV_REQ_OK;
}

// grid (B, ceil(H / heads_per_wg))
template <int kElemBytes>
__global__ __launch_bounds__(kThreads) void kv_compact_kernel(
    int N, int H, int D, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, int num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ num_accepted,
    int32_t* __restrict__ status, int heads_per_wg) {
  const int b = blockIdx.x;
  __shared__ int s_go;
  if (threadIdx.x == 0) {
    int go = 0;
    const int k = num_accepted[b];
    if (status[b] == TV_REQ_OK && k >= 0) {
      const int st = commit_checks(b, N, num_blocks, block_table, max_blocks, prefix_len[b], k, accepted);
      if (st != TV_REQ_OK) status[b] = st;  // same value from every workgroup of b
      go = st == TV_REQ_OK && k > 0;
    }
    s_go = go;
  }
  __syncthreads();
  if (!s_go) return;

  const int L = prefix_len[b];
  const int k = num_accepted[b];
  const int row_bytes = D * kElemBytes;
  const int cpt = row_bytes / 16;           // 16-byte chunks per token row
  const int total = 2 * k * cpt;            // K and V
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;
  const int32_t* acc = accepted + static_cast<size_t>(b) * N;
  const size_t head_stride = static_cast<size_t>(TV_BLOCK) * row_bytes;
  const size_t block_stride = static_cast<size_t>(H) * head_stride;

  const int h_begin = blockIdx.y * heads_per_wg;
  const int h_end = min(H, h_begin + heads_per_wg);
  for (int h = h_begin; h < h_end; ++h) {
    uint4 buf[kMaxChunksPerThread];
#pragma unroll
    for (int r = 0; r < kMaxChunksPerThread; ++r) {
      const int c = threadIdx.x + r * kThreads;
      if (c < total) {
        const int which = c / (k * cpt);          // 0 = K, 1 = V
        const int rem = c - which * k * cpt;
        const int j = rem / cpt, ch = rem - j * cpt;
        const int src = L + acc[j];
        const uint8_t* base = which ? vc : kc;
        const uint8_t* p = base + bt[src / TV_BLOCK] * block_stride + h * head_stride +
                           (src % TV_BLOCK) * static_cast<size_t>(row_bytes) + ch * 16;
        buf[r] = *reinterpret_cast<const uint4*>(p);
      }
    }
    __syncthreads();  // every read of this head precedes every write of it
#pragma unroll
    for (int r = 0; r < kMaxChunksPerThread; ++r) {
      const int c = threadIdx.x + r * kThreads;
      if (c < total) {
        const int which = c / (k * cpt);
        const int rem = c - which * k * cpt;
        const int j = rem / cpt, ch = rem - j * cpt;
        const int dst = L + j;
        uint8_t* base = which ? vc : kc;
        uint8_t* p = base + bt[dst / TV_BLOCK] * block_stride + h * head_stride +
                     (dst % TV_BLOCK) * static_cast<size_t>(row_bytes) + ch * 16;
        *reinterpret_cast<uint4*>(p) = buf[r];
      }
    }
    // The next head touches other memory: no barrier needed before its loads.
  }
}

__global__ void bump_prefix_kernel(int B, int32_t* __restrict__ prefix_len,
                                   const int32_t* __restrict__ num_accepted,
                                   const int32_t* __restrict__ status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B && status[b] == TV_REQ_OK && num_accepted[b] >= 0) prefix_len[b] += num_accepted[b];
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
  const int heads_per_wg = 4;
  dim3 grid(B, (H + heads_per_wg - 1) / heads_per_wg);
  if (dt == TV_BF16)
    hipLaunchKernelGGL(kv_compact_kernel<2>, grid, dim3(kThreads), 0, stream, N, H, D,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_blocks,
                       block_table, max_blocks, prefix_len, accepted, num_accepted, status,
                       heads_per_wg);
  else
    hipLaunchKernelGGL(kv_compact_kernel<4>, grid, dim3(kThreads), 0, stream, N, H, D,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_blocks,
                       block_table, max_blocks, prefix_len, accepted, num_accepted, status,
                       heads_per_wg);
  if (hipGetLastError() != hipSuccess) return TV_EHIP;
  hipLaunchKernelGGL(bump_prefix_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, prefix_len,
                     num_accepted, status);
  return tv::launch_status();
}
