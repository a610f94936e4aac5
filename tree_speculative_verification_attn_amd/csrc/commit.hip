// kv_commit_accepted: keep only the accepted path's KV entries.
//
// SpecInfer summary, "KV-cache for verified tokens": after verification only
// the accepted tokens keep their cache entries.  Wiki concept page
// "Speculative decoding", "KV-cache rollback": the accepted path is compacted
// into contiguous slots.  For request b with prefix L and accepted nodes
// a_0..a_{k-1}, slot L + a_j moves to slot L + j (all heads, K and V), then
// the prefix grows by k.
//
// One workgroup per request.  The first round trip fetches the request's
// header and its accepted ids together; the ids are checked in parallel
// threads, and the move itself (block ids, then the rows in batches of whole
// heads, so any ids are safe) is the shared compaction of kv_move.h.  The
// workgroup is the only reader of its request's prefix length, so it bumps
// the length itself at the end.
#include "kv_move.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kChunks = 8;                 // 16-byte chunks per thread per batch

__global__ __launch_bounds__(kThreads) void kv_commit_kernel(int N, tv::KvRef kv,
                                                              const int32_t* __restrict__ accepted,
                                                              const int32_t* __restrict__ num_accepted,
                                                              int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ int s_st, s_k, s_L, s_bad_ids;
  __shared__ int s_path[TV_MAX_NODES];
  __shared__ tv::CommitLds s_mv;

  // first round trip: the request's header and its accepted ids together
  // (an id is only used once k is known to cover it)
  const int a_t = t < N ? accepted[static_cast<size_t>(b) * N + t] : 0;
  if (t == 0) {
    s_st = status[b];
    s_k = num_accepted[b];
    s_L = kv.prefix_len[b];
    s_bad_ids = 0;
  }
  __syncthreads();
  const int st = s_st, k = s_k, L = s_L;
  if (st == TV_REQ_OK && k >= 0) {
    if (k > N) {
      if (t == 0) s_bad_ids = 1;
    } else if (t < k) {
      if (a_t < 0 || a_t >= N) atomicOr(&s_bad_ids, 1);
      s_path[t] = a_t;
    }
  }
  __syncthreads();
  const int res = tv::commit_request<kThreads, kChunks, false>(kv, b, N, st, L, k, s_path, s_bad_ids != 0, s_mv);
  if (t == 0 && res != st) status[b] = res;
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
  tv::KvRef kv;
  kv.H = H;
  kv.D = D;
  kv.elem = dt == TV_BF16 ? 2 : 4;
  kv.kc = static_cast<uint8_t*>(k_cache);
  kv.vc = static_cast<uint8_t*>(v_cache);
  kv.num_blocks = num_blocks;
  kv.block_table = block_table;
  kv.max_blocks = max_blocks;
  kv.prefix_len = prefix_len;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(B), dim3(kThreads), 0, stream, N, kv, accepted, num_accepted, status);
  return tv::launch_status();
}
