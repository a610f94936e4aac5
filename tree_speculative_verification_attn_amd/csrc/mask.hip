// tree_build_mask: ancestor / child bitmasks and depths of every tree.
//
// TreeMask (SpecInfer summary, "Tree-based Parallel Decoding: Topology-Aware
// Causal Mask"): node u may attend node v iff v is u or one of u's ancestors.
// One wave64 per request; lane i owns node i.  parent[i] = -2 marks a padding
// slot: no ancestors, nobody's child, never a parent.  Each lane climbs its parent
// chain through cross-lane reads (depth <= 64 steps), so no mask is ever
// materialised on the host.
#include "tv_common.h"

namespace {

__global__ __launch_bounds__(64) void build_mask_kernel(int N, const int32_t* __restrict__ parent,
                                                        uint64_t* __restrict__ anc,
                                                        uint64_t* __restrict__ child,
                                                        int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool live = i < N;
  // parent -2 marks a padding slot (trees of different sizes in one batch);
  // lanes past N behave like padding
  const int p = live ? parent[static_cast<size_t>(b) * N + i] : -2;
  const int pp = __shfl(p, p >= 0 ? p : 0, 64);      // parent of my parent
  const int bad = __any(live && (p < -2 || p >= i || (p >= 0 && pp == -2)));
  const bool node = live && p != -2;

  uint64_t a = 0;
  int d = 0;
  if (!bad && node) {
    a = 1ull << i;
    d = 1;
  }
  // climb: cur = current ancestor of node i (-1 = reached the root)
  int cur = (bad || !node) ? -1 : p;
  for (int step = 0; step < N; ++step) {
    const int any_left = __any(cur >= 0);
    if (!any_left) break;
    const int src = cur >= 0 ? cur : 0;
    const int up = __shfl(p, src, 64);   // parent of my current ancestor
    if (cur >= 0) {
      a |= 1ull << cur;
      ++d;
      cur = up;
    }
  }
  if (live) {
    anc[static_cast<size_t>(b) * N + i] = a;
    depth[static_cast<size_t>(b) * N + i] = d;
  }
  // child[u + 1] = set of nodes whose parent is u, u = -1 .. N-1: each node
  // ORs its bit into its parent's word (LDS), then lane u + 1 stores word u + 1
  __shared__ unsigned long long s_child[TV_MAX_NODES + 1];
  s_child[i] = 0ull;
  if (i == 0) s_child[TV_MAX_NODES] = 0ull;
  __syncthreads();
  if (!bad && node) atomicOr(&s_child[p + 1], 1ull << i);
  __syncthreads();
  uint64_t* crow = child + static_cast<size_t>(b) * (N + 1);
  if (i <= N) crow[i] = s_child[i];
  if (i == 0 && N == TV_MAX_NODES) crow[N] = s_child[N];
  if (i == 0) status[b] = bad ? TV_REQ_BAD_PARENT : TV_REQ_OK;
}

}  // namespace

extern "C" tv_status tree_build_mask(int B, int N, const int32_t* parent, uint64_t* anc,
                                     uint64_t* child, int32_t* depth, int32_t* status,
                                     hipStream_t stream) {
  if (B < 0 || N < 0) return TV_EINVAL;
  if (N > TV_MAX_NODES) return TV_ETOOBIG;
  if (B == 0) return TV_OK;
  if (!child || !status || (N > 0 && (!parent || !anc || !depth))) return TV_EINVAL;
  hipLaunchKernelGGL(build_mask_kernel, dim3(B), dim3(64), 0, stream, N, parent, anc, child, depth,
                     status);
  return tv::launch_status();
}

extern "C" const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_EINVAL: return "invalid argument";
    case TV_ETOOBIG: return "tree larger than 64 nodes";
    case TV_EDTYPE: return "unsupported dtype";
    case TV_EWORKSPACE: return "workspace too small";
    case TV_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}
