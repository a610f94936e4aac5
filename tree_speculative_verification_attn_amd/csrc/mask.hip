// tree_build_mask: ancestor / child bitmasks and depths of every tree.
//
// TreeMask (SpecInfer summary, "Tree-based Parallel Decoding: Topology-Aware
// Causal Mask"): node u may attend node v iff v is u or one of u's ancestors.
// One wave64 per request; lane i owns node i.  parent[i] = -2 marks a padding
// slot: no ancestors, nobody's child, never a parent.  Each lane climbs its parent
// chain through cross-lane reads (depth <= 64 steps), so no mask is ever
// materialised on the host.
#include "tree_mask.h"

namespace {

__global__ __launch_bounds__(64) void build_mask_kernel(int N, const int32_t* __restrict__ parent,
                                                        uint64_t* __restrict__ anc,
                                                        uint64_t* __restrict__ child,
                                                        int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  // parent -2 marks a padding slot (trees of different sizes in one batch);
  // lanes past N behave like padding
  const int p = i < N ? parent[static_cast<size_t>(b) * N + i] : -2;
  uint64_t a;
  int d;
  const bool bad = tv::wave_tree_masks(N, p, a, d);
  if (i < N) {
    anc[static_cast<size_t>(b) * N + i] = a;
    depth[static_cast<size_t>(b) * N + i] = d;
  }
  __shared__ unsigned long long s_child[TV_MAX_NODES + 1];
  tv::wave_child_masks(N, p, bad, s_child, child + static_cast<size_t>(b) * (N + 1));
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
    case TV_ESCRATCH: return "call needs more than the fixed scratch";
  }
  return "unknown status";
}
