// The masks of one request's token tree, built by one wave.
//
// SpecInfer summary, section "Tree-based Parallel Decoding: Topology-Aware
// Causal Mask" (TreeMask equation): node u attends node v iff v is u or an
// ancestor of u.  Lane i of the wave handles node i (N <= 64); the ancestor
// set of node i is bit i plus the bits met while climbing parent links, which
// every lane does at once with cross-lane reads (the climb takes as many
// steps as the deepest path).  Used by tree_build_mask and by the attention
// kernel that builds the masks of its request itself.
#pragma once

#include "tv_common.h"

namespace tv {

// p: parent of node `lane` (-1: child of the root, -2: padding); lanes at or
// past N pass -2.  Returns true, in every lane, when the tree is malformed (a
// parent outside {-2, -1} U [0, i), or a node whose parent is a padding slot);
// then anc and depth are 0 in every lane.  Otherwise anc holds bit i and the
// bits of every ancestor of node i, and depth the number of nodes on the
// root-to-i path (both 0 for a padding slot).  Every lane of the wave must
// call it.
__device__ __forceinline__ bool wave_tree_masks(int N, int p, uint64_t& anc, int& depth) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  const bool live = lane < N;
  const int pp = __shfl(p, p >= 0 ? p : 0, 64);      // parent of my parent
  const bool bad = __any(live && (p < -2 || p >= lane || (p >= 0 && pp == -2)));
  const bool node = !bad && live && p != -2;
  anc = node ? 1ull << lane : 0ull;
  depth = node ? 1 : 0;
  // climb: cur = the ancestor reached so far (-1 once past the root).  In a
  // well-formed tree every parent precedes its child, so cur drops at each
  // step and the loop ends within N steps.
  int cur = node ? p : -1;
  for (int step = 0; step < 64 && __any(cur >= 0); ++step) {
    const int up = __shfl(p, cur >= 0 ? cur : 0, 64);   // parent of my current ancestor
    if (cur >= 0) {
      anc |= 1ull << cur;
      ++depth;
      cur = up;
    }
  }
  return bad;
}

// child[u + 1] = the set of nodes whose parent is u, u = -1 .. N-1, written
// to crow[0 .. N].  Each node ORs its bit into its parent's word in s_child
// (LDS, TV_MAX_NODES + 1 words that only this wave uses), then lane u + 1
// stores word u + 1.  bad: the result of wave_tree_masks (all words 0).
__device__ __forceinline__ void wave_child_masks(int N, int p, bool bad, unsigned long long* s_child,
                                                 uint64_t* crow) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  s_child[lane] = 0ull;
  if (lane == 0) s_child[TV_MAX_NODES] = 0ull;
  // LDS operations of one wave complete in issue order; the fence keeps the
  // compiler from reordering the three phases
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (!bad && lane < N && p != -2) atomicOr(&s_child[p + 1], 1ull << lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (lane <= N) crow[lane] = s_child[lane];
  if (lane == 0 && N == TV_MAX_NODES) crow[N] = s_child[N];
}

}  // namespace tv
