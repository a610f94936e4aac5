// tree_attn_verify: tree attention over a paged KV cache.
//
// Definition 4.1 of the SpecInfer summary: TreeAttention(u) = Attention(S_u).
// Tree-based parallel decoding computes it for every node in one launch by
// placing the tree tokens after the verified prefix in one KV cache and
// masking scores with the TreeMask rule (node u sees the prefix, its
// ancestors and itself) - section "Tree-based Parallel Decoding:
// Topology-Aware Causal Mask".  Scores are scale * q.k (Equations 1-4).
//
// Work decomposition (MI355X, 256 CUs): one workgroup per (request b, head h,
// key chunk s).  A chunk is a contiguous range of logical key slots; every
// key K/V row is read from HBM exactly once and reused by all N tree queries
// of that (b, h), which is what makes the tree pass cheaper than per-path
// decoding.  The pass is bound by HBM bandwidth, so the bf16 kernel runs one
// workgroup per CU that streams its chunk through LDS (or, when a launch has
// at least three rounds of items, three single-group workgroups per CU that
// take the requests longest first).  The number of chunks
// per (b, h) comes from a small cost
// model: as few as keep every CU busy, because each extra chunk leaves an
// unnormalised partial (O, max, sum) that a second kernel reads back and
// merges with log-sum-exp weights.
//
// bf16 path (matrix cores): K/V stages of 32 keys go HBM -> LDS with
// direct-to-LDS loads that carry the non-temporal hint (each K/V byte is read
// once, so it should not displace cached lines); three independent 4-wave groups per workgroup each
// run a two-buffer ring (48 KB of loads in flight per CU) and take the
// chunk's stages in turn, so every call sums in the same order.  Within a group, wave w < ceil(N/16) owns query
// tile w and keeps its running max, sum and O in registers.  Per 32 keys:
//   S^T[key][query] = K . Q^T     on v_mfma_f32_16x16x32_bf16
//     (A = 16 keys x 32 dims of K from LDS, B = 32 dims x 16 queries of Q)
//   O^T[dim][query] += V^T . P^T  on the same instruction
//     (A = V^T from LDS transpose reads, B = P^T straight from the S^T
//      accumulator, which already has the B-operand layout)
//
// The bf16 kernel can also build the masks itself (tree_mask_attn_verify):
// every workgroup rebuilds its request's masks from the parents with the
// one-wave builder that tree_build_mask uses, and the request's first
// workgroup writes the mask outputs and the status.
//
// fp32 path (vector ALU): chunks of at least 64 keys, 16-key tiles (one
// cache block) staged in LDS with the next tile's loads in flight, all
// queries of the (b, h) per workgroup.
#include "tree_mask.h"

#include <algorithm>
#include <atomic>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;
constexpr int kMaxSplits = 64;                      // chunks per (request, head)
constexpr int kMaxChunkKeys = 32768;                // keys per workgroup chunk (bf16 path)
constexpr int kMaxChunkKeysG1 = 8192;               //   the same for single-group workgroups
constexpr int kRankMaxB = 256;                      // requests the single-group kernel ranks
constexpr int kMaxChunkBlocks = kMaxChunkKeys / TV_BLOCK + 1;

struct AttnArgs {
  int B, N, H, D;
  float scale_log2;          // scale * log2(e)
  const void* q;
  const void* kc;
  const void* vc;
  int num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* prefix_len;
  const uint64_t* anc;
  int32_t* status;
  // masks built in the kernel (attn_mfma_kernel<..., true>): parent [B][N]
  // in, and the tree_build_mask outputs
  const int32_t* parent;
  uint64_t* anc_out;
  uint64_t* child_out;
  int32_t* depth_out;
  void* out;
  float* part_o;             // [B][H][S][Npad][D] unnormalised partial outputs
  float* part_ml;            // [B][H][S][Npad][2] (max in log2 domain, sum)
  int chunk;                 // keys per chunk (multiple of 128)
  int splits;                // S
  int npad;                  // queries padded to a multiple of 16
  int rank;                  // single-group bf16 kernel: take requests longest first
};

// Request-level checks done by every workgroup of request b.  Returns
// 0 to proceed, otherwise the status code (already nonzero ones included).
__device__ __forceinline__ int request_gate(const AttnArgs& a, int b) {
  const int st = a.status[b];
  if (st != TV_REQ_OK) return st;
  const int L = a.prefix_len[b];
  if (L < 0 || static_cast<int64_t>(L) + a.N > static_cast<int64_t>(a.max_blocks) * TV_BLOCK)
    return TV_REQ_KV_CAPACITY;
  return TV_REQ_OK;
}

// A status written while other workgroups of the request run (in-kernel
// masks): a device-scope store, so it reaches memory in the order it is made
// rather than with its XCD's cache at the end of the kernel.
__device__ __forceinline__ void store_status(const AttnArgs& a, int b, int v) {
  __hip_atomic_store(a.status + b, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) { *p = tv::f32_to_bf16(v); }

// Zero the output rows of (b, h): used for requests that are skipped.
template <typename T>
__device__ void zero_out(const AttnArgs& a, int b, int h) {
  T* out = static_cast<T*>(a.out);
  for (int e = threadIdx.x; e < a.N * a.D; e += blockDim.x) {
    const int n = e / a.D, d = e - n * a.D;
    store_out<T>(out + ((static_cast<size_t>(b) * a.N + n) * a.H + h) * a.D + d, 0.f);
  }
}

// Epilogue shared by both paths: the workgroup's combined (O, m, l) for
// query n is in LDS; write either the final output (one chunk) or a partial.
template <typename T>
__device__ void write_result(const AttnArgs& a, int b, int h, int s, const float* o_lds,
                             const float* m_lds, const float* l_lds, int nq) {
  if (a.splits == 1) {
    T* out = static_cast<T*>(a.out);
    for (int e = threadIdx.x; e < a.N * a.D; e += blockDim.x) {
      const int n = e / a.D, d = e - n * a.D;
      const float l = l_lds[n];
      const float v = l > 0.f ? o_lds[n * a.D + d] / l : 0.f;
      store_out<T>(out + ((static_cast<size_t>(b) * a.N + n) * a.H + h) * a.D + d, v);
    }
  } else {
    const size_t base = ((static_cast<size_t>(b) * a.H + h) * a.splits + s) * a.npad;
    for (int e = threadIdx.x; e < nq * a.D; e += blockDim.x)
      a.part_o[base * a.D + e] = o_lds[e];
    for (int n = threadIdx.x; n < nq; n += blockDim.x) {
      a.part_ml[(base + n) * 2 + 0] = m_lds[n];
      a.part_ml[(base + n) * 2 + 1] = l_lds[n];
    }
  }
}

// ===========================================================================
// bf16 matrix-core kernel
// ===========================================================================
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  uint4 r;
  r.x = tv::pack_bf16x2(lo[0], lo[1]);
  r.y = tv::pack_bf16x2(lo[2], lo[3]);
  r.z = tv::pack_bf16x2(hi[0], hi[1]);
  r.w = tv::pack_bf16x2(hi[2], hi[3]);
  return as_bf16x8(r);
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tile of K or V for one 64-key stage: row-major [64 keys][D] bf16 with
// the 16-byte chunks of row r permuted (XOR) so that the 16 rows one matrix
// operand read touches fall in different banks.
template <int D>
__device__ __forceinline__ int swz(int r, int c16) {
  if constexpr (D == 128) return c16 ^ (r & 15);
  else return c16 ^ ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int c16) {   // byte offset
  return r * (2 * D) + swz<D>(r, c16) * 16;
}

// One workgroup per (request b, head h, key chunk s), made of kGroups groups of 4
// waves.  The chunk is cut into stages of 32 keys, dealt to the groups in
// turn (see the loop below); each group runs as if it were a workgroup of its own: a
// two-buffer ring of K/V stages filled HBM -> LDS with direct-to-LDS loads
// (no registers), one stage in flight while the other is read, and its own
// barrier (an LDS counter), so the groups drift independently and one
// group's loads overlap another's matrix work.  NQT waves of a group each own
// one 16-query tile of the tree; every LDS read of a stage is issued before
// its products, so the reads' latency hides behind them.  Per 32 keys and
// query tile:
//   S^T[key][query] = K . Q^T     (A = K rows from LDS, B = Q^T in registers)
//   O^T[dim][query] += V^T . P^T  (A = V^T via LDS transpose reads,
//                                  B = P^T straight from the S^T accumulator)
// At the end the groups' softmax states are merged through LDS; with several
// chunks per (b, h) the merged state is written as an unnormalised partial
// that attn_merge_kernel combines.
//
// G = 1 (the plan's `single`): one group per workgroup and three workgroups
// per CU.  Each item then takes three times as long, but the start and end of
// one workgroup (block ids, status, Q, the first stage's trip; the output)
// overlap the other two's streaming instead of leaving the CU idle.  With
// many rounds the launch's end would then be set by the long items that
// happen to start last, so these workgroups rank the requests by prefix
// length and blockIdx.z = r takes the request of rank r, longest first.
constexpr int kGroups = 3;                  // 4-wave groups per workgroup (G of the default kernel)
constexpr int kRing = 2;                    // stage buffers per group
constexpr int kGroupThreads = 256;
constexpr int kAttnThreads = kGroups * kGroupThreads;
constexpr unsigned kGroupSpinLimit = 1u << 26;

// MASK: the kernel also builds the request's tree masks (one chunk per
// (request, head) only).  Every workgroup of request b reads the parents and
// derives the ancestor masks of its query rows, the tree's validity and the
// request's status from its own loads; workgroup (b, 0, 0) alone writes the
// status (device-scope stores) and the mask outputs of tree_build_mask, so no
// two workgroups write the same word, except a timeout (which comes only after
// a workgroup's spin limit, long after the first workgroup's setup).
template <int D, int NQT, bool MASK, int G>
__global__ __launch_bounds__(G * kGroupThreads) __attribute__((amdgpu_waves_per_eu(3)))
void attn_mfma_kernel(AttnArgs a) {
  constexpr int kGroups = G;
  constexpr int kAttnThreads = G * kGroupThreads;
  constexpr int kMaxChunkBlocks = (G == 1 ? kMaxChunkKeysG1 : kMaxChunkKeys) / TV_BLOCK + 1;
  constexpr int KC = D / 32;               // contraction steps over D
  constexpr int DT = D / 16;               // output dim tiles
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int SK = 32;                   // keys per stage
  constexpr int TILE = SK * D * 2;         // bytes of one K or V stage tile
  constexpr int LPW = (2 * TILE / 1024) / 4;   // 1 KB wave-loads per wave per stage
  static_assert(LPW == 4 || LPW == 2, "stage size");
  constexpr int SLOT = (DT * 4 + 2) * 64;       // floats of one merge slot (see the end)
  static_assert((kGroups - 1) * NQT * SLOT * 4 <= kGroups * kRing * 2 * TILE, "merge area");
  static_assert(kRing >= 2 && kRing <= 4, "ring depth");

  const int s = blockIdx.x, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = wave >> 2, gw = wave & 3;          // group, wave within the group
  const int lr = lane & 15, lg = lane >> 4;

  // per group: kRing stage buffers, each [K tile | V tile]
  __shared__ __attribute__((aligned(16))) uint8_t ring[kGroups * kRing * 2 * TILE];
  // per group: a copy of the (request, head)'s Q rows, in the K tiles' layout
  constexpr int QROWS = 16 * NQT;
  constexpr int QBYTES = QROWS * D * 2;
  static_assert(QBYTES % 1024 == 0, "Q copy in whole wave loads");
  __shared__ __attribute__((aligned(16))) uint8_t sq[kGroups * QBYTES];
  __shared__ int s_hung;
  __shared__ int s_wflag[kAttnThreads / 64];      // per wave: 1 = request skipped, 2 = bad block id
  __shared__ int s_gbar[kGroups];
  __shared__ int s_blk[kMaxChunkBlocks];

  // The request of this workgroup: blockIdx.z, or with a.rank the request of
  // that rank when requests are ordered by prefix length, longest first (ties
  // by index).  Workgroups are dispatched in blockIdx order, so the longest
  // items start first and the launch ends on short ones.  The ranking uses
  // the stage ring, which nothing has written yet.
  int b = blockIdx.z;
  if constexpr (G == 1) {
    if (a.rank) {
      int* s_pl = reinterpret_cast<int*>(ring + 1024);    // clear of the mask builder's child words
      int* s_rb = reinterpret_cast<int*>(ring + 2048);
      const int t = threadIdx.x;
      if (t < a.B) s_pl[t] = a.prefix_len[t];
      __syncthreads();
      if (t < a.B) {
        const int mine = s_pl[t];
        int r = 0;
        for (int i = 0; i < a.B; ++i) {
          const int v = s_pl[i];
          r += (v > mine) | ((v == mine) & (i < t));
        }
        if (r == static_cast<int>(blockIdx.z)) *s_rb = t;
      }
      __syncthreads();
      b = __builtin_amdgcn_readfirstlane(*s_rb);
    }
  }

  // Every load that depends on nothing goes out first, in every thread:
  // the request's status and prefix length (same address in all threads),
  // this wave's Q tile and ancestor masks, and the chunk's block ids.  The
  // prefix length is not written during the launch, so every thread sees
  // the same value; the status can be (another workgroup of the request may
  // flag a bad block), so the workgroup agrees on it at a barrier below.
  // Status and prefix length are read with vector loads (the request index
  // is moved to a vector register first): as scalar loads of a uniform
  // address the compiler issues them where they are first used, after the
  // wait below, and every workgroup would start with two more dependent
  // trips to memory.
  // The kernel arguments the start reads are fetched in one batch of scalar
  // loads (otherwise a second batch waits on the first).
  if constexpr (MASK)
    asm volatile("" :: "s"(a.q), "s"(a.kc), "s"(a.vc), "s"(a.block_table), "s"(a.prefix_len), "s"(a.parent),
                 "s"(a.N), "s"(a.H), "s"(a.num_blocks), "s"(a.max_blocks), "s"(a.chunk));
  else
    asm volatile("" :: "s"(a.q), "s"(a.kc), "s"(a.vc), "s"(a.block_table), "s"(a.prefix_len), "s"(a.anc),
                 "s"(a.status), "s"(a.N), "s"(a.H), "s"(a.num_blocks), "s"(a.max_blocks), "s"(a.chunk));
  const int N = a.N;
  int b_v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(b_v) : "s"(b));
  const int st_v = MASK ? TV_REQ_OK : a.status[b_v];
  const int L_v = a.prefix_len[b_v];
  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  // Query tile of this wave.  Wave gw of a group runs on SIMD gw, so the
  // tile index is rotated by the group: with fewer tiles than waves, the
  // idle waves of different groups sit on different SIMDs and every SIMD
  // carries the same matrix work.
  const int qt = (gw - grp) & 3;
  const bool computes = qt < NQT;
  const int n_q = 16 * qt + lr;
  bf16x8 qv[KC];            // this wave's Q tile: read from the group's copy at its first stage
  uint64_t ancq = 0;
  int par = -2;             // MASK: parent of node `lane` (every wave builds the masks)
  if constexpr (MASK) {
    if (lane < N) par = a.parent[static_cast<size_t>(b) * N + lane];
  } else {
    if (computes && n_q < N) ancq = a.anc[static_cast<size_t>(b) * N + n_q];
  }
  // Block ids of every block the chunk can cover, before the prefix length
  // is known (the table index is clamped to the table).  Ids outside
  // [0, num_blocks) are stored as 0, so every K/V load stays in bounds; the
  // ones that matter (blocks covering the chunk's keys) are reported below.
  const int32_t* __restrict__ bt = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  const int k_begin = s * a.chunk;          // < max_blocks * 16 (the plan's last chunk starts inside)
  const int blk_first = k_begin / TV_BLOCK;
  const int nblk_max = min(a.chunk / TV_BLOCK + 1, a.max_blocks - blk_first);   // <= kMaxChunkBlocks
  constexpr int kPer = (kMaxChunkBlocks + kAttnThreads - 1) / kAttnThreads;
  int raw[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = threadIdx.x + r * kAttnThreads;
    raw[r] = i < nblk_max ? bt[blk_first + i] : 0;
  }
  // A wait the compiler can see: every load above is complete from here on,
  // so it adds no wait of its own inside the stage loop, where a wait would
  // also drain the stage loads in flight, which it does not know about.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));    // vmcnt(0)
  const int L = __builtin_amdgcn_readfirstlane(L_v);
  const bool first_wg = h == 0 && s == 0;
  int st;
  if constexpr (MASK) {
    uint64_t anc_l;
    int dep_l;
    const bool bad_tree = tv::wave_tree_masks(N, par, anc_l, dep_l);
    st = bad_tree ? TV_REQ_BAD_PARENT : TV_REQ_OK;
    const int src = n_q & 63;
    const uint32_t lo = __shfl(static_cast<uint32_t>(anc_l), src, 64);
    const uint32_t hi = __shfl(static_cast<uint32_t>(anc_l >> 32), src, 64);
    ancq = (computes && n_q < N) ? (static_cast<uint64_t>(hi) << 32 | lo) : 0ull;
    if (first_wg && wave == 0) {
      if (lane < N) {
        a.anc_out[static_cast<size_t>(b) * N + lane] = anc_l;
        a.depth_out[static_cast<size_t>(b) * N + lane] = dep_l;
      }
      // (the ring is not written before the barrier below)
      tv::wave_child_masks(N, par, bad_tree, reinterpret_cast<unsigned long long*>(ring),
                           a.child_out + static_cast<size_t>(b) * (N + 1));
    }
  } else {
    st = __builtin_amdgcn_readfirstlane(st_v);
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = threadIdx.x + r * kAttnThreads;
    if (i < nblk_max) s_blk[i] = (raw[r] < 0 || raw[r] >= a.num_blocks) ? 0 : raw[r];
  }
  if (L < 0 || static_cast<int64_t>(L) + N > static_cast<int64_t>(a.max_blocks) * TV_BLOCK) {
    // no workgroup of this request gets further, so no bad-block flag can race this
    if constexpr (MASK) {
      if (first_wg && threadIdx.x == 0) store_status(a, b, st != TV_REQ_OK ? st : TV_REQ_KV_CAPACITY);
    } else {
      if (threadIdx.x == 0 && st == TV_REQ_OK) a.status[b] = TV_REQ_KV_CAPACITY;
    }
    if (s == 0) zero_out<uint16_t>(a, b, h);
    return;
  }
  const int T = L + N;
  if (k_begin >= T) return;                 // empty chunk (never chunk 0): not counted by the merge
  const int k_end = min(T, k_begin + a.chunk);
  const int nst = (k_end - k_begin + SK - 1) / SK;                // stages of the chunk
  const int nblk = (k_end - 1) / TV_BLOCK - blk_first + 1;        // blocks covering the chunk's keys

  const uint8_t* __restrict__ kg = static_cast<const uint8_t*>(a.kc);
  const uint8_t* __restrict__ vg = static_cast<const uint8_t*>(a.vc);
  const size_t head_bytes = static_cast<size_t>(TV_BLOCK) * D * 2;
  const size_t blk_bytes = static_cast<size_t>(a.H) * head_bytes;
  const int last_blk = (T - 1) / TV_BLOCK, last_row = (T - 1) % TV_BLOCK;

  int bad = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = threadIdx.x + r * kAttnThreads;
    if (i < nblk && (raw[r] < 0 || raw[r] >= a.num_blocks)) bad = 1;
  }
  if (threadIdx.x < kGroups) s_gbar[threadIdx.x] = 0;
  if (threadIdx.x == 0) s_hung = 0;
  // The workgroup agrees on the status (another workgroup of the request
  // may flag a bad block meanwhile) and on the bad-block flag with one
  // barrier: each wave leaves its flags in a slot of its own.
  const bool wave_bad = __any(bad);          // (voted by the whole wave)
  if (lane == 0) s_wflag[wave] = (st != TV_REQ_OK ? 1 : 0) | (wave_bad ? 2 : 0);
  __syncthreads();
  int wflags = 0;
#pragma unroll
  for (int w = 0; w < kAttnThreads / 64; ++w) wflags |= s_wflag[w];
  if (wflags & 1) {                          // a skipped request: zero output
    if (MASK && first_wg && threadIdx.x == 0) store_status(a, b, st);
    if (s == 0) zero_out<uint16_t>(a, b, h);
    return;
  }
  const int badblk = wflags & 2;
  // (MASK: one chunk, so this chunk's blocks are all the request's blocks)
  if (MASK && first_wg && threadIdx.x == 0) store_status(a, b, badblk ? TV_REQ_BAD_BLOCK : TV_REQ_OK);

  uint8_t* gring = ring + grp * kRing * 2 * TILE;   // this group's stage buffers
  uint8_t* gq = sq + grp * QBYTES;                   // this group's Q copy

  // The group's Q copy goes HBM -> LDS by direct-to-LDS loads issued just
  // before the group's first stages, so Q is not waited for at the start: a
  // stage's wait (loads complete in issue order) covers the copy, and each
  // wave reads its tile from it at its first stage.  Rows past N repeat row
  // N - 1 (the tile reads zero them).
  auto issue_q = [&]() {
    constexpr int RPL = 1024 / (2 * D);            // rows per 1 KB wave load
    for (int li = gw; li < QBYTES / 1024; li += 4) {
      const int row = li * RPL + lane / CPR, phys = lane % CPR;
      const int n = min(row, N - 1);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(qg + ((static_cast<size_t>(b) * N + n) * a.H + h) * D) +
                           swz<D>(row, phys) * 16;
      const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(gq + li * 1024));
      asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds_addr) : "memory");
    }
  };

  // Issue this wave's share of chunk stage `st` into `dst` (K tile then V
  // tile).  Each 1 KB load covers 64/CPR consecutive keys of one cache
  // block, so its block id is uniform across the wave.  The loads go HBM ->
  // LDS directly; they are issued and awaited by hand (see below).
  auto issue = [&](int st, uint8_t* dst) {
    const int t0 = k_begin + SK * st;
#pragma unroll
    for (int r = 0; r < LPW; ++r) {
      const int li = gw * LPW + r;                   // 1 KB load index within the stage
      const int which = li / (TILE / 1024);          // 0 = K, 1 = V
      const int lt = li % (TILE / 1024);
      const int key0 = lt * (64 / CPR);              // first key of this load
      int blk_i = (t0 + key0) / TV_BLOCK;
      const bool past_blk = blk_i > last_blk;
      if (past_blk) blk_i = last_blk;
      const int blk = __builtin_amdgcn_readfirstlane(s_blk[blk_i - blk_first]);
      const int p = lt * 64 + lane;                  // 16-byte slot within the tile
      const int key = p / CPR, phys = p % CPR;
      const int c16 = swz<D>(key, phys);             // XOR swizzle is its own inverse
      int row = (t0 + key) % TV_BLOCK;
      if (past_blk || (blk_i == last_blk && row > last_row)) row = last_row;   // past the last slot
      const uint8_t* src = (which ? vg : kg) + static_cast<size_t>(blk) * blk_bytes + h * head_bytes +
                           static_cast<size_t>(row) * D * 2 + c16 * 16;
      const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst + which * TILE + lt * 1024));
      // lane i's 16 bytes land at M0 + 16 * i.  The K/V stream is read once:
      // the non-temporal hint (nt) keeps it from displacing cached lines,
      // which measured 5-11% faster launches than default caching (sc0 or
      // sc1 alone changed nothing).
      asm volatile("global_load_lds_dwordx4 %0, off nt" :: "v"(src), "{m0}"(lds_addr) : "memory");
    }
  };

  f32x4 o[DT];
  float mrun = -INFINITY, lrun = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const uint8_t* cur) {
    const int t0 = k_begin + SK * st;
    const uint8_t* kt_base = cur;
    const uint8_t* vt_base = cur + TILE;
    // ---- every LDS read of the stage goes out first: K rows, then the V^T
    // operands (two transpose reads per 16-dim tile: lane s of group lg
    // supplies row 16*half + 4lg + s/4, dims 16dt + 4(s%4) .. +3; lane j then
    // holds those 4 rows at dim 16dt + j), so the V latency hides behind the
    // score products and the softmax ----
    bf16x8 kop[2][KC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        kop[kt][c] = as_bf16x8(*reinterpret_cast<const uint4*>(kt_base + tile_off<D>(16 * kt + lr, 4 * c + lg)));
    typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
    s16x8 vop[DT];
    {
      const int vrow0 = 4 * lg + (lr >> 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d0 = 16 * dt + 4 * (lr & 3);
        const int c16 = d0 >> 3, within = (d0 & 7) * 2;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt_base + tile_off<D>(vrow0, c16) + within));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt_base + tile_off<D>(vrow0 + 16, c16) + within));
        vop[dt] = s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
    }
    // ---- scores S^T for the stage's 32 keys ----
    f32x4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt][c], qv[c], acc, 0, 0, 0);
      sc[kt] = acc;
    }
    // scale and mask: a stage of prefix keys only (all but the last one or
    // two of a chunk) is visible to every node, so only the others test the
    // ancestor bits (branch-free: one select per score)
    float mx = -INFINITY;
    if (t0 + SK <= L) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[kt][i] *= a.scale_log2;
          mx = fmaxf(mx, sc[kt][i]);
        }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * kt + 4 * lg + i;
          const int rel = t - L;
          const bool vis = (t < T) & ((rel < 0) | (((ancq >> (rel & 63)) & 1ull) != 0ull));
          const float v = vis ? sc[kt][i] * a.scale_log2 : -INFINITY;
          sc[kt][i] = v;
          mx = fmaxf(mx, v);
        }
    }
    // Lazy rescaling: the running max (one per query column, uniform over
    // the column's 4 lane groups) moves, and O is rescaled, only when a score
    // exceeds it by more than 2^8; otherwise probabilities up to 256 are
    // accumulated against the old max (exact in O / l).  Only then is the
    // column max formed across lane groups.
    if (__any(mx > mrun + 8.f)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(mrun, mx);
      const float corr = tv::exp2_fast(mrun - (m_new == -INFINITY ? 0.f : m_new));
      mrun = m_new;
      lrun *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt][0] *= corr; o[dt][1] *= corr; o[dt][2] *= corr; o[dt][3] *= corr;
      }
    }
    const float m_use = mrun == -INFINITY ? 0.f : mrun;
    // P in bf16 (the value the PV product uses, rounded by the hardware
    // convert), and l accumulated from the same rounded values
    uint32_t pk[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const f32x2 e2 = {tv::exp2_fast(sc[kt][i] - m_use), tv::exp2_fast(sc[kt][i + 1] - m_use)};
        const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(e2, bf16x2));
        pk[kt * 2 + i / 2] = u;
        lrun += __uint_as_float(u << 16) + __uint_as_float(u & 0xFFFF0000u);
      }
    const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[dt]), pb, o[dt], 0, 0, 0);
  };

  // ---- the group's pipeline: kRing stage buffers, kRing - 1 stages in flight ----
  // Group barrier: the 4 waves of the group count into an LDS word; a wave
  // leaves once all 4 have arrived at this barrier (the count only grows).
  // A wave arrives only after its LDS reads and its stage loads it waited
  // for are complete, so a stage is read only after all its loads landed
  // and refilled only after every wave of the group has read it.  The
  // waits are explicit (the atomics are relaxed: acquire/release would also
  // drain the loads of the stage in flight); the asm statements keep the
  // compiler from moving LDS accesses across the barrier.
  int phase = 0;
  auto group_barrier = [&]() {
    ++phase;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(&s_gbar[grp], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    unsigned polls = 0;
    while (__hip_atomic_load(&s_gbar[grp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < 4 * phase) {
      if (++polls > kGroupSpinLimit) {
        s_hung = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
  };
  auto wait_stage = [&](int later) {        // later stages allowed in flight
    if constexpr (LPW == 4) {
      if (later >= 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      else if (later == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (later >= 3) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else if (later == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };
  // Stages are dealt in turn: group g takes stages g, g + kGroups,
  // g + 2 kGroups, ... in that order, the first kRing of them loading now,
  // the next one whenever a buffer frees up.  Each group thus sums a fixed
  // set of stages in a fixed order, and the groups merge in group order, so
  // the result does not depend on timing: repeated calls give the same bits.
  // (Handing each freed buffer the next unclaimed stage instead balances
  // the groups a little better but makes the summation order, and so the
  // last bits of bf16 outputs, vary from call to call.)  held[0] is the
  // stage being computed, held[1..] the ones in flight; they only grow, so
  // once held[0] is past the chunk every later one is too.
  //
  // In the loop, one barrier per stage: after it, the stage's loads have
  // landed for every wave, and every wave has finished reading the buffer
  // of the stage before, which is then refilled with the group's next
  // stage, in flight during this stage's compute.
  int held[kRing];
  issue_q();
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    held[r] = grp + kGroups * r;
    if (held[r] < nst) issue(held[r], gring + r * 2 * TILE);
  }
  for (int it = 0;; ++it) {
    if (held[0] >= nst) break;
    // in flight: held[1 .. kRing - 1] at it = 0, held[1 .. kRing - 2] after
    // (the last buffer is refilled after this iteration's barrier)
    int later = 0;
#pragma unroll
    for (int r = 1; r < kRing; ++r)
      if ((it == 0 || r < kRing - 1) && held[r] < nst) ++later;
    wait_stage(later);
    group_barrier();
    if (it >= 1) {
      const int nx = grp + kGroups * (it + kRing - 1);
      held[kRing - 1] = nx;
      if (nx >= 0 && nx < nst) issue(nx, gring + ((it + kRing - 1) % kRing) * 2 * TILE);
    }
    if (it == 0 && computes) {
      // the group's Q copy has landed (its loads precede this stage's)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        qv[c] = n_q < N ? as_bf16x8(*reinterpret_cast<const uint4*>(gq + tile_off<D>(n_q, 4 * c + lg)))
                        : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
    if (computes) compute(held[0], gring + (it % kRing) * 2 * TILE);
#pragma unroll
    for (int r = 0; r + 1 < kRing; ++r) held[r] = held[r + 1];
    held[kRing - 1] = INT_MAX;                // set at the next iteration
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lrun += __shfl_xor(lrun, 16, 64);
  lrun += __shfl_xor(lrun, 32, 64);
  __syncthreads();

  // ---- merge the groups' states through LDS (the ring is free now) ----
  // Slot layout [group - 1][query tile][DT*4 + 2][lane] floats: each lane
  // writes and reads only its own column, so there are no bank conflicts.
  float* mg = reinterpret_cast<float*>(ring);
  if (grp > 0 && computes) {
    float* dst = mg + ((grp - 1) * NQT + qt) * SLOT + lane;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(dt * 4 + i) * 64] = o[dt][i];
    dst[(DT * 4) * 64] = mrun;
    dst[(DT * 4 + 1) * 64] = lrun;
  }
  __syncthreads();
  if (!MASK && badblk && threadIdx.x == 0) a.status[b] = TV_REQ_BAD_BLOCK;
  if (s_hung && threadIdx.x == 0) {
    if (MASK) store_status(a, b, TV_REQ_TIMEOUT);
    else a.status[b] = TV_REQ_TIMEOUT;
  }
  if (grp != 0 || !computes) return;
  float mo[kGroups], lo_[kGroups];
  mo[0] = mrun;
  lo_[0] = lrun;
#pragma unroll
  for (int g2 = 1; g2 < kGroups; ++g2) {
    const float* src = mg + ((g2 - 1) * NQT + qt) * SLOT + lane;
    mo[g2] = src[(DT * 4) * 64];
    lo_[g2] = src[(DT * 4 + 1) * 64];
  }
  float M = mo[0];
#pragma unroll
  for (int g2 = 1; g2 < kGroups; ++g2) M = fmaxf(M, mo[g2]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float wgt[kGroups];
  float lsum = 0.f;
#pragma unroll
  for (int g2 = 0; g2 < kGroups; ++g2) {
    wgt[g2] = tv::exp2_fast(mo[g2] - Mu);
    lsum += wgt[g2] * lo_[g2];
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = wgt[0] * o[dt][i];
#pragma unroll
      for (int g2 = 1; g2 < kGroups; ++g2) acc += wgt[g2] * mg[((g2 - 1) * NQT + qt) * SLOT + (dt * 4 + i) * 64 + lane];
      o[dt][i] = acc;
    }

  if (a.splits == 1) {
    if (n_q < N) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + ((static_cast<size_t>(b) * N + n_q) * a.H + h) * D;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 v;
        v.x = tv::pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
        v.y = tv::pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
        *reinterpret_cast<uint2*>(out + 16 * dt + 4 * lg) = v;
      }
    }
    return;
  }
  // ---- several chunks: write this chunk's unnormalised partial ----
  // (merged by attn_merge_kernel after this kernel; the kernel boundary makes
  // the partials of every XCD's L2 visible, no device-scope fence is needed)
  const size_t pbase = ((static_cast<size_t>(b) * a.H + h) * a.splits + s) * a.npad;
  if (n_q < N) {
    float* po = a.part_o + (pbase + n_q) * D;
#pragma unroll
    // (written once and read once by the merge: non-temporal both ways, measured 1-4% faster
    // launches on the split plans)
    for (int dt = 0; dt < DT; ++dt) __builtin_nontemporal_store(o[dt], reinterpret_cast<f32x4*>(po + 16 * dt + 4 * lg));
    if (lg == 0) {
      a.part_ml[(pbase + n_q) * 2 + 0] = M;
      a.part_ml[(pbase + n_q) * 2 + 1] = lsum;
    }
  }
}

// ===========================================================================
// fp32 vector-ALU kernel
// ===========================================================================
// Thread (n = tid / 4, g = tid % 4) owns query n and output dims
// [g*D/4, (g+1)*D/4).  K/V tiles of 16 keys (one cache block) are staged in
// LDS; the next tile's loads are in flight while the current one is used,
// rows are padded to D + 4 floats so every product reads LDS 16 bytes at a
// time (in the same order of summation), and waves whose queries are all past
// N skip the arithmetic.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_valu_kernel(AttnArgs a) {
  constexpr int KT = 16;          // keys per tile (one cache block)
  constexpr int DQ = D / 4;       // dims per thread
  constexpr int QS = D + 4;       // padded LDS row stride (floats), 16-byte aligned
  constexpr int PER = KT * D / kThreads;      // tile elements each thread moves
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = threadIdx.x >> 2, g = threadIdx.x & 3;

  __shared__ __attribute__((aligned(16))) float q_s[64 * QS];
  __shared__ __attribute__((aligned(16))) float k_s[KT * QS];
  __shared__ __attribute__((aligned(16))) float v_s[KT * D];
  __shared__ float sc_s[64 * (KT + 1)];
  __shared__ int s_gate, s_badblk;
  if (threadIdx.x == 0) {
    s_gate = request_gate(a, b);
    s_badblk = 0;
  }
  __syncthreads();
  const int gate = s_gate;
  if (gate != TV_REQ_OK) {
    if (gate == TV_REQ_KV_CAPACITY && threadIdx.x == 0 && a.status[b] == TV_REQ_OK)
      a.status[b] = TV_REQ_KV_CAPACITY;
    if (a.splits == 1) zero_out<float>(a, b, h);
    return;
  }
  const int N = a.N;
  const int L = a.prefix_len[b];
  const int T = L + N;
  const int k_begin = s * a.chunk;
  if (k_begin >= T) return;
  const int k_end = min(T, k_begin + a.chunk);
  const float* __restrict__ qg = static_cast<const float*>(a.q);
  const float* __restrict__ kg = static_cast<const float*>(a.kc);
  const float* __restrict__ vg = static_cast<const float*>(a.vc);
  const int32_t* __restrict__ bt = a.block_table + static_cast<size_t>(b) * a.max_blocks;

  for (int e = threadIdx.x; e < 64 * D; e += kThreads) {
    const int qn = e / D, d = e - qn * D;
    q_s[qn * QS + d] = qn < N ? qg[((static_cast<size_t>(b) * N + qn) * a.H + h) * D + d] : 0.f;
  }
  const uint64_t ancn = n < N ? a.anc[static_cast<size_t>(b) * N + n] : 0ull;
  float o[DQ];
#pragma unroll
  for (int j = 0; j < DQ; ++j) o[j] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const size_t head_off = static_cast<size_t>(h) * TV_BLOCK * D;
  const size_t blk_stride = static_cast<size_t>(a.H) * TV_BLOCK * D;

  // this thread's share of a tile, fetched into registers one tile ahead
  float kn[PER], vn[PER];
  auto fetch = [&](int t0) {
    int blk = bt[t0 / TV_BLOCK];
    if (blk < 0 || blk >= a.num_blocks) {
      if (threadIdx.x == 0) s_badblk = 1;
      blk = -1;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int r = e / D, d = e - r * D;
      kn[i] = vn[i] = 0.f;
      if (blk >= 0 && t0 + r < T) {
        const size_t off = blk * blk_stride + head_off + static_cast<size_t>(r) * D + d;
        kn[i] = kg[off];
        vn[i] = vg[off];
      }
    }
  };
  const bool rows_here = 16 * static_cast<int>(threadIdx.x >> 6) < N;   // (wave-uniform)
  fetch(k_begin);
  for (int t0 = k_begin; t0 < k_end; t0 += KT) {
    __syncthreads();   // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * kThreads;
      const int r = e / D, d = e - r * D;
      k_s[r * QS + d] = kn[i];
      v_s[r * D + d] = vn[i];
    }
    __syncthreads();
    if (t0 + KT < k_end) fetch(t0 + KT);      // in flight during this tile
    if (!rows_here) continue;
    const float4* qrow = reinterpret_cast<const float4*>(q_s + n * QS);
#pragma unroll
    for (int j = 0; j < KT / 4; ++j) {
      const int r = 4 * g + j;
      const int t = t0 + r;
      const float4* krow = reinterpret_cast<const float4*>(k_s + r * QS);
      float acc = 0.f;
#pragma unroll 4
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 qv = qrow[d4], kv = krow[d4];
        acc = fmaf(qv.x, kv.x, acc);
        acc = fmaf(qv.y, kv.y, acc);
        acc = fmaf(qv.z, kv.z, acc);
        acc = fmaf(qv.w, kv.w, acc);
      }
      bool vis = t < k_end;
      if (t >= L) vis = vis && ((ancn >> ((t - L) & 63)) & 1ull);
      sc_s[n * (KT + 1) + r] = vis ? acc * a.scale_log2 : -INFINITY;
    }
    // the four threads of query n exchange their scores through LDS (a
    // wave's own writes and reads, in order)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < KT; ++r) mx = fmaxf(mx, sc_s[n * (KT + 1) + r]);
    const float m_new = fmaxf(mrun, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float corr = tv::exp2_fast(mrun - m_use);
    mrun = m_new;
    lrun *= corr;
#pragma unroll
    for (int j = 0; j < DQ; ++j) o[j] *= corr;
#pragma unroll
    for (int r = 0; r < KT; ++r) {
      const float p = tv::exp2_fast(sc_s[n * (KT + 1) + r] - m_use);
      lrun += p;
      const float4* vrow = reinterpret_cast<const float4*>(v_s + r * D + g * DQ);
#pragma unroll
      for (int j4 = 0; j4 < DQ / 4; ++j4) {
        const float4 vv = vrow[j4];
        o[4 * j4] = fmaf(p, vv.x, o[4 * j4]);
        o[4 * j4 + 1] = fmaf(p, vv.y, o[4 * j4 + 1]);
        o[4 * j4 + 2] = fmaf(p, vv.z, o[4 * j4 + 2]);
        o[4 * j4 + 3] = fmaf(p, vv.w, o[4 * j4 + 3]);
      }
    }
  }
  __syncthreads();
  if (s_badblk) {
    if (threadIdx.x == 0) a.status[b] = TV_REQ_BAD_BLOCK;
    return;
  }
  if (n >= N) return;
  if (a.splits == 1) {
    float* out = static_cast<float*>(a.out) + ((static_cast<size_t>(b) * N + n) * a.H + h) * D + g * DQ;
    const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
    for (int j = 0; j < DQ; ++j) out[j] = o[j] * inv;
  } else {
    const size_t base = (((static_cast<size_t>(b) * a.H + h) * a.splits + s) * a.npad + n);
#pragma unroll
    for (int j = 0; j < DQ; ++j) a.part_o[base * D + g * DQ + j] = o[j];
    if (g == 0) {
      a.part_ml[base * 2 + 0] = mrun;
      a.part_ml[base * 2 + 1] = lrun;
    }
  }
}

// ===========================================================================
// Split merge: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per 4 output dims of (b, n, h): the loads of a thread are
// independent, so the kernel runs at the speed of its reads.
// ===========================================================================
template <typename T>
__device__ __forceinline__ void store4(T* p, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float x0, float x1, float x2, float x3) {
  uint2 v;
  v.x = tv::pack_bf16x2(x0, x1);
  v.y = tv::pack_bf16x2(x2, x3);
  *reinterpret_cast<uint2*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnArgs a) {
  const int D4 = a.D / 4;
  const size_t idx = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  const size_t total = static_cast<size_t>(a.B) * a.N * a.H * D4;
  if (idx >= total) return;
  const int d4 = static_cast<int>(idx % D4);
  const int h = static_cast<int>((idx / D4) % a.H);
  const int n = static_cast<int>((idx / D4 / a.H) % a.N);
  const int b = static_cast<int>(idx / D4 / a.H / a.N);
  T* out = static_cast<T*>(a.out) + ((static_cast<size_t>(b) * a.N + n) * a.H + h) * a.D + 4 * d4;
  if (a.status[b] != TV_REQ_OK) {
    store4<T>(out, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int T_ = a.prefix_len[b] + a.N;
  const int Sb = min(a.splits, (T_ + a.chunk - 1) / a.chunk);
  const size_t bh = (static_cast<size_t>(b) * a.H + h) * a.splits;
  float M = -INFINITY;
  for (int s = 0; s < Sb; ++s) M = fmaxf(M, a.part_ml[((bh + s) * a.npad + n) * 2]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float l = 0.f;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < Sb; ++s) {
    const size_t row = (bh + s) * a.npad + n;
    const float w = tv::exp2_fast(a.part_ml[row * 2] - Mu);
    l += w * a.part_ml[row * 2 + 1];
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.part_o + row * a.D + 4 * d4));
    acc[0] += w * x[0]; acc[1] += w * x[1]; acc[2] += w * x[2]; acc[3] += w * x[3];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  store4<T>(out, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
}

// ===========================================================================
// Host side
// ===========================================================================
struct Plan {
  int chunk, splits, npad;
  bool single;               // bf16: single-group workgroups, requests longest first
  size_t off_ml, ws_bytes;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// bf16 attention workgroups resident at once on the current device
// (compute units x workgroups per CU at head dim D; cached per device: every
// thread that fills an entry computes the same value, so relaxed atomics
// suffice).
int attn_slots(int D) {
  static std::atomic<int> cache[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const int di = D == 128 ? 1 : 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev][di].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const void* fn = D == 128 ? reinterpret_cast<const void*>(attn_mfma_kernel<128, 4, false, kGroups>)
                            : reinterpret_cast<const void*>(attn_mfma_kernel<64, 4, false, kGroups>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kAttnThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int slots = cus * per_cu;
  if (dev >= 0 && dev < 64) cache[dev][di].store(slots, std::memory_order_relaxed);
  return slots;
}

// Chunking of the key range.
// bf16: a launch runs in rounds of as many workgroups as are resident at
// once (one per CU at D = 128); the chunk count minimises rounds x (chunk keys + the partial
// written and read back, 2 * npad key-equivalents) + the merge launch
// (about 4 us, ~19000 / D key-loads of one CU).
// fp32: about 512 workgroups, chunks of at least 256 keys.
Plan make_plan(tv_dtype dt, int B, int N, int H, int D, int max_blocks) {
  Plan p;
  const long keys_max = static_cast<long>(max_blocks) * TV_BLOCK;
  const long pairs = static_cast<long>(B) * H;
  p.npad = (N + 15) / 16 * 16;
  long c = 0;
  if (dt == TV_BF16) {
    const long slots = attn_slots(D);
    const double merge_keys = 19000.0 / D;
    const long s_min = (keys_max + kMaxChunkKeys - 1) / kMaxChunkKeys;
    double best = 0.0;
    for (long s = s_min; s <= std::max<long>(s_min, kMaxSplits); ++s) {
      long cs = (keys_max + s - 1) / s;
      cs = (cs + 63) / 64 * 64;
      const long se = (keys_max + cs - 1) / cs;
      if (se != s) continue;                          // same chunking as a smaller s
      const long rounds = (pairs * se + slots - 1) / slots;
      const double cost = static_cast<double>(rounds) * (static_cast<double>(cs) + (se > 1 ? 2.0 * p.npad : 0.0)) +
                          (se > 1 ? merge_keys : 0.0);
      if (c == 0 || cost < best) {
        best = cost;
        c = cs;
      }
    }
  } else {
    long s = (512 + pairs - 1) / pairs;
    s = std::min(s, (keys_max + 63) / 64);         // chunks of at least 64 keys
    s = std::max(1L, std::min(s, static_cast<long>(kMaxSplits)));
    c = (keys_max + s - 1) / s;
    c = (c + 63) / 64 * 64;
  }
  p.chunk = static_cast<int>(c);
  p.splits = static_cast<int>((keys_max + c - 1) / c);
  // With one chunk per (request, head) and at least three rounds of
  // workgroups, three single-group workgroups share each CU and the requests
  // are taken longest first: one workgroup's start and end then overlap the
  // other two's streaming, and the launch ends on its shortest items.
  p.single = dt == TV_BF16 && p.splits == 1 && p.chunk <= kMaxChunkKeysG1 && B <= kRankMaxB &&
             pairs >= 3L * attn_slots(D);
  if (p.splits > 1) {
    const size_t rows = static_cast<size_t>(B) * H * p.splits * p.npad;
    p.off_ml = align256(rows * D * sizeof(float));
    p.ws_bytes = p.off_ml + align256(rows * 2 * sizeof(float));
  } else {
    p.off_ml = p.ws_bytes = 0;
  }
  return p;
}

}  // namespace

extern "C" size_t tree_attn_verify_workspace(tv_dtype dt, int B, int N, int H, int D, int max_blocks) {
  if (B <= 0 || N <= 0 || H <= 0 || max_blocks <= 0) return 0;
  if (dt != TV_F32 && dt != TV_BF16) return 0;
  return make_plan(dt, B, N, H, D, max_blocks).ws_bytes;
}

template <int D, int NQT, bool MASK = false>
static void launch_mfma(dim3 grid, hipStream_t st, const AttnArgs& a) {
  if (a.rank)
    hipLaunchKernelGGL((attn_mfma_kernel<D, NQT, MASK, 1>), grid, dim3(kGroupThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, NQT, MASK, kGroups>), grid, dim3(kAttnThreads), 0, st, a);
}

// Argument checks shared by both entry points and the kernel arguments;
// ptrs_ok: the caller's own pointers (anc, or the mask's) are non-null.
static tv_status attn_setup(tv_dtype dt, int B, int N, int H, int D, float scale, const void* q,
                            const void* k_cache, const void* v_cache, int num_blocks, int block_size,
                            const int32_t* block_table, int max_blocks, const int32_t* prefix_len,
                            int32_t* status, void* out, void* workspace, size_t ws_bytes, bool ptrs_ok,
                            AttnArgs& a, Plan& p) {
  if (dt != TV_F32 && dt != TV_BF16) return TV_EDTYPE;
  if (B < 0 || N < 0 || H < 1 || (D != 64 && D != 128) || block_size != TV_BLOCK ||
      max_blocks < 1 || num_blocks < 1)
    return TV_EINVAL;
  if (N > TV_MAX_NODES) return TV_ETOOBIG;
  if (B > 65535 || H > 65535) return TV_EINVAL;      // grid y/z limits
  if (B == 0 || N == 0) return TV_OK;
  if (!q || !k_cache || !v_cache || !block_table || !prefix_len || !status || !out || !ptrs_ok)
    return TV_EINVAL;
  p = make_plan(dt, B, N, H, D, max_blocks);
  if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes)) return TV_EWORKSPACE;

  a = AttnArgs{};
  a.B = B; a.N = N; a.H = H; a.D = D;
  a.scale_log2 = scale * kLog2e;
  a.q = q; a.kc = k_cache; a.vc = v_cache;
  a.num_blocks = num_blocks; a.block_table = block_table; a.max_blocks = max_blocks;
  a.prefix_len = prefix_len; a.status = status; a.out = out;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.part_o = p.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_ml = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
  a.chunk = p.chunk; a.splits = p.splits; a.npad = p.npad;
  a.rank = p.single ? 1 : 0;
  return TV_OK;
}

extern "C" tv_status tree_attn_verify(tv_dtype dt, int B, int N, int H, int D, float scale,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      int num_blocks, int block_size, const int32_t* block_table,
                                      int max_blocks, const int32_t* prefix_len, const uint64_t* anc,
                                      int32_t* status, void* out, void* workspace, size_t ws_bytes,
                                      hipStream_t stream) {
  AttnArgs a;
  Plan p;
  const tv_status e = attn_setup(dt, B, N, H, D, scale, q, k_cache, v_cache, num_blocks, block_size,
                                 block_table, max_blocks, prefix_len, status, out, workspace, ws_bytes,
                                 anc != nullptr, a, p);
  if (e != TV_OK || B == 0 || N == 0) return e;
  a.anc = anc;

  const dim3 grid(p.splits, H, B);
  if (dt == TV_BF16) {
    const int nqt = (N + 15) / 16;
    if (D == 128) {
      switch (nqt) {
        case 1: launch_mfma<128, 1>(grid, stream, a); break;
        case 2: launch_mfma<128, 2>(grid, stream, a); break;
        case 3: launch_mfma<128, 3>(grid, stream, a); break;
        default: launch_mfma<128, 4>(grid, stream, a); break;
      }
    } else {
      switch (nqt) {
        case 1: launch_mfma<64, 1>(grid, stream, a); break;
        case 2: launch_mfma<64, 2>(grid, stream, a); break;
        case 3: launch_mfma<64, 3>(grid, stream, a); break;
        default: launch_mfma<64, 4>(grid, stream, a); break;
      }
    }
  } else if (D == 128) {
    hipLaunchKernelGGL(attn_valu_kernel<128>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_valu_kernel<64>, grid, dim3(kThreads), 0, stream, a);
  }
  if (hipGetLastError() != hipSuccess) return TV_EHIP;
  if (p.splits > 1) {
    const size_t threads = static_cast<size_t>(B) * N * H * (D / 4);
    const dim3 mgrid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
    if (dt == TV_BF16)
      hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, mgrid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_merge_kernel<float>, mgrid, dim3(kThreads), 0, stream, a);
  }
  return tv::launch_status();
}

extern "C" tv_status tree_mask_attn_verify(tv_dtype dt, int B, int N, int H, int D, float scale,
                                           const void* q, const void* k_cache, const void* v_cache,
                                           int num_blocks, int block_size, const int32_t* block_table,
                                           int max_blocks, const int32_t* prefix_len,
                                           const int32_t* parent, uint64_t* anc, uint64_t* child,
                                           int32_t* depth, int32_t* status, void* out, void* workspace,
                                           size_t ws_bytes, hipStream_t stream) {
  AttnArgs a;
  Plan p;
  const tv_status e = attn_setup(dt, B, N, H, D, scale, q, k_cache, v_cache, num_blocks, block_size,
                                 block_table, max_blocks, prefix_len, status, out, workspace, ws_bytes,
                                 parent && anc && child && depth, a, p);
  if (e != TV_OK || B == 0) return e;
  if (!child || !status) return TV_EINVAL;          // (N = 0: only the mask's outputs)
  if (N == 0) return tree_build_mask(B, N, parent, anc, child, depth, status, stream);
  if (dt != TV_BF16 || p.splits > 1) {
    // the two calls this one stands for
    const tv_status r = tree_build_mask(B, N, parent, anc, child, depth, status, stream);
    if (r != TV_OK) return r;
    return tree_attn_verify(dt, B, N, H, D, scale, q, k_cache, v_cache, num_blocks, block_size, block_table,
                            max_blocks, prefix_len, anc, status, out, workspace, ws_bytes, stream);
  }
  a.parent = parent;
  a.anc_out = anc;
  a.child_out = child;
  a.depth_out = depth;
  const dim3 grid(1, H, B);
  const int nqt = (N + 15) / 16;
  if (D == 128) {
    switch (nqt) {
      case 1: launch_mfma<128, 1, true>(grid, stream, a); break;
      case 2: launch_mfma<128, 2, true>(grid, stream, a); break;
      case 3: launch_mfma<128, 3, true>(grid, stream, a); break;
      default: launch_mfma<128, 4, true>(grid, stream, a); break;
    }
  } else {
    switch (nqt) {
      case 1: launch_mfma<64, 1, true>(grid, stream, a); break;
      case 2: launch_mfma<64, 2, true>(grid, stream, a); break;
      case 3: launch_mfma<64, 3, true>(grid, stream, a); break;
      default: launch_mfma<64, 4, true>(grid, stream, a); break;
    }
  }
  return tv::launch_status();
}
