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
// decoding.  Long prefixes are cut into several chunks so that the grid has
// enough workgroups; each chunk leaves an unnormalised partial (O, max, sum)
// and a second kernel merges them with log-sum-exp weights.
//
// bf16 path (matrix cores): each wave walks 32-key steps of the chunk (the
// 4 waves interleave steps) and keeps, for all N queries, the running max,
// sum and O in registers.
//   S^T[key][query] = K . Q^T   on v_mfma_f32_16x16x32_bf16
//     (A = 16 keys x 32 dims of K straight from the paged cache,
//      B = 32 dims x 16 queries of Q)
//   O^T[dim][query] += V^T . P^T on the same instruction
//     (A = 16 dims x 32 keys of V^T, B = 32 keys x 16 queries of P^T)
// P^T comes out of the S^T accumulator already in the B-operand layout.  V^T
// is produced without LDS: multiplying the row-major V tile (A operand) by a
// 0/1 selection matrix on the matrix cores is exact and leaves each lane
// holding 4 keys of one dim, the layout the V^T operand needs.
//
// fp32 path (vector ALU): same chunking, K/V tiles staged in LDS, all
// queries of the (b, h) per workgroup.
#include "tv_common.h"

#include <algorithm>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;

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
  void* out;
  float* part_o;             // [B][H][S][Npad][D] unnormalised partial outputs
  float* part_ml;            // [B][H][S][Npad][2] (max in log2 domain, sum)
  int chunk;                 // keys per chunk (multiple of 128)
  int splits;                // S
  int npad;                  // queries padded to a multiple of 16
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

template <int D, int NQT>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(AttnArgs a) {
  constexpr int KC = D / 32;     // 32-dim chunks of the contraction over D
  constexpr int DT = D / 16;     // 16-dim output tiles
  constexpr int NQ = 16 * NQT;   // padded queries

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;

  __shared__ int s_gate;
  __shared__ int s_badblk;
  if (threadIdx.x == 0) {
    s_gate = request_gate(a, b);
    s_badblk = 0;
  }
  __syncthreads();
  const int gate = s_gate;
  if (gate != TV_REQ_OK) {
    if (gate == TV_REQ_KV_CAPACITY && threadIdx.x == 0 && a.status[b] == TV_REQ_OK)
      a.status[b] = TV_REQ_KV_CAPACITY;
    if (a.splits == 1) zero_out<uint16_t>(a, b, h);
    return;
  }
  const int L = a.prefix_len[b];
  const int N = a.N;
  const int T = L + N;
  const int k_begin = s * a.chunk;
  if (k_begin >= T) return;  // empty chunk: the merge never reads it
  const int k_end = min(T, k_begin + a.chunk);

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.kc);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.vc);
  const int32_t* __restrict__ bt = a.block_table + static_cast<size_t>(b) * a.max_blocks;

  // Q^T operand (B of S^T): lane holds Q[n = 16qt + lr][32c + 8lg .. +7].
  // Kept in registers, or - when registers are short (64 queries, D = 128) -
  // in LDS with rows padded by 16 bytes so the 16 rows of one read fall in
  // different banks.
  constexpr bool kQInLds = (NQT == 4 && D == 128);
  constexpr int QROW = D + 8;                      // bf16 elements per LDS row
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kQInLds ? NQ * QROW : 8];
  bf16x8 qv[kQInLds ? 1 : NQT][KC];
  uint64_t ancq[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int n = 16 * qt + lr;
    ancq[qt] = n < N ? a.anc[static_cast<size_t>(b) * N + n] : 0ull;
  }
  if constexpr (kQInLds) {
    for (int e = threadIdx.x; e < NQ * (D / 8); e += kThreads) {
      const int n = e / (D / 8), c8 = e - n * (D / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < N)
        v = *reinterpret_cast<const uint4*>(qg + ((static_cast<size_t>(b) * N + n) * a.H + h) * D + 8 * c8);
      *reinterpret_cast<uint4*>(q_lds + n * QROW + 8 * c8) = v;
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int qt = 0; qt < (kQInLds ? 1 : NQT); ++qt) {
      const int n = 16 * qt + lr;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N)
          v = *reinterpret_cast<const uint4*>(qg + ((static_cast<size_t>(b) * N + n) * a.H + h) * D +
                                              32 * c + 8 * lg);
        qv[qt][c] = as_bf16x8(v);
      }
    }
  }
  auto q_operand = [&](int qt, int c) -> bf16x8 {
    if constexpr (kQInLds)
      return as_bf16x8(*reinterpret_cast<const uint4*>(q_lds + (16 * qt + lr) * QROW + 32 * c + 8 * lg));
    else
      return qv[qt][c];
  };

  // selection matrices for the V transpose: B[k][n] = (k == 16*hh + n)
  bf16x8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint4 v;
    uint32_t w[4];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const int k0 = 8 * lg + 2 * j2;
      const uint32_t lo = (k0 == 16 * hh + lr) ? 0x3F80u : 0u;
      const uint32_t hi = (k0 + 1 == 16 * hh + lr) ? 0x3F80u : 0u;
      w[j2] = lo | (hi << 16);
    }
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    sel[hh] = as_bf16x8(v);
  }

  f32x4 o[NQT][DT];
  float mrun[NQT], lrun[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t head_off = static_cast<size_t>(h) * TV_BLOCK * D;
  const size_t blk_stride = static_cast<size_t>(a.H) * TV_BLOCK * D;
  int badblk = 0;

  // one 32-key step: keys t0 .. t0+31 as two 16-key tiles
  auto load_step = [&](int t0, bf16x8 (&kv)[2][KC], bf16x8 (&vv)[2][KC]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int tt = t0 + 16 * kt;
      int blk = -1;
      if (tt < T) {
        blk = bt[tt / TV_BLOCK];
        if (blk < 0 || blk >= a.num_blocks) {
          badblk = 1;
          blk = -1;
        }
      }
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
        if (blk >= 0) {
          const size_t off = blk * blk_stride + head_off + static_cast<size_t>(lr) * D + 32 * c + 8 * lg;
          kx = *reinterpret_cast<const uint4*>(kg + off);
          vx = *reinterpret_cast<const uint4*>(vg + off);
          if (tt + lr >= T) vx = make_uint4(0, 0, 0, 0);   // rows past the last slot
        }
        kv[kt][c] = as_bf16x8(kx);
        vv[kt][c] = as_bf16x8(vx);
      }
    }
  };

  // Register prefetch of the next step, except for the widest variant where
  // the registers are needed for the accumulators.
  constexpr bool kPrefetch = !(NQT == 4 && D == 128);
  bf16x8 kv[2][KC], vv[2][KC], kn[kPrefetch ? 2 : 1][KC], vn[kPrefetch ? 2 : 1][KC];
  int t0 = k_begin + 32 * wave;
  if (t0 < k_end) load_step(t0, kv, vv);
  for (; t0 < k_end; t0 += 128) {
    const int t1 = t0 + 128;
    if constexpr (kPrefetch) {
      if (t1 < k_end) load_step(t1, kn, vn);
    }

    // 1) scores, online-softmax update and P^T operands for every query tile
    bf16x8 pb[NQT];
    float corr[NQT];
    int rescale[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x4 sc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[kt][c], q_operand(qt, c), acc, 0, 0, 0);
        sc[kt] = acc;
      }
      // mask + scale; lane holds keys t0 + 16kt + 4lg + i for query 16qt + lr
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * kt + 4 * lg + i;
          bool vis = t < T;
          if (t >= L) vis = vis && ((ancq[qt] >> ((t - L) & 63)) & 1ull);
          const float v = vis ? sc[kt][i] * a.scale_log2 : -INFINITY;
          sc[kt][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescaling: the running max only moves (and O is only rescaled)
      // when this tile's max exceeds it by more than 2^8; otherwise
      // probabilities up to 256 are accumulated against the old max, which
      // is exact in the final O / l.
      rescale[qt] = __any(mx > mrun[qt] + 8.f);
      if (rescale[qt]) {
        const float m_new = fmaxf(mrun[qt], mx);
        const float m_use_new = m_new == -INFINITY ? 0.f : m_new;
        corr[qt] = tv::exp2_fast(mrun[qt] - m_use_new);
        mrun[qt] = m_new;
      }
      const float m_use = mrun[qt] == -INFINITY ? 0.f : mrun[qt];
      f32x4 p[2];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = tv::exp2_fast(sc[kt][i] - m_use);
          const float eb = tv::bf16_to_f32(tv::f32_to_bf16(e));   // the value the PV product uses
          p[kt][i] = eb;
          psum += eb;
        }
      }
      if (rescale[qt]) lrun[qt] *= corr[qt];
      lrun[qt] += psum;
      pb[qt] = pack8(p[0], p[1]);
    }

    // 2) V^T tiles for this step (A operand of the PV product), 3) O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 z{0.f, 0.f, 0.f, 0.f};
        const f32x4 t_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv[0][c], sel[hh], z, 0, 0, 0);
        const f32x4 t_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv[1][c], sel[hh], z, 0, 0, 0);
        const bf16x8 va = pack8(t_lo, t_hi);
        const int dt = 2 * c + hh;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
          f32x4 acc = o[qt][dt];
          if (rescale[qt]) {
            acc[0] *= corr[qt]; acc[1] *= corr[qt]; acc[2] *= corr[qt]; acc[3] *= corr[qt];
          }
          o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qt], acc, 0, 0, 0);
        }
      }
    }
    if constexpr (kPrefetch) {
      if (t1 < k_end) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int c = 0; c < KC; ++c) {
            kv[kt][c] = kn[kt][c];
            vv[kt][c] = vn[kt][c];
          }
      }
    } else {
      if (t1 < k_end) load_step(t1, kv, vv);
    }
  }

  // ---- combine the 4 waves: wave 0 absorbs waves 1, 2, 3 through LDS ----
  __shared__ float po[NQ * D];
  __shared__ float pm[NQ], pl[NQ];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    lrun[qt] += __shfl_xor(lrun[qt], 16, 64);
    lrun[qt] += __shfl_xor(lrun[qt], 32, 64);
  }
  if (badblk) s_badblk = 1;
  for (int src = 1; src < 4; ++src) {
    if (wave == src) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        const int n = 16 * qt + lr;
        if (lg == 0) {
          pm[n] = mrun[qt];
          pl[n] = lrun[qt];
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(po + n * D + 16 * dt + 4 * lg) = o[qt][dt];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        const int n = 16 * qt + lr;
        const float m2 = pm[n], l2 = pl[n];
        const float M = fmaxf(mrun[qt], m2);
        const float Mu = M == -INFINITY ? 0.f : M;
        const float w1 = tv::exp2_fast(mrun[qt] - Mu), w2 = tv::exp2_fast(m2 - Mu);
        mrun[qt] = M;
        lrun[qt] = lrun[qt] * w1 + l2 * w2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(po + n * D + 16 * dt + 4 * lg);
          f32x4 r = o[qt][dt];
          r[0] = r[0] * w1 + x[0] * w2;
          r[1] = r[1] * w1 + x[1] * w2;
          r[2] = r[2] * w1 + x[2] * w2;
          r[3] = r[3] * w1 + x[3] * w2;
          o[qt][dt] = r;
        }
      }
    }
    __syncthreads();
  }
  if (s_badblk) {
    if (threadIdx.x == 0) a.status[b] = TV_REQ_BAD_BLOCK;
    return;
  }
  if (wave == 0) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int n = 16 * qt + lr;
      if (lg == 0) {
        pm[n] = mrun[qt];
        pl[n] = lrun[qt];
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(po + n * D + 16 * dt + 4 * lg) = o[qt][dt];
    }
  }
  __syncthreads();
  write_result<uint16_t>(a, b, h, s, po, pm, pl, min(NQ, N));
}

// ===========================================================================
// fp32 vector-ALU kernel
// ===========================================================================
// Thread (n = tid / 4, g = tid % 4) owns query n and output dims
// [g*D/4, (g+1)*D/4).  K/V tiles of 16 keys are staged in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_valu_kernel(AttnArgs a) {
  constexpr int KT = 16;          // keys per tile
  constexpr int DQ = D / 4;       // dims per thread
  constexpr int QS = D + 1;       // padded LDS row stride (floats)
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = threadIdx.x >> 2, g = threadIdx.x & 3;

  __shared__ float q_s[64 * QS];
  __shared__ float k_s[KT * QS];
  __shared__ float v_s[KT * D];
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

  for (int t0 = k_begin; t0 < k_end; t0 += KT) {
    __syncthreads();   // previous tile fully consumed
    int blk = bt[t0 / TV_BLOCK];
    if (blk < 0 || blk >= a.num_blocks) {
      if (threadIdx.x == 0) s_badblk = 1;
      blk = -1;
    }
    for (int e = threadIdx.x; e < KT * D; e += kThreads) {
      const int r = e / D, d = e - r * D;
      float kx = 0.f, vx = 0.f;
      if (blk >= 0 && t0 + r < T) {
        const size_t off = blk * blk_stride + head_off + static_cast<size_t>(r) * D + d;
        kx = kg[off];
        vx = vg[off];
      }
      k_s[r * QS + d] = kx;
      v_s[r * D + d] = vx;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KT / 4; ++j) {
      const int r = 4 * g + j;
      const int t = t0 + r;
      float acc = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) acc = fmaf(q_s[n * QS + d], k_s[r * QS + d], acc);
      bool vis = t < k_end;
      if (t >= L) vis = vis && ((ancn >> ((t - L) & 63)) & 1ull);
      sc_s[n * (KT + 1) + r] = vis ? acc * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
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
#pragma unroll
      for (int j = 0; j < DQ; ++j) o[j] = fmaf(p, v_s[r * D + g * DQ + j], o[j]);
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
// Split merge: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// ===========================================================================
constexpr int kMaxSplits = 64;

template <typename T>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  __shared__ float w_s[kMaxSplits * 64];
  __shared__ float inv_l[64];
  if (a.status[b] != TV_REQ_OK) {
    zero_out<T>(a, b, h);
    return;
  }
  const int N = a.N;
  const int T_ = a.prefix_len[b] + N;
  const int Sb = min(a.splits, (T_ + a.chunk - 1) / a.chunk);
  const size_t base = (static_cast<size_t>(b) * a.H + h) * a.splits;
  for (int n = threadIdx.x; n < N; n += kThreads) {
    float M = -INFINITY;
    for (int s = 0; s < Sb; ++s) M = fmaxf(M, a.part_ml[((base + s) * a.npad + n) * 2]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float l = 0.f;
    for (int s = 0; s < Sb; ++s) {
      const float w = tv::exp2_fast(a.part_ml[((base + s) * a.npad + n) * 2] - Mu);
      w_s[s * 64 + n] = w;
      l += w * a.part_ml[((base + s) * a.npad + n) * 2 + 1];
    }
    inv_l[n] = l > 0.f ? 1.f / l : 0.f;
  }
  __syncthreads();
  T* out = static_cast<T*>(a.out);
  const int D = a.D;
  for (int e = threadIdx.x; e < N * D; e += kThreads) {
    const int n = e / D, d = e - n * D;
    float acc = 0.f;
    for (int s = 0; s < Sb; ++s) acc += w_s[s * 64 + n] * a.part_o[((base + s) * a.npad + n) * D + d];
    store_out<T>(out + ((static_cast<size_t>(b) * N + n) * a.H + h) * D + d, acc * inv_l[n]);
  }
}

// ===========================================================================
// Host side
// ===========================================================================
struct Plan {
  int chunk, splits, npad;
  size_t ws_bytes;
};

Plan make_plan(int B, int N, int H, int D, int max_blocks) {
  Plan p;
  const long keys_max = static_cast<long>(max_blocks) * TV_BLOCK;
  const long bh = static_cast<long>(B) * H;
  long s = (1024 + bh - 1) / bh;                       // aim for >= 1024 workgroups
  s = std::min(s, (keys_max + 511) / 512);             // chunks of at least ~512 keys
  s = std::max(1L, std::min(s, static_cast<long>(kMaxSplits)));
  long c = (keys_max + s - 1) / s;
  c = (c + 127) / 128 * 128;
  p.chunk = static_cast<int>(c);
  p.splits = static_cast<int>((keys_max + c - 1) / c);
  p.npad = (N + 15) / 16 * 16;
  p.ws_bytes = p.splits > 1 ? static_cast<size_t>(B) * H * p.splits * p.npad * (D + 2) * sizeof(float) : 0;
  return p;
}

}  // namespace

extern "C" size_t tree_attn_verify_workspace(tv_dtype dt, int B, int N, int H, int D, int max_blocks) {
  (void)dt;
  if (B <= 0 || N <= 0 || H <= 0 || max_blocks <= 0) return 0;
  return make_plan(B, N, H, D, max_blocks).ws_bytes;
}

template <int D, int NQT>
static void launch_mfma(dim3 grid, hipStream_t st, const AttnArgs& a) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, NQT>), grid, dim3(kThreads), 0, st, a);
}

extern "C" tv_status tree_attn_verify(tv_dtype dt, int B, int N, int H, int D, float scale,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      int num_blocks, int block_size, const int32_t* block_table,
                                      int max_blocks, const int32_t* prefix_len, const uint64_t* anc,
                                      int32_t* status, void* out, void* workspace, size_t ws_bytes,
                                      hipStream_t stream) {
  if (dt != TV_F32 && dt != TV_BF16) return TV_EDTYPE;
  if (B < 0 || N < 0 || H < 1 || (D != 64 && D != 128) || block_size != TV_BLOCK ||
      max_blocks < 1 || num_blocks < 1)
    return TV_EINVAL;
  if (N > TV_MAX_NODES) return TV_ETOOBIG;
  if (B > 65535 || H > 65535) return TV_EINVAL;      // grid y/z limits
  if (B == 0 || N == 0) return TV_OK;
  if (!q || !k_cache || !v_cache || !block_table || !prefix_len || !anc || !status || !out)
    return TV_EINVAL;
  const Plan p = make_plan(B, N, H, D, max_blocks);
  if (p.ws_bytes > 0 && (!workspace || ws_bytes < p.ws_bytes)) return TV_EWORKSPACE;

  AttnArgs a;
  a.B = B; a.N = N; a.H = H; a.D = D;
  a.scale_log2 = scale * kLog2e;
  a.q = q; a.kc = k_cache; a.vc = v_cache;
  a.num_blocks = num_blocks; a.block_table = block_table; a.max_blocks = max_blocks;
  a.prefix_len = prefix_len; a.anc = anc; a.status = status; a.out = out;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = p.ws_bytes ? a.part_o + static_cast<size_t>(B) * H * p.splits * p.npad * D : nullptr;
  a.chunk = p.chunk; a.splits = p.splits; a.npad = p.npad;

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
  } else {
    if (D == 128)
      hipLaunchKernelGGL(attn_valu_kernel<128>, grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_valu_kernel<64>, grid, dim3(kThreads), 0, stream, a);
  }
  if (hipGetLastError() != hipSuccess) return TV_EHIP;
  if (p.splits > 1) {
    if (dt == TV_BF16)
      hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, dim3(H, B), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_merge_kernel<float>, dim3(H, B), dim3(kThreads), 0, stream, a);
  }
  return tv::launch_status();
}
