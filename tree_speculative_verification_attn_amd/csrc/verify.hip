// tree_verify_greedy / tree_verify_mss: verification of a token tree.
//
// SpecInfer summary, "Token Verification: Greedy Decoding (VerifyGreedy)" and
// "Token Verification: Stochastic Decoding and Multi-Step Speculative
// Sampling (VerifyStochastic)"; the leaf bonus token and the zero-normaliser
// guard follow the wiki concept page "Speculative decoding", "Implementation
// sketch".
//
// Two phases, both on the GPU so no logits travel to the host:
//  1. row_stats: one pass over every target logits row (B * (N+1) rows of V
//     floats, the dominant HBM traffic).  Rows are cut into pieces of 8192
//     values so that even a few requests fill the chip; each piece yields
//     (max, sum of exp(l - max) in fp64, first index of the max, NaN/+inf
//     flags).  Consumers merge the pieces of the rows they visit.
//  2. the walk: one workgroup per request.
//     greedy: one wave; integer walk over the child bitmasks.
//     MSS: 1024 threads; control decisions on thread 0, and every full-vocab
//     step (a residual after a rejection, the final inverse-CDF sample) as a
//     parallel pass with fp64 accumulation.
#include "tv_common.h"

namespace {

constexpr int kPiece = 8192;               // logits per row_stats workgroup
constexpr int kStatThreads = 256;
constexpr int kPerThread = kPiece / kStatThreads;   // 32
constexpr int kWalkThreads = 1024;

enum : int { FLAG_NAN = 1, FLAG_PINF = 2, FLAG_FINITE = 4 };

struct Stats {            // views into the workspace
  float* m;               // [rows][P]
  int* arg;               // [rows][P]
  int* flag;              // [rows][P]
  double* s;              // [rows][P]
  int P;
};

__host__ __device__ inline int num_pieces(int V) { return (V + kPiece - 1) / kPiece; }

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct WsLayout {
  size_t off_m, off_arg, off_flag, off_s, off_res, total;
};

WsLayout ws_layout(int B, int N, int V) {
  const size_t rows = static_cast<size_t>(B) * (N + 1);
  const size_t P = num_pieces(V);
  WsLayout w;
  w.off_m = 0;
  w.off_arg = align256(w.off_m + rows * P * sizeof(float));
  w.off_flag = align256(w.off_arg + rows * P * sizeof(int));
  w.off_s = align256(w.off_flag + rows * P * sizeof(int));
  w.off_res = align256(w.off_s + rows * P * sizeof(double));
  w.total = align256(w.off_res + 2 * static_cast<size_t>(B) * V * sizeof(float));
  return w;
}

Stats stats_view(void* ws, const WsLayout& w, int V) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  Stats s;
  s.m = reinterpret_cast<float*>(p + w.off_m);
  s.arg = reinterpret_cast<int*>(p + w.off_arg);
  s.flag = reinterpret_cast<int*>(p + w.off_flag);
  s.s = reinterpret_cast<double*>(p + w.off_s);
  s.P = num_pieces(V);
  return s;
}

// ---------------------------------------------------------------------------
// Phase 1: per-piece row statistics.  grid (P, rows).  kWithSum = false
// computes only the argmax and flags (greedy).
// ---------------------------------------------------------------------------
template <bool kWithSum>
__global__ __launch_bounds__(kStatThreads) void row_stats_kernel(const float* __restrict__ logits,
                                                                 int V, Stats st) {
  const size_t row = blockIdx.x;
  const int p = blockIdx.y;
  const float* __restrict__ lr = logits + row * static_cast<size_t>(V);
  const int x0 = p * kPiece;
  const int x1 = min(V, x0 + kPiece);
  const int t = threadIdx.x;

  float v[kPerThread];
  // thread t holds x = x0 + 4*t + 1024*k + e (k < 8, e < 4): coalesced
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    const int xb = x0 + 4 * t + 1024 * k;
    if (vec && xb + 3 < x1) {
      const float4 f = *reinterpret_cast<const float4*>(lr + xb);
      v[4 * k + 0] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * k + e] = (xb + e < x1) ? lr[xb + e] : -INFINITY;
    }
  }
  float mx = -INFINITY;
  int arg = 0x7FFFFFFF;
  int flags = 0;
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = x0 + 4 * t + 1024 * k + e;
      const float f = v[4 * k + e];
      if (x < x1) {
        if (f != f) flags |= FLAG_NAN;
        else if (f == INFINITY) flags |= FLAG_PINF;
        else if (f != -INFINITY) flags |= FLAG_FINITE;
        if (f > mx || (f == mx && x < arg && f == f)) {
          mx = f;
          arg = x;
        }
      }
    }
  }
  // workgroup reduction of (max, first index, flags)
  __shared__ float r_m[kStatThreads / 64];
  __shared__ int r_a[kStatThreads / 64], r_f[kStatThreads / 64];
  __shared__ double r_s[kStatThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64);
    const int a2 = __shfl_xor(arg, o, 64);
    if (m2 > mx || (m2 == mx && a2 < arg)) {
      mx = m2;
      arg = a2;
    }
    flags |= __shfl_xor(flags, o, 64);
  }
  const int wave = t >> 6, lane = t & 63;
  if (lane == 0) {
    r_m[wave] = mx;
    r_a[wave] = arg;
    r_f[wave] = flags;
  }
  __syncthreads();
  float M = r_m[0];
  int A = r_a[0];
  int F = r_f[0];
  for (int w = 1; w < kStatThreads / 64; ++w) {
    if (r_m[w] > M || (r_m[w] == M && r_a[w] < A)) {
      M = r_m[w];
      A = r_a[w];
    }
    F |= r_f[w];
  }
  double S = 0.0;
  if (kWithSum && M != -INFINITY && M == M) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const float f = v[k];
      if (f != -INFINITY) acc += static_cast<double>(tv::exp_acc(f - M));
    }
    acc = tv::wave_sum(acc);
    if (lane == 0) r_s[wave] = acc;
    __syncthreads();
    for (int w = 0; w < kStatThreads / 64; ++w) S += r_s[w];
  }
  if (t == 0) {
    const size_t i = row * st.P + p;
    st.m[i] = M;
    st.arg[i] = A == 0x7FFFFFFF ? x0 : A;
    st.flag[i] = F;
    if (kWithSum) st.s[i] = S;
  }
}

// Children of u can only be nodes u+1 .. N-1 (parents precede children).
// Masking with this keeps every walk finite and in bounds even for child
// masks that did not come from tree_build_mask.
__device__ __forceinline__ uint64_t later_nodes(int u, int N) {
  const uint64_t below_n = N >= 64 ? ~0ull : ((1ull << N) - 1);
  const uint64_t upto_u = u < 0 ? 0ull : (u >= 63 ? ~0ull : ((2ull << u) - 1));
  return below_n & ~upto_u;
}

// Merge the pieces of one row (single thread).
struct RowStat {
  float m;
  double s;
  int arg;
  bool ok;   // no NaN, no +inf, some finite value
};

__device__ RowStat merge_row(const Stats& st, size_t row, bool with_sum) {
  RowStat r;
  r.m = -INFINITY;
  r.arg = 0;
  r.s = 0.0;
  int F = 0;
  for (int p = 0; p < st.P; ++p) {
    const size_t i = row * st.P + p;
    const float m = st.m[i];
    F |= st.flag[i];
    if (m > r.m) {          // strict: the earlier piece keeps ties
      r.m = m;
      r.arg = st.arg[i];
    }
  }
  r.ok = !(F & (FLAG_NAN | FLAG_PINF)) && (F & FLAG_FINITE);
  if (with_sum && r.ok) {
    for (int p = 0; p < st.P; ++p) {
      const size_t i = row * st.P + p;
      const float m = st.m[i];
      if (m != -INFINITY) r.s += st.s[i] * exp(static_cast<double>(m) - static_cast<double>(r.m));
    }
  }
  return r;
}

// Per-request small arrays staged in LDS by the walk kernels.
struct ReqLds {
  int tok[TV_MAX_NODES];
  int qrow[TV_MAX_NODES];
  uint64_t child[TV_MAX_NODES + 1];
  // merged statistics of every row (root + nodes)
  float m[TV_MAX_NODES + 1];
  double s[TV_MAX_NODES + 1];
  int arg[TV_MAX_NODES + 1];
  int ok[TV_MAX_NODES + 1];
};

// Load tokens, draft rows and child masks, merge every row's pieces, and run
// the up-front checks.  Returns the request status (shared by all threads).
// Tokens and draft rows are only checked for nodes that are somebody's child
// (padding slots are nobody's child).
__device__ int stage_request(ReqLds& R, int b, int N, int V, int Rrows, const int32_t* token,
                             const int32_t* q_row, const uint64_t* child, const Stats& st,
                             bool with_sum, int status_in, uint64_t* s_real, int* s_flag) {
  const int t = threadIdx.x;
  if (t == 0) {
    *s_real = 0ull;
    *s_flag = 0;
  }
  __syncthreads();
  for (int i = t; i <= N; i += blockDim.x) {
    const uint64_t c = child[static_cast<size_t>(b) * (N + 1) + i] & later_nodes(i - 1, N);
    R.child[i] = c;
    if (c) atomicOr(reinterpret_cast<unsigned long long*>(s_real), static_cast<unsigned long long>(c));
    const RowStat r = merge_row(st, static_cast<size_t>(b) * (N + 1) + i, with_sum);
    R.m[i] = r.m;
    R.s[i] = r.s;
    R.arg[i] = r.arg;
    R.ok[i] = r.ok;
  }
  for (int i = t; i < N; i += blockDim.x) {
    R.tok[i] = token[static_cast<size_t>(b) * N + i];
    R.qrow[i] = q_row ? q_row[static_cast<size_t>(b) * N + i] : 0;
  }
  __syncthreads();
  const uint64_t real = *s_real;
  for (int i = t; i < N; i += blockDim.x) {
    if ((real >> i) & 1ull) {
      if (R.tok[i] < 0 || R.tok[i] >= V) atomicOr(s_flag, 1);
      if (q_row && (R.qrow[i] < 0 || R.qrow[i] >= Rrows)) atomicOr(s_flag, 2);
    }
  }
  __syncthreads();
  if (status_in != TV_REQ_OK) return status_in;
  const int f = *s_flag;
  if (f & 1) return TV_REQ_BAD_TOKEN;
  if (f & 2) return TV_REQ_BAD_QROW;
  return TV_REQ_OK;
}

// ---------------------------------------------------------------------------
// Phase 2a: greedy walk, one workgroup of one wave per request.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void greedy_walk_kernel(int N, int V, const int32_t* __restrict__ token,
                                                         const uint64_t* __restrict__ child,
                                                         int32_t* __restrict__ status,
                                                         int32_t* __restrict__ accepted,
                                                         int32_t* __restrict__ num_accepted,
                                                         int32_t* __restrict__ bonus, Stats st) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ ReqLds R;
  __shared__ uint64_t s_real;
  __shared__ int s_flag, s_k;
  __shared__ int s_acc[TV_MAX_NODES];
  int stt = stage_request(R, b, N, V, 0, token, nullptr, child, st, false, status[b], &s_real, &s_flag);
  if (t == 0) {
    int k = 0, bn = -1;
    if (stt == TV_REQ_OK) {
      int u = -1;
      while (true) {
        if (!R.ok[u + 1]) {
          stt = TV_REQ_NONFINITE;
          break;
        }
        const int o = R.arg[u + 1];
        uint64_t kids = R.child[u + 1];
        int nxt = -1;
        while (kids) {
          const int c = __builtin_ctzll(kids);
          kids &= kids - 1;
          if (R.tok[c] == o) {
            nxt = c;
            break;
          }
        }
        if (nxt < 0) {
          bn = o;
          break;
        }
        s_acc[k++] = nxt;
        u = nxt;
      }
    }
    if (stt != TV_REQ_OK) {
      status[b] = stt;
      num_accepted[b] = -1;
      bonus[b] = -1;
      k = 0;
    } else {
      num_accepted[b] = k;
      bonus[b] = bn;
    }
    s_k = k;
  }
  __syncthreads();
  for (int i = t; i < N; i += blockDim.x) accepted[static_cast<size_t>(b) * N + i] = i < s_k ? s_acc[i] : -1;
}

// ---------------------------------------------------------------------------
// Phase 2b: multi-step speculative sampling, one 1024-thread workgroup per
// request.  The current target distribution of node u is either its fresh
// row, p(x) = exp(l(x) - m) / S, or a residual buffer r with p = r / Z.
// A rejection of a child proposed from q writes r'(x) = max(0, c(x) - Z q(x))
// (c = exp(l - m) or r, Z = S or the old Z) into the other buffer, which
// equals Z * max(0, p - q); Z' = sum r'.  If Z' = 0 the distribution is kept.
//
// Thread 0 makes every decision from LDS; each step that needs global data
// is one parallel round trip: at a node, all children's target logits and
// draft probabilities; after a residual pass, the children's new residuals.
// ---------------------------------------------------------------------------
struct MssArgs {
  int N, V, R;
  const float* logits;
  const float* ssm;
  const int32_t* q_row;
  const int32_t* token;
  const uint64_t* child;
  int32_t* status;
  uint64_t seed, offset;
  int32_t* accepted;
  int32_t* num_accepted;
  int32_t* bonus;
  int32_t* rounds;
  Stats st;
  float* resid;            // [B][2][V]
};

__device__ __forceinline__ double block_sum(double v, double* red) {
  v = tv::wave_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) s += red[w];
  return s;
}

// Inclusive scan within a wave (double).
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// The current distribution's unnormalised value at x.
__device__ __forceinline__ float cur_value(int mode, const float* lrow, float m, const float* src, int x) {
  if (mode == 0) {
    const float l = lrow[x];
    return l == -INFINITY ? 0.f : tv::exp_acc(l - m);
  }
  return src[x];
}

__global__ __launch_bounds__(kWalkThreads) void mss_walk_kernel(MssArgs a) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int N = a.N, V = a.V;
  const float* lbase = a.logits + static_cast<size_t>(b) * (N + 1) * V;
  const float* sbase = a.ssm + static_cast<size_t>(b) * a.R * V;
  float* rbuf0 = a.resid + static_cast<size_t>(b) * 2 * V;

  __shared__ ReqLds R;
  __shared__ uint64_t s_real;
  __shared__ int s_flag;
  __shared__ float lx_s[TV_MAX_NODES], qx_s[TV_MAX_NODES], rx_s[TV_MAX_NODES];
  __shared__ double red[kWalkThreads / 64];
  __shared__ int s_acc[TV_MAX_NODES];
  // walk state (written by thread 0 only, read by all after a barrier)
  __shared__ int s_status, s_action, s_u, s_mode, s_cur, s_qrow, s_slot, s_k, s_rounds, s_found;
  __shared__ uint64_t s_untested;
  __shared__ float s_m;
  __shared__ double s_Z, s_T;

  const int st0 = stage_request(R, b, N, V, a.R, a.token, a.q_row, a.child, a.st, true, a.status[b],
                                &s_real, &s_flag);
  if (t == 0) {
    s_status = st0;
    s_u = -1;
    s_slot = 0;
    s_k = 0;
    s_rounds = 0;
    s_mode = 0;
    s_cur = 0;
    s_action = 0;   // 0 = enter node
    if (st0 == TV_REQ_OK && !R.ok[0]) s_status = TV_REQ_NONFINITE;
    if (s_status == TV_REQ_OK) {
      s_m = R.m[0];
      s_Z = R.s[0];
      s_untested = R.child[0];
    }
  }
  __syncthreads();

  int j = 0;   // round at the current node (thread 0)
  while (s_status == TV_REQ_OK) {
    const int action = s_action;
    const int u = s_u;
    const int mode = s_mode, cb = s_cur;
    const float* lrow = lbase + static_cast<size_t>(u + 1) * V;
    const float mm = s_m;
    const double ZZ = s_Z;
    float* src = rbuf0 + static_cast<size_t>(cb) * V;

    if (action == 0) {
      // node entry: every child's target logit and draft probability at once
      const uint64_t kids = s_untested;
      if (t < N && ((kids >> t) & 1ull)) {
        const int x = R.tok[t];
        lx_s[t] = lrow[x];
        qx_s[t] = sbase[static_cast<size_t>(R.qrow[t]) * V + x];
      }
    } else if (action == 1) {
      // residual pass after rejecting a child proposed from row s_qrow
      const float* q = sbase + static_cast<size_t>(s_qrow) * V;
      float* dst = rbuf0 + static_cast<size_t>(cb ^ 1) * V;
      double acc = 0.0;
      int bad = 0;
      const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(q) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(lrow) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(src) & 15) == 0;
      if (vec) {
        for (int x4 = t; x4 < V / 4; x4 += kWalkThreads) {
          const float4 qv = reinterpret_cast<const float4*>(q)[x4];
          const float4 cv = mode == 0 ? reinterpret_cast<const float4*>(lrow)[x4]
                                      : reinterpret_cast<const float4*>(src)[x4];
          float c[4] = {cv.x, cv.y, cv.z, cv.w};
          const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (mode == 0) c[e] = c[e] == -INFINITY ? 0.f : tv::exp_acc(c[e] - mm);
            if (!(qq[e] >= 0.f) || qq[e] == INFINITY) bad = 1;
            r[e] = static_cast<float>(fmax(0.0, static_cast<double>(c[e]) - ZZ * static_cast<double>(qq[e])));
            acc += static_cast<double>(r[e]);
          }
          reinterpret_cast<float4*>(dst)[x4] = make_float4(r[0], r[1], r[2], r[3]);
        }
      } else {
        for (int x = t; x < V; x += kWalkThreads) {
          const float c = cur_value(mode, lrow, mm, src, x);
          const float qv = q[x];
          if (!(qv >= 0.f) || qv == INFINITY) bad = 1;
          const float r = static_cast<float>(fmax(0.0, static_cast<double>(c) - ZZ * static_cast<double>(qv)));
          dst[x] = r;
          acc += static_cast<double>(r);
        }
      }
      if (bad) atomicOr(&s_flag, 4);
      const double Znew = block_sum(acc, red);
      const int flag = s_flag;
      __syncthreads();
      const bool take = !(flag & 4) && Znew > 0.0;
      if (take) {
        // the remaining children's values under the new distribution
        const uint64_t kids = s_untested;
        if (t < N && ((kids >> t) & 1ull)) rx_s[t] = dst[R.tok[t]];
      }
      if (t == 0) {
        if (flag & 4) {
          s_status = TV_REQ_NONFINITE;
        } else if (take) {
          s_mode = 1;
          s_cur = cb ^ 1;
          s_Z = Znew;
        }
      }
    } else {
      // final sample: smallest x with cumsum >= u2 * total; thread t owns a
      // contiguous chunk, chunk sums are scanned across the workgroup
      const int chunk = (V + kWalkThreads - 1) / kWalkThreads;
      const int xa = min(V, t * chunk), xb = min(V, xa + chunk);
      double part = 0.0;
      for (int x = xa; x < xb; ++x) part += static_cast<double>(cur_value(mode, lrow, mm, src, x));
      const double wincl = wave_incl_scan(part);
      const int wave = t >> 6, lane = t & 63;
      if (lane == 63) red[wave] = wincl;
      __syncthreads();
      double wbase = 0.0, total = 0.0;
      for (int w2 = 0; w2 < kWalkThreads / 64; ++w2) {
        if (w2 < wave) wbase += red[w2];
        total += red[w2];
      }
      const double incl = wbase + wincl;
      // the previous thread's inclusive sum, bit for bit: the same wave base
      // plus its wave-scan value (lane 0: the base itself, which equals the
      // last lane of the previous wave summed in the same order)
      const double prev_w = __shfl_up(wincl, 1, 64);
      const double excl = lane > 0 ? wbase + prev_w : wbase;
      if (t == 0) {
        const tv::u32x4 w = tv::mss_words(a.seed, a.offset, b, s_slot, 0);
        s_T = tv::unit_open0(w.z) * total;
        s_found = -1;
      }
      __syncthreads();
      const double T = s_T;
      // exactly one owner: the first thread whose inclusive sum reaches T
      if (excl < T && incl >= T) {
        double accd = excl;
        int xs = -1, last_pos = -1;
        for (int x = xa; x < xb; ++x) {
          const float c = cur_value(mode, lrow, mm, src, x);
          if (c > 0.f) last_pos = x;
          accd += static_cast<double>(c);
          if (accd >= T) {
            xs = x;
            break;
          }
        }
        s_found = xs >= 0 ? xs : last_pos;   // rounding left the chunk short: last positive entry
      }
      __syncthreads();
      if (t == 0) {
        s_action = 3;   // done
      }
      __syncthreads();
      break;
    }
    __syncthreads();

    // ---- thread 0: ratio tests until a full-vocab pass is needed ----
    if (t == 0 && s_status == TV_REQ_OK) {
      int uu = s_u;
      uint64_t untested = s_untested;
      int md = s_mode;
      float m_ = s_m;
      double Z = s_Z;
      int k = s_k, rounds = s_rounds, slot = s_slot;
      int next = 2;     // default: final sample
      while (untested) {
        const tv::u32x4 w = tv::mss_words(a.seed, a.offset, b, slot, j);
        const int mcnt = __builtin_popcountll(untested);
        int idx = tv::pick_index(w.x, mcnt);
        uint64_t bits = untested;
        while (idx--) bits &= bits - 1;
        const int sidx = __builtin_ctzll(bits);
        const float qx = qx_s[sidx];
        if (!(qx >= 0.f) || qx == INFINITY) {
          s_status = TV_REQ_NONFINITE;
          next = -1;
          break;
        }
        double px;
        if (md == 0) {
          const float lx = lx_s[sidx];
          px = lx == -INFINITY ? 0.0 : exp(static_cast<double>(lx) - static_cast<double>(m_)) / Z;
        } else {
          px = static_cast<double>(rx_s[sidx]) / Z;
        }
        const double ratio = qx > 0.f ? px / static_cast<double>(qx) : (px > 0.0 ? INFINITY : 0.0);
        const double u1 = tv::unit_open0(w.y);
        ++rounds;
        if (u1 <= ratio) {
          s_acc[k++] = sidx;
          uu = sidx;
          slot = sidx + 1;
          j = 0;
          if (!R.ok[slot]) {
            s_status = TV_REQ_NONFINITE;
            next = -1;
            break;
          }
          s_m = R.m[slot];
          s_Z = R.s[slot];
          s_mode = 0;
          untested = R.child[slot];
          next = 0;     // enter the new node: fetch its children's values
          break;
        }
        untested &= ~(1ull << sidx);
        ++j;
        s_qrow = R.qrow[sidx];
        next = 1;
        break;
      }
      s_u = uu;
      s_untested = untested;
      s_k = k;
      s_rounds = rounds;
      s_slot = slot;
      s_flag = 0;
      if (next >= 0) s_action = next;
    }
    __syncthreads();
  }
  __syncthreads();
  if (t == 0) {
    const int stt = s_status;
    if (stt != TV_REQ_OK) {
      a.status[b] = stt;
      a.num_accepted[b] = -1;
      a.bonus[b] = -1;
      if (a.rounds) a.rounds[b] = -1;
      s_k = 0;
    } else {
      a.num_accepted[b] = s_k;
      a.bonus[b] = s_found;
      if (a.rounds) a.rounds[b] = s_rounds;
    }
  }
  __syncthreads();
  for (int i = t; i < N; i += kWalkThreads)
    a.accepted[static_cast<size_t>(b) * N + i] = i < s_k ? s_acc[i] : -1;
}

tv_status check_verify_args(int B, int N, int V) {
  if (B < 0 || N < 0 || V < 1 || V > (1 << 20)) return TV_EINVAL;
  if (N > TV_MAX_NODES) return TV_ETOOBIG;
  return TV_OK;
}

}  // namespace

extern "C" size_t tree_verify_workspace(int B, int N, int V) {
  if (check_verify_args(B, N, V) != TV_OK || B == 0) return 0;
  return ws_layout(B, N, V).total;
}

extern "C" tv_status tree_verify_greedy(int B, int N, int V, const float* target_logits,
                                        const int32_t* token, const uint64_t* child, int32_t* status,
                                        int32_t* accepted, int32_t* num_accepted, int32_t* bonus,
                                        void* workspace, size_t ws_bytes, hipStream_t stream) {
  const tv_status c = check_verify_args(B, N, V);
  if (c != TV_OK) return c;
  if (B == 0) return TV_OK;
  if (!target_logits || !child || !status || !num_accepted || !bonus ||
      (N > 0 && (!token || !accepted)))
    return TV_EINVAL;
  const WsLayout w = ws_layout(B, N, V);
  if (!workspace || ws_bytes < w.total) return TV_EWORKSPACE;
  const Stats st = stats_view(workspace, w, V);
  hipLaunchKernelGGL(row_stats_kernel<false>, dim3(B * (N + 1), st.P), dim3(kStatThreads), 0, stream,
                     target_logits, V, st);
  if (hipGetLastError() != hipSuccess) return TV_EHIP;
  hipLaunchKernelGGL(greedy_walk_kernel, dim3(B), dim3(64), 0, stream, N, V, token, child, status,
                     accepted, num_accepted, bonus, st);
  return tv::launch_status();
}

extern "C" tv_status tree_verify_mss(int B, int N, int V, int R, const float* target_logits,
                                     const float* ssm_probs, const int32_t* q_row, const int32_t* token,
                                     const uint64_t* child, int32_t* status, uint64_t seed,
                                     uint64_t offset, int32_t* accepted, int32_t* num_accepted,
                                     int32_t* bonus, int32_t* rounds, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  const tv_status c = check_verify_args(B, N, V);
  if (c != TV_OK) return c;
  if (R < 1) return TV_EINVAL;
  if (B == 0) return TV_OK;
  if (!target_logits || !ssm_probs || !child || !status || !num_accepted || !bonus ||
      (N > 0 && (!token || !accepted || !q_row)))
    return TV_EINVAL;
  const WsLayout w = ws_layout(B, N, V);
  if (!workspace || ws_bytes < w.total) return TV_EWORKSPACE;
  const Stats st = stats_view(workspace, w, V);
  hipLaunchKernelGGL(row_stats_kernel<true>, dim3(B * (N + 1), st.P), dim3(kStatThreads), 0, stream,
                     target_logits, V, st);
  if (hipGetLastError() != hipSuccess) return TV_EHIP;
  MssArgs a;
  a.N = N; a.V = V; a.R = R;
  a.logits = target_logits; a.ssm = ssm_probs; a.q_row = q_row; a.token = token; a.child = child;
  a.status = status; a.seed = seed; a.offset = offset;
  a.accepted = accepted; a.num_accepted = num_accepted; a.bonus = bonus; a.rounds = rounds;
  a.st = st;
  a.resid = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + w.off_res);
  hipLaunchKernelGGL(mss_walk_kernel, dim3(B), dim3(kWalkThreads), 0, stream, a);
  return tv::launch_status();
}
