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

// ---------------------------------------------------------------------------
// Phase 2a: greedy walk, one wave per request.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void greedy_walk_kernel(int N, int V, const int32_t* __restrict__ token,
                                                         const uint64_t* __restrict__ child,
                                                         int32_t* __restrict__ status,
                                                         int32_t* __restrict__ accepted,
                                                         int32_t* __restrict__ num_accepted,
                                                         int32_t* __restrict__ bonus, Stats st) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int32_t* tok = token + static_cast<size_t>(b) * N;
  if (i < N) accepted[static_cast<size_t>(b) * N + i] = -1;
  int stt = status[b];
  if (stt == TV_REQ_OK) {
    const int bad = __any(i < N && (tok[i] < 0 || tok[i] >= V));
    if (bad) stt = TV_REQ_BAD_TOKEN;
  }
  if (i != 0) return;
  int k = 0, bn = -1;
  if (stt == TV_REQ_OK) {
    int u = -1;
    while (true) {
      const RowStat r = merge_row(st, static_cast<size_t>(b) * (N + 1) + (u + 1), false);
      if (!r.ok) {
        stt = TV_REQ_NONFINITE;
        break;
      }
      const int o = r.arg;
      uint64_t kids = child[static_cast<size_t>(b) * (N + 1) + (u + 1)] & later_nodes(u, N);
      int nxt = -1;
      while (kids) {
        const int c = __builtin_ctzll(kids);
        kids &= kids - 1;
        if (tok[c] == o) {
          nxt = c;
          break;
        }
      }
      if (nxt < 0) {
        bn = o;
        break;
      }
      accepted[static_cast<size_t>(b) * N + k] = nxt;
      ++k;
      u = nxt;
    }
  }
  if (stt != TV_REQ_OK) {
    for (int j = 0; j < k; ++j) accepted[static_cast<size_t>(b) * N + j] = -1;
    status[b] = stt;
    num_accepted[b] = -1;
    bonus[b] = -1;
  } else {
    num_accepted[b] = k;
    bonus[b] = bn;
  }
}

// ---------------------------------------------------------------------------
// Phase 2b: multi-step speculative sampling, one 1024-thread workgroup per
// request.  The current target distribution of node u is either its fresh
// row, p(x) = exp(l(x) - m) / S, or a residual buffer r with p = r / Z.
// A rejection of a child proposed from q writes r'(x) = max(0, c(x) - Z q(x))
// (c = exp(l - m) or r, Z = S or the old Z) into the other buffer, which
// equals Z * max(0, p - q); Z' = sum r'.  If Z' = 0 the distribution is kept.
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

__device__ __forceinline__ double block_sum_1024(double v, double* red) {
  v = tv::wave_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kWalkThreads / 64; ++w) s += red[w];
  return s;
}

__global__ __launch_bounds__(kWalkThreads) void mss_walk_kernel(MssArgs a) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int N = a.N, V = a.V;
  const int32_t* tok = a.token + static_cast<size_t>(b) * N;
  const int32_t* qr = a.q_row + static_cast<size_t>(b) * N;
  const float* lbase = a.logits + static_cast<size_t>(b) * (N + 1) * V;
  const float* sbase = a.ssm + static_cast<size_t>(b) * a.R * V;
  float* rbuf[2] = {a.resid + static_cast<size_t>(b) * 2 * V, a.resid + (static_cast<size_t>(b) * 2 + 1) * V};

  __shared__ int s_status, s_done, s_action, s_mode, s_cur, s_row, s_qrow, s_k, s_rounds, s_bonus;
  __shared__ float s_m;
  __shared__ double s_Z, s_T;
  __shared__ double red[kWalkThreads / 64];
  __shared__ int s_acc[TV_MAX_NODES];
  __shared__ int s_flag, s_found;
  __shared__ double s_excl[kWalkThreads];

  if (t == 0) {
    s_status = a.status[b];
    s_flag = 0;
  }
  __syncthreads();
  if (s_status == TV_REQ_OK) {
    int bt_ = 0, bq = 0;
    if (t < N) {
      bt_ = tok[t] < 0 || tok[t] >= V;
      bq = qr[t] < 0 || qr[t] >= a.R;
    }
    if (bt_) atomicOr(&s_flag, 1);
    if (bq) atomicOr(&s_flag, 2);
  }
  __syncthreads();
  if (t == 0 && s_status == TV_REQ_OK) {
    if (s_flag & 1) s_status = TV_REQ_BAD_TOKEN;
    else if (s_flag & 2) s_status = TV_REQ_BAD_QROW;
  }

  // control state lives in thread 0's registers; shared copies drive passes
  int u = -1, slot = 0, j = 0, k = 0, rounds = 0, mode = 0, cur = 0;
  uint64_t untested = 0;
  float m = 0.f;
  double Z = 0.0;
  if (t == 0) {
    s_done = s_status != TV_REQ_OK;
    if (!s_done) {
      const RowStat r = merge_row(a.st, static_cast<size_t>(b) * (N + 1), true);
      if (!r.ok) {
        s_status = TV_REQ_NONFINITE;
        s_done = 1;
      } else {
        m = r.m;
        Z = r.s;
        untested = a.child[static_cast<size_t>(b) * (N + 1)] & later_nodes(-1, N);
      }
    }
  }
  __syncthreads();

  while (!s_done) {
    // ---- thread 0: ratio tests until a full-vocab pass is needed ----
    if (t == 0) {
      s_action = 0;  // 1 = residual pass, 2 = final sample
      while (true) {
        if (!untested) {
          s_action = 2;
          break;
        }
        const tv::u32x4 w = tv::mss_words(a.seed, a.offset, b, slot, j);
        const int mcnt = __builtin_popcountll(untested);
        int idx = tv::pick_index(w.x, mcnt);
        uint64_t bits = untested;
        while (idx--) bits &= bits - 1;
        const int sidx = __builtin_ctzll(bits);
        const int x = tok[sidx];
        const float qx = sbase[static_cast<size_t>(qr[sidx]) * V + x];
        if (!(qx >= 0.f) || qx == INFINITY) {
          s_status = TV_REQ_NONFINITE;
          s_action = 3;
          break;
        }
        double px;
        if (mode == 0) {
          const float lx = lbase[static_cast<size_t>(u + 1) * V + x];
          px = lx == -INFINITY ? 0.0 : exp(static_cast<double>(lx) - static_cast<double>(m)) / Z;
        } else {
          px = static_cast<double>(rbuf[cur][x]) / Z;
        }
        const double ratio = qx > 0.f ? px / static_cast<double>(qx) : (px > 0.0 ? INFINITY : 0.0);
        const double u1 = tv::unit_open0(w.y);
        ++rounds;
        if (u1 <= ratio) {
          if (k < TV_MAX_NODES) s_acc[k] = sidx;
          ++k;
          u = sidx;
          slot = sidx + 1;
          j = 0;
          const RowStat r = merge_row(a.st, static_cast<size_t>(b) * (N + 1) + slot, true);
          if (!r.ok) {
            s_status = TV_REQ_NONFINITE;
            s_action = 3;
            break;
          }
          m = r.m;
          Z = r.s;
          mode = 0;
          untested = a.child[static_cast<size_t>(b) * (N + 1) + slot] & later_nodes(u, N);
          continue;
        }
        // rejection: residual pass over the full vocabulary
        untested &= ~(1ull << sidx);
        ++j;
        s_qrow = qr[sidx];
        s_action = 1;
        break;
      }
      s_mode = mode;
      s_cur = cur;
      s_row = u + 1;
      s_m = m;
      s_Z = Z;
      s_flag = 0;
    }
    __syncthreads();
    const int action = s_action;
    if (action == 3) break;
    const int md = s_mode, cb = s_cur;
    const float* lrow = lbase + static_cast<size_t>(s_row) * V;
    const float mm = s_m;
    const double ZZ = s_Z;
    if (action == 1) {
      const float* q = sbase + static_cast<size_t>(s_qrow) * V;
      const float* src = rbuf[cb];
      float* dst = rbuf[cb ^ 1];
      double acc = 0.0;
      int bad = 0;
      for (int x = t; x < V; x += kWalkThreads) {
        const float c = md == 0 ? (lrow[x] == -INFINITY ? 0.f : tv::exp_acc(lrow[x] - mm)) : src[x];
        const float qv = q[x];
        if (!(qv >= 0.f) || qv == INFINITY) bad = 1;
        const double r = fmax(0.0, static_cast<double>(c) - ZZ * static_cast<double>(qv));
        const float rf = static_cast<float>(r);
        dst[x] = rf;
        acc += static_cast<double>(rf);
      }
      if (bad) atomicOr(&s_flag, 1);
      const double Znew = block_sum_1024(acc, red);
      if (t == 0) {
        if (s_flag) {
          s_status = TV_REQ_NONFINITE;
          s_done = 1;
        } else if (Znew > 0.0) {
          mode = 1;
          cur ^= 1;
          Z = Znew;
        }
        // Znew == 0: keep the current distribution (zero-normaliser guard)
      }
      __syncthreads();
      continue;
    }
    // ---- action 2: final sample, smallest x with cumsum >= u2 * total ----
    const int chunk = (V + kWalkThreads - 1) / kWalkThreads;
    const int xa = min(V, t * chunk), xb = min(V, xa + chunk);
    const float* src = rbuf[cb];
    double part = 0.0;
    for (int x = xa; x < xb; ++x) {
      const float c = md == 0 ? (lrow[x] == -INFINITY ? 0.f : tv::exp_acc(lrow[x] - mm)) : src[x];
      part += static_cast<double>(c);
    }
    // exclusive scan of the per-thread sums
    s_excl[t] = part;
    __syncthreads();
    for (int o = 1; o < kWalkThreads; o <<= 1) {
      const double add = t >= o ? s_excl[t - o] : 0.0;
      __syncthreads();
      s_excl[t] += add;
      __syncthreads();
    }
    const double incl = s_excl[t];
    const double excl = t > 0 ? s_excl[t - 1] : 0.0;   // the previous thread's inclusive sum
    if (t == 0) {
      const tv::u32x4 w = tv::mss_words(a.seed, a.offset, b, slot, 0);
      s_T = tv::unit_open0(w.z) * s_excl[kWalkThreads - 1];
      s_found = -1;
    }
    __syncthreads();
    const double T = s_T;
    // exactly one thread has excl < T <= incl (sums are non-negative)
    if (excl < T && incl >= T) {
      double accd = excl;
      int xs = -1, last_pos = -1;
      for (int x = xa; x < xb; ++x) {
        const float c = md == 0 ? (lrow[x] == -INFINITY ? 0.f : tv::exp_acc(lrow[x] - mm)) : src[x];
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
      s_bonus = s_found;
      s_done = 1;
    }
    __syncthreads();
    break;
  }
  __syncthreads();
  if (t == 0) {
    const int stt = s_status;
    int32_t* acc = a.accepted + static_cast<size_t>(b) * N;
    if (stt != TV_REQ_OK) {
      a.status[b] = stt;
      a.num_accepted[b] = -1;
      a.bonus[b] = -1;
      if (a.rounds) a.rounds[b] = -1;
    } else {
      a.num_accepted[b] = k;
      a.bonus[b] = s_bonus;
      if (a.rounds) a.rounds[b] = rounds;
    }
    s_k = stt == TV_REQ_OK ? k : 0;
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
