// tree_verify_greedy / tree_verify_mss: verification of a token tree.
//
// SpecInfer summary, "Token Verification: Greedy Decoding (VerifyGreedy)" and
// "Token Verification: Stochastic Decoding and Multi-Step Speculative
// Sampling (VerifyStochastic)"; the leaf bonus token and the zero-normaliser
// guard follow the wiki concept page "Speculative decoding", "Implementation
// sketch".
//
// Work decomposition.  The walk over a request's tree is sequential, but each
// of its steps touches a whole vocabulary row (32K-50K floats): the target
// statistics of the node reached, the residual after a rejection, the final
// inverse-CDF sample.  One request therefore gets G = ceil(V / (256 E))
// workgroups that run at the same time (E = 4, 8 or 16 entries per thread,
// chosen per launch); workgroup g owns the vocabulary slice
// [256 E g, 256 E (g + 1)) and keeps its slice of the current distribution in
// registers.  Every workgroup of a request makes the same decisions (random
// child, ratio test) from the same data, so only a few scalars per step cross
// workgroups: slice max / sum / argmax when a node is entered, slice residual
// mass and the residual at the remaining children's tokens after a
// rejection.  The final sample needs no exchange: the slice totals of the
// current distribution are already known everywhere, so every workgroup can
// tell which slice holds the inverse-CDF threshold, and that slice's
// workgroup finishes the search alone.
//
// Latency, not bandwidth, bounds a walk (a handful of 128 KB rows per
// request), so each pass issues its loads as early as their addresses are
// known: the root row at kernel start, and in every MSS pass the logits row
// and draft row of the child tested after the pass (the random choice of that
// child does not depend on the test's outcome).
//
// Exchange protocol.  Each exchanged value is one 64-bit word whose high half
// is a tag (the exchange's number + 1) and whose low half is the data; the
// word is written and read with device-scope atomics, which stay coherent
// across the per-XCD L2 caches without cache-wide fences.  A reader polls a
// word until it carries the tag it expects, so one store and one load are
// the whole cost of an exchange.  Words alternate between two banks by the
// parity of the exchange number: a workgroup can only reach exchange n + 2
// after every workgroup has published exchange n + 1, which each does only
// after it has finished reading exchange n, so bank reuse never overwrites a
// word that is still to be read.  The last workgroup to leave zeroes the
// words, so every call starts from a zeroed workspace.
#include "kv_move.h"

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>

namespace {

constexpr int kOwnThreads = 256;                   // threads that own vocabulary entries
constexpr int kCoThreads = kOwnThreads + 64;       // threads per workgroup: the owners and the poll wave
constexpr int kPollWave = kOwnThreads / 64;        // stages the request and polls the exchanges
constexpr int kMaxG = 512;                         // workgroups per request (LDS arrays)
constexpr int kHdr = 4;                            // header words per workgroup per exchange
constexpr unsigned kSpinLimit = 1u << 22;          // polls of one word before giving up

enum : int { FLAG_NAN = 1, FLAG_PINF = 2, FLAG_FINITE = 4 };
enum : int { MODE_GREEDY = 0, MODE_MSS = 1, MODE_NAIVE = 2 };
enum : int { P_ENTER = 0, P_RESID = 1, P_NSAMPLE = 2, P_FINAL = 3, P_DONE = 4 };   // passes of the walk

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// Workspace, per request (all zero between calls):
//   done [B][64] uint32            workgroups that have left (one 256-byte line)
//   hdr  [B][2][G][kHdr] uint64    tagged header words, bank = exchange parity
//   kid  [B][2][64] uint64         tagged residual value at child c's token,
//                                  written by the workgroup owning that token
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t off_hdr, off_kid, total;
};

// Vocabulary entries per owner thread of the sliced MSS and naive walks (E =
// 4, 8 or 16; greedy keeps 8) are chosen per launch in launch_walk: the
// smallest E that puts every workgroup of the call on a compute unit of its
// own, else the E that needs the fewest launches (ties: the larger E, fewer
// workgroups per CU).  Two workgroups of a walk sharing a CU slow every pass
// of their requests at least as much as twice the entries per thread do, and
// fewer entries per thread shorten each pass.  G = slice_groups(V, E) <=
// kMaxG is required (V <= 2^20 keeps E = 16 at most 256 workgroups per
// request).
int slice_groups(int V, int E) { return (V + kOwnThreads * E - 1) / (kOwnThreads * E); }

// Workgroups per request the workspace is laid out for: the most any choice
// above can give.
int ws_groups(int V) {
  for (int E = 4; E <= 16; E *= 2)
    if (slice_groups(V, E) <= kMaxG) return slice_groups(V, E);
  return slice_groups(V, 16);
}

WsLayout ws_layout(int B, int V) {
  const size_t G = static_cast<size_t>(ws_groups(V));
  WsLayout w;
  w.off_hdr = align256(static_cast<size_t>(B) * 64 * sizeof(uint32_t));
  w.off_kid = w.off_hdr + align256(static_cast<size_t>(B) * 2 * G * kHdr * sizeof(uint64_t));
  w.total = w.off_kid + align256(static_cast<size_t>(B) * 2 * 64 * sizeof(uint64_t));
  return w;
}

struct WalkArgs {
  int mode;
  int N, V, R, G;
  int b0;                   // first request of this launch
  const float* logits;      // [B][N+1][V]
  const float* ssm;         // [B][R][V]
  const int32_t* q_row;     // [B][N]
  const int32_t* token;     // [B][N]
  const uint64_t* child;    // [B][N+1]
  int32_t* status;
  uint64_t seed, offset;
  int32_t* accepted;
  int32_t* num_accepted;
  int32_t* bonus;
  int32_t* rounds;
  uint32_t* done;            // [B][64]: word 0 counts the workgroups that left; words 2-3 hold
                            // MSS's sampled token, tagged, from the slice that found it;
                            // with the commit, words 4-5 workgroup 0's tagged decision to
                            // move and word 6 the other workgroups' reports
  uint64_t* hdr;
  uint64_t* kid;
  bool commit;              // MSS: also compact the accepted path in the KV cache
  tv::KvRef kv;             //   the cache, block table and prefix lengths
  bool multi;               // MSS over proposals (several per node):
  int S;                    //   slots per request
  const int32_t* prop_node; //   [B][S] node of each proposal, -1 = unused slot
  const int32_t* prop_row;  //   [B][S] its proposer's row of ssm
  unsigned spin_limit;      // polls of one exchanged word before a wait gives up
};
constexpr int kMoveChunks = 8;                     // 16-byte chunks per thread per batch of the move

// device-scope relaxed atomics: coherent across XCDs without L2 flushes
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_u64(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t tag, uint32_t v) {
  st_u64(p, (static_cast<uint64_t>(tag) << 32) | v);
}

// Poll n consecutive tagged words until all carry `tag`; their data go to
// out[0..n).  Returns false when `limit` polls did not see it.
template <int n>
__device__ __forceinline__ bool take_tagged(uint64_t* p, uint32_t tag, uint32_t (&out)[kHdr], unsigned limit) {
  for (unsigned polls = 0; polls < limit; ++polls) {
    uint64_t x[n];
#pragma unroll
    for (int i = 0; i < n; ++i) x[i] = ld_u64(p + i);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < n; ++i) ok = ok && static_cast<uint32_t>(x[i] >> 32) == tag;
    if (ok) {
#pragma unroll
      for (int i = 0; i < n; ++i) out[i] = static_cast<uint32_t>(x[i]);
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

__device__ __forceinline__ uint32_t lo32(double d) {
  return static_cast<uint32_t>(static_cast<uint64_t>(__double_as_longlong(d)));
}
__device__ __forceinline__ uint32_t hi32(double d) {
  return static_cast<uint32_t>(static_cast<uint64_t>(__double_as_longlong(d)) >> 32);
}
__device__ __forceinline__ double join64(uint32_t lo, uint32_t hi) {
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Children of u can only be nodes u+1 .. N-1 (parents precede children).
// Masking with this keeps every walk finite and in bounds even for child
// masks that did not come from tree_build_mask.
__device__ __forceinline__ uint64_t later_nodes(int u, int N) {
  const uint64_t below_n = N >= 64 ? ~0ull : ((1ull << N) - 1);
  const uint64_t upto_u = u < 0 ? 0ull : (u >= 63 ? ~0ull : ((2ull << u) - 1));
  return below_n & ~upto_u;
}

// Index of the i-th set bit of m (i < popcount(m)).
__device__ __forceinline__ int nth_bit(uint64_t m, int i) {
  while (i--) m &= m - 1;
  return __builtin_ctzll(m);
}

__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(tv::wave_or_dpp(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(tv::wave_or_dpp(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sum of a double and OR of an int over the workgroup with one barrier.  The
// per-wave partials go to one of two banks; callers alternate banks, so a
// call never overwrites partials that a wave may still be reading from the
// previous call (every wave has left that call before it can pass this
// call's barrier).
__device__ __forceinline__ double block_sum_or(double v, int f, double (*red)[kCoThreads / 64],
                                               int (*redf)[kCoThreads / 64], int bank, int* f_out) {
  v = tv::wave_sum_dpp(v);
  f = tv::wave_or_dpp(f);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[bank][wave] = v;
    redf[bank][wave] = f;
  }
  __syncthreads();
  double s = 0.0;
  int o = 0;
#pragma unroll
  for (int w = 0; w < kCoThreads / 64; ++w) {
    s += red[bank][w];
    o |= redf[bank][w];
  }
  *f_out = o;
  return s;
}

__device__ __forceinline__ bool q_bad(float q) { return !(q >= 0.f) || q == INFINITY; }

// ---------------------------------------------------------------------------
// Staging of a walk over proposals (MSS on merged trees), one wave: lane s is
// proposal slot s and, as in the one-proposal staging, lane i is node i with
// child mask cm and token tok.  A slot's node must be a node of the tree
// (some node's child: `real`) and its row in [0, R); *bad is the ballot of
// the used slots that are not.  child_slots of lane u + 1 is the mask of the
// slots whose node is a child of u, so the walk picks among proposals
// exactly as it picks among children when every node has one proposal.
struct SlotStage {
  uint64_t child_slots;
  int node, tok, row;       // this lane's slot (node -1: unused or invalid)
};
__device__ SlotStage stage_slots(const WalkArgs& a, int b, int N, uint64_t cm, int tok, uint64_t real,
                                 uint64_t* bad) {
  const int lane = threadIdx.x & 63;
  const size_t rb = static_cast<size_t>(b);
  const int pn = lane < a.S ? a.prop_node[rb * a.S + lane] : -1;
  const int pr = lane < a.S ? a.prop_row[rb * a.S + lane] : 0;
  const bool node_ok = pn >= 0 && pn < N && ((real >> (pn & 63)) & 1ull);
  *bad = __ballot(lane < a.S && pn != -1 && (!node_ok || pr < 0 || pr >= a.R));
  SlotStage r;
  r.node = node_ok ? pn : -1;
  r.tok = __shfl(tok, node_ok ? pn : 0, 64);
  r.row = node_ok ? pr : 0;
  r.child_slots = 0ull;
  const int last = min(N, 63);          // node 63 has no children
  for (int uu = 0; uu <= last; ++uu) {
    const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(static_cast<uint32_t>(cm)), uu, 64));
    const uint32_t hi = static_cast<uint32_t>(__shfl(static_cast<int>(static_cast<uint32_t>(cm >> 32)), uu, 64));
    const uint64_t cmu = (static_cast<uint64_t>(hi) << 32) | lo;
    const uint64_t m = __ballot(node_ok && ((cmu >> (pn & 63)) & 1ull));
    if (lane == uu) r.child_slots = m;
  }
  return r;
}

// ---------------------------------------------------------------------------
// The walk kernel.  grid = (requests in this launch) * G, block = 256.
//
// Every wave of every workgroup of a request reads the same exchanged words
// and makes the same decisions from them with the same operations, so the
// walk state lives in registers and a pass needs no barrier beyond those of
// its workgroup reductions.
// ---------------------------------------------------------------------------
template <int MODE, bool VEC, bool COMMIT, bool MULTI, int E>
__global__ __launch_bounds__(kCoThreads) void walk_kernel(WalkArgs a) {
  constexpr int kElem = E;                           // vocabulary entries per owner thread
  constexpr int kSlice = kOwnThreads * kElem;        // entries per workgroup
  constexpr int NW = kCoThreads / 64;
  const int G = a.G;
  const int b = a.b0 + static_cast<int>(blockIdx.x) / G;
  const int g = static_cast<int>(blockIdx.x) % G;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int N = a.N, V = a.V;
  constexpr bool mss = MODE == MODE_MSS, naive = MODE == MODE_NAIVE;
  constexpr bool need_z = mss || naive;               // the walk needs the normaliser
  const int xa = g * kSlice + t * kElem;              // first entry of this thread
  const int nx = t < kOwnThreads ? max(0, min(kElem, V - xa)) : 0;   // entries it owns
  const float* lbase = a.logits + static_cast<size_t>(b) * (N + 1) * V;
  const float* sbase = mss ? a.ssm + static_cast<size_t>(b) * a.R * V : nullptr;
  uint32_t* done = a.done + static_cast<size_t>(b) * 64;
  uint64_t* hdr = a.hdr + static_cast<size_t>(b) * 2 * G * kHdr;
  uint64_t* kid = a.kid + static_cast<size_t>(b) * 2 * 64;

  // per child (per proposal slot when MULTI): token and draft row; s_child[u + 1]
  // the children (proposals) of u; s_node the slot's node (MULTI)
  __shared__ int s_tok[TV_MAX_NODES], s_qrow[TV_MAX_NODES], s_acc[TV_MAX_NODES], s_node[TV_MAX_NODES];
  __shared__ uint64_t s_child[TV_MAX_NODES + 1];
  __shared__ double s_red[2][NW];
  __shared__ int s_redf[2][NW];
  __shared__ float s_wm[2][NW];                  // per-wave max / argmax / flags, two banks
  __shared__ int s_wa[2][NW], s_wf[2][NW];
  // gathered slice values, two banks by exchange parity (wave 0 writes them)
  __shared__ float s_gm[2][kMaxG];
  __shared__ double s_gs[2][kMaxG];
  __shared__ int s_ga[2][kMaxG];
  __shared__ float s_rx2[2][TV_MAX_NODES];
  __shared__ float s_lxq[2][2];                  // MSS: p and q at the candidate's token, from wave 0
  __shared__ uint32_t s_spec[2][2][8];           // the next pass's words and candidate per outcome, from wave 0
  __shared__ double s_gt[NW][kMaxG];             // slice totals of the current distribution (per wave)
  __shared__ double s_scan[NW];
  __shared__ int s_status0, s_timeout, s_found, s_last, s_xs;
  __shared__ int s_dec, s_acks;                  // COMMIT: workgroup 0's decision / the others' reports
  __shared__ int s_L;                            // COMMIT: the request's prefix length
  __shared__ tv::CommitLds s_mv;                 // COMMIT: the move's block offsets
  __shared__ int s_tblk[tv::kMaxTreeBlocks];     // COMMIT: block ids covering the tree's slots
  __shared__ float own_s[kElem];

  static_assert(kElem % 4 == 0, "entries per thread");
  // VEC (V a multiple of 4, rows 16-byte aligned): a thread owns a multiple
  // of 4 entries (up to kElem) and loads them as float4s.  The choice is made at compile time: a
  // run-time choice leaves both paths writing the same registers, and the
  // compiler then drains every load in flight before the float4 ones.
  // Entries past the vocabulary (and all of the poll wave's) get a neutral
  // value, so the passes over a row need no bounds tests: -inf for logits
  // (never a max, no mass) and 0 for draft rows (a zero residual).
  auto load8 = [&](const float* row, float (&dst)[kElem], float pad) {
    if constexpr (VEC) {
#pragma unroll
      for (int e = 0; e < kElem; e += 4) {
        float4 f = make_float4(pad, pad, pad, pad);
        if (e < nx) f = *reinterpret_cast<const float4*>(row + xa + e);
        dst[e] = f.x; dst[e + 1] = f.y; dst[e + 2] = f.z; dst[e + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kElem; ++k) dst[k] = k < nx ? row[xa + k] : pad;
    }
  };

  // ---------------- issue the first loads, stage the request ----------------
  float lv[kElem];         // logits of the current node's row, this thread's entries
  load8(lbase, lv, -INFINITY);   // the root row is always visited
  if (wave == kPollWave) {
    const size_t rb = static_cast<size_t>(b);
    const int st0 = lane == 0 ? a.status[b] : 0;
    // child[N] (children of the last node) is empty after masking
    const uint64_t cm = lane < N ? a.child[rb * (N + 1) + lane] & later_nodes(lane - 1, N) : 0ull;
    const int tok = lane < N ? a.token[rb * N + lane] : 0;
    const int qr = (mss && !MULTI && lane < N) ? a.q_row[rb * N + lane] : 0;
    const uint64_t real = wave_or64(cm);     // padding slots are nobody's child: unchecked
    const uint64_t bad_tok = __ballot(lane < N && (tok < 0 || tok >= V));
    uint64_t bad_q = __ballot(mss && !MULTI && lane < N && (qr < 0 || qr >= a.R)) & real;
    if constexpr (MULTI) {
      const SlotStage ss = stage_slots(a, b, N, cm, tok, real, &bad_q);
      s_child[lane] = ss.child_slots;
      s_tok[lane] = ss.tok;
      s_qrow[lane] = ss.row;
      s_node[lane] = ss.node;
    } else {
      s_child[lane] = cm;
      s_tok[lane] = tok;
      s_qrow[lane] = qr;
    }
    if (lane == 0) {
      s_child[TV_MAX_NODES] = 0ull;
      int st = st0;
      if (st == TV_REQ_OK) {
        if (bad_tok & real) st = TV_REQ_BAD_TOKEN;
        else if (bad_q) st = TV_REQ_BAD_QROW;
      }
      s_status0 = st;
      s_timeout = 0;
      // nothing writes the prefix length before the move at the end
      // nothing writes the prefix length before every workgroup has moved its heads
      if constexpr (COMMIT) s_L = a.kv.prefix_len[b];
    }
  }
  __syncthreads();

  // COMMIT: the poll wave fetches the block ids of the tree's slots now; the
  // loads land long before its first poll waits (in issue order) for anything
  int tblk = 0;
  if constexpr (COMMIT)
    if (wave == kPollWave && lane < tv::kMaxTreeBlocks) tblk = tv::tree_block_id(a.kv, b, N, s_L, lane);

  // ---- walk state: registers, identical in every thread of the request ----
  int status = s_status0;
  int pass = P_ENTER, u = -1, j = 0, k = 0, rounds = 0, mode = 0, bonus = -1;
  uint64_t U = s_child[0];
  float m = 0.f;           // max of the current node's row
  double Z = 1.0;          // normaliser of the current distribution
  float rx = 0.f;          // lane c: the residual at child c's token (mode 1)
  int owner = -1;          // final sample: the slice holding the threshold
  double Tloc = 0.0;       //   and the threshold inside it
  bool timed_out = false;  // wave-uniform

  float cv[kElem], rn[kElem];   // residual in use / residual of this pass
  float qv[kElem], qn[kElem];   // draft row of the rejected child / of the next candidate
  float lvn[kElem];             // logits row of the next candidate
#pragma unroll
  for (int e = 0; e < kElem; ++e) cv[e] = rn[e] = qv[e] = qn[e] = lvn[e] = 0.f;

  int ex_no = 0;                // exchanges done
  int rs_no = 0;                // workgroup sums done (bank parity)
  int pre = 0;                  // greedy/naive: the entered node's row is in lvn (1), qn (2), or not loaded (0)
  int c1 = -1, c2 = -1;         // greedy/naive: the children whose rows are prefetched

  // MSS: the next pass's Philox words and candidate (node, token, draft row),
  // worked out during the previous exchange for both outcomes of its test;
  // absent before the first test.  zdraw: the word of the final draw at u.
  bool have_next = false;
  tv::u32x4 w_next{0u, 0u, 0u, 0u};
  int c_next = -1, node_next = -1, tok_next = 0, qr_next = 0;
  uint32_t zdraw = 0u;

  // The slice holding u2 * total, from the slice totals in index order, and
  // the threshold inside it (every wave, same values).
  auto locate = [&](uint32_t word) {
    double run = 0.0;
    for (int base = 0; base < G; base += 64) {     // the same sums as the search below
      const double v = base + lane < G ? s_gt[wave][base + lane] : 0.0;
      double ex;
      run = tv::readlane_f64(run + tv::wave_scan_dpp(v, &ex), 63);
    }
    const double T = tv::unit_open0(word) * run;
    double carry = 0.0, ex_owner = 0.0, ex_last = 0.0;
    int last = -1;
    owner = -1;
    for (int base = 0; base < G && owner < 0; base += 64) {
      const double v = base + lane < G ? s_gt[wave][base + lane] : 0.0;
      double excl;
      const double incl = carry + tv::wave_scan_dpp(v, &excl);
      excl += carry;
      const uint64_t hit = __ballot(v > 0.0 && excl < T && incl >= T);
      const uint64_t pos = __ballot(v > 0.0);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        owner = base + l;
        ex_owner = tv::readlane_f64(excl, l);
      } else if (pos) {
        const int l = 63 - __builtin_clzll(pos);
        last = base + l;
        ex_last = tv::readlane_f64(excl, l);
      }
      carry = tv::readlane_f64(incl, 63);
    }
    if (owner < 0) {       // rounding left the total short: last non-empty slice
      owner = last;
      ex_owner = ex_last;
    }
    Tloc = fmax(T - ex_owner, 1e-300);
  };

  // The owner slice's workgroup finds the sampled token (all its threads
  // call this; every thread gets the token).
  auto slice_search = [&]() -> int {
    float (&cur)[kElem] = rn;          // the residual array is free during a draw
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < kElem; ++e) {
      cur[e] = mode == 0 ? (lv[e] == -INFINITY ? 0.f : tv::exp_acc(lv[e] - m)) : cv[e];   // padding: 0
      part += static_cast<double>(cur[e]);
    }
    double wexcl;
    const double wincl = tv::wave_scan_dpp(part, &wexcl);
    if (lane == 63) s_scan[wave] = wincl;
    if (t == 0) s_found = -1;
    __syncthreads();
    double wbase = 0.0, total = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      if (w2 < wave) wbase += s_scan[w2];
      total += s_scan[w2];
    }
    const double incl = wbase + wincl;
    const double excl = wbase + wexcl;     // the previous thread's incl, bit for bit (wexcl = 0 in lane 0)
    // threshold in (0, slice total]: exactly one thread has excl < T <= incl
    const double T = fmin(Tloc, total);
    if (excl < T && incl >= T) {
#pragma unroll
      for (int e = 0; e < kElem; ++e) own_s[e] = cur[e];
      double accd = excl;
      int xs = -1, last_pos = -1;
      for (int e = 0; e < nx; ++e) {
        const float c = own_s[e];
        if (c > 0.f) last_pos = xa + e;
        accd += static_cast<double>(c);
        if (accd >= T) {
          xs = xa + e;
          break;
        }
      }
      s_found = xs >= 0 ? xs : last_pos;   // rounding left the chunk short: last positive entry
    }
    __syncthreads();
    return s_found;
  };

  for (;;) {
    if (status != TV_REQ_OK || pass >= P_FINAL || timed_out) break;
    if (naive && pass == P_NSAMPLE) {
      // ---- naive: the owner slice draws the token, every workgroup takes it ----
      const uint32_t tag = static_cast<uint32_t>(ex_no + 1);
      const int par = ex_no & 1;
      if (g == owner) {
        const int x = slice_search();
        if (t == 0) put_tagged(kid + par * 64, tag, static_cast<uint32_t>(x));
      }
      if (wave == kPollWave) {
        bool to = false;
        if (lane == 0) {
          uint32_t v[kHdr] = {0u, 0u, 0u, 0u};
          if (!take_tagged<1>(kid + par * 64, tag, v, a.spin_limit)) to = true;
          s_xs = static_cast<int>(v[0]);
        }
        if (__any(to) && lane == 0) s_timeout = 1;
      }
      __syncthreads();
      ++ex_no;
      if (s_timeout) {
        timed_out = true;
        break;
      }
      const int x = s_xs;
      const uint64_t hit = __ballot(lane < N && ((U >> lane) & 1ull) && s_tok[lane] == x);
      if (!hit) {
        bonus = x;
        pass = P_DONE;
        continue;
      }
      const int nxt = __builtin_ctzll(hit);
      if (t == 0) s_acc[k] = nxt;
      ++k;
      u = nxt;
      U = s_child[nxt + 1];
      pre = nxt == c1 ? 1 : (nxt == c2 ? 2 : 0);
      pass = P_ENTER;
      continue;
    }
    if (pass == P_RESID) {
#pragma unroll
      for (int e = 0; e < kElem; ++e) qv[e] = qn[e];
    }
    const float* lrow = lbase + static_cast<size_t>(u + 1) * V;
    if (pass == P_ENTER && u >= 0) {
      if (mss || pre == 1) {
#pragma unroll
        for (int e = 0; e < kElem; ++e) lv[e] = lvn[e];
      } else if (pre == 2) {
#pragma unroll
        for (int e = 0; e < kElem; ++e) lv[e] = qn[e];
      } else {
        load8(lrow, lv, -INFINITY);
      }
    }
    // Every load issued so far is complete here: the rows just moved were
    // requested a pass ago, and the root row or a row loaded just above is
    // needed now anyway.  Waiting before the next candidates' rows are
    // requested matters: otherwise the compiler makes this pass's arithmetic
    // wait for those loads too (it cannot tell them apart across the loop),
    // and each pass pays a whole memory round trip the prefetch was meant
    // to hide.
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));    // vmcnt(0)
    // greedy/naive: the rows of the first two children, in case the walk enters one
    if (!mss && pass == P_ENTER) c1 = c2 = -1;
    if (!mss && pass == P_ENTER && U) {
      c1 = __builtin_ctzll(U);
      load8(lbase + static_cast<size_t>(c1 + 1) * V, lvn, -INFINITY);
      const uint64_t rest = U & (U - 1);
      if (rest) {
        c2 = __builtin_ctzll(rest);
        load8(lbase + static_cast<size_t>(c2 + 1) * V, qn, -INFINITY);
      }
    }
    // the child tested after this pass, and its rows (loads in flight during the pass)
    int cand = -1;
    tv::u32x4 w{0u, 0u, 0u, 0u};
    float lx_c = 0.f, qx_c = 0.f;
    if (mss && (U || pass == P_ENTER)) {
      // the word of round j at u (a P_ENTER pass is round 0, whose third
      // word also serves the final draw at u)
      w = have_next ? w_next : tv::mss_words(a.seed, a.offset, b, u + 1, j);
      if (pass == P_ENTER) zdraw = w.z;
    }
    if (mss && U) {
      int node_c, tok_c, qr_c;
      if (have_next) {
        cand = c_next;
        node_c = node_next;
        tok_c = tok_next;
        qr_c = qr_next;
      } else {
        cand = nth_bit(U, tv::pick_index(w.x, __builtin_popcountll(U)));
        node_c = MULTI ? s_node[cand] : cand;
        tok_c = s_tok[cand];
        qr_c = s_qrow[cand];
      }
      const float* qrow_c = sbase + static_cast<size_t>(qr_c) * V;
      // p and q at the candidate's token go out before the rows, so that
      // waiting for them does not wait for the rows; the poll wave loads
      // nothing here and takes them from wave 0 after the exchange
      if (wave != kPollWave) {
        lx_c = lrow[tok_c];
        qx_c = qrow_c[tok_c];
      }
      load8(qrow_c, qn, 0.f);
      load8(lbase + static_cast<size_t>(node_c + 1) * V, lvn, -INFINITY);
    }
    const uint32_t tag = static_cast<uint32_t>(ex_no + 1);
    const int par = ex_no & 1;
    uint64_t* bank = hdr + static_cast<size_t>(par) * G * kHdr;

    if (pass == P_ENTER) {
      // ---- statistics of u's row over this slice ----
      // Branch-free: a strict > keeps the first index of the max; a thread
      // whose entries are all -inf keeps no index, which only matters for a
      // row that fails anyway.  The flags only decide "any NaN, or no finite
      // maximum", so they follow from a NaN bit and the thread's maximum:
      // +inf present <=> max = +inf; some finite entry <=> max finite (NaN
      // never wins a >).
      float mx = -INFINITY;
      int arg = 0x7FFFFFFF;
      bool nan = false;
#pragma unroll
      for (int e = 0; e < kElem; ++e) {
        const float f = lv[e];
        nan |= f != f;
        const bool take = f > mx;
        mx = take ? f : mx;
        arg = take ? xa + e : arg;
      }
      int flags = (nan ? FLAG_NAN : 0) | (mx == INFINITY ? FLAG_PINF : 0) |
                  ((mx != INFINITY && mx != -INFINITY) ? FLAG_FINITE : 0);
      tv::wave_argmax_dpp(mx, arg);
      flags = tv::wave_or_dpp(flags);
      if (lane == 0) {
        s_wm[par][wave] = mx;
        s_wa[par][wave] = arg;
        s_wf[par][wave] = flags;
      }
      __syncthreads();
      float M = s_wm[par][0];
      int A = s_wa[par][0], F = s_wf[par][0];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) {
        tv::argmax_merge(M, A, s_wm[par][w2], s_wa[par][w2]);
        F |= s_wf[par][w2];
      }
      double S = 0.0;
      if (need_z && M != -INFINITY && M == M && M != INFINITY) {
        double acc = 0.0;
#pragma unroll
        for (int e = 0; e < kElem; ++e)
          acc += lv[e] != -INFINITY ? static_cast<double>(tv::exp_acc(lv[e] - M)) : 0.0;
        int unused;
        S = block_sum_or(acc, 0, s_red, s_redf, rs_no & 1, &unused);
        ++rs_no;
      }
      // slice argmax in bits 0..23 (< 2^20; a slice of -inf entries has no
      // index, 0x7FFFFFFF, cut to 0xFFFFFF so it cannot reach the flags),
      // flags in bits 24..26
      if (t == 0) {
        uint64_t* p = bank + static_cast<size_t>(g) * kHdr;
        put_tagged(p + 0, tag, __float_as_uint(M));
        put_tagged(p + 1, tag, lo32(S));
        put_tagged(p + 2, tag, hi32(S));
        put_tagged(p + 3, tag, (static_cast<uint32_t>(A) & 0xFFFFFFu) | (static_cast<uint32_t>(F) << 24));
      }
    } else {
      // ---- residual after rejecting the child whose draft row is in qv ----
      double acc = 0.0;
      int bad = 0;
#pragma unroll
      for (int e = 0; e < kElem; ++e) {      // padding: c = 0 and q = 0, so rn = 0
        const float c = mode == 0 ? (lv[e] == -INFINITY ? 0.f : tv::exp_acc(lv[e] - m)) : cv[e];
        bad |= q_bad(qv[e]) ? 1 : 0;
        rn[e] = static_cast<float>(fmax(0.0, static_cast<double>(c) - Z * static_cast<double>(qv[e])));
        acc += static_cast<double>(rn[e]);
      }
      int anyb;
      const double Zg = block_sum_or(acc, bad, s_red, s_redf, rs_no & 1, &anyb);
      ++rs_no;
      // the new residual at the remaining children's tokens: the owner of
      // each child's token publishes it
      {
        uint64_t kk = U;
        while (kk) {
          const int c = __builtin_ctzll(kk);
          kk &= kk - 1;
          const int x = s_tok[c];
          if (x >= xa && x < xa + nx) {
            float v = 0.f;
#pragma unroll
            for (int e = 0; e < kElem; ++e) v = (xa + e == x) ? rn[e] : v;
            put_tagged(kid + par * 64 + c, tag, __float_as_uint(v));
          }
        }
      }
      if (t == 0) {
        uint64_t* p = bank + static_cast<size_t>(g) * kHdr;
        put_tagged(p + 0, tag, lo32(Zg));
        put_tagged(p + 1, tag, hi32(Zg));
        put_tagged(p + 2, tag, static_cast<uint32_t>(anyb));
      }
    }

    // ---- while the exchange is under way: the next pass's words ----
    // MSS: lane 0 takes the outcome "accepted" (round 0 at the candidate's
    // node), lane 1 "rejected" (round j + 1 at u, the candidate removed);
    // each works out the Philox words, the next candidate and its node,
    // token and draft row, so that none of it follows the decision.  Naive:
    // the word of the draw at u.  The poll wave is polling; it takes wave
    // 0's values from LDS after the exchange.
    uint32_t spec[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    const bool speculate = (mss && cand >= 0) || (naive && pass == P_ENTER);
    if (speculate && wave != kPollWave) {
      const bool acc_lane = mss && lane == 0;
      const int node = mss ? (MULTI ? s_node[cand] : cand) : u;
      const tv::u32x4 ws = tv::mss_words(a.seed, a.offset, b, acc_lane || !mss ? node + 1 : u + 1,
                                         acc_lane || !mss ? 0 : j + 1);
      spec[0] = ws.x;
      spec[1] = ws.y;
      spec[2] = ws.z;
      spec[3] = ws.w;
      if (mss) {
        const uint64_t Un = acc_lane ? s_child[node + 1] : U & ~(1ull << cand);
        const int cs = Un ? nth_bit(Un, tv::pick_index(ws.x, __builtin_popcountll(Un))) : -1;
        spec[4] = static_cast<uint32_t>(cs);
        if (cs >= 0) {
          spec[5] = static_cast<uint32_t>(MULTI ? s_node[cs] : cs);
          spec[6] = static_cast<uint32_t>(s_tok[cs]);
          spec[7] = static_cast<uint32_t>(s_qrow[cs]);
        }
      }
      if (wave == 0 && lane < 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s_spec[par][lane][i] = spec[i];
      }
    }

    // ---- the poll wave gathers every workgroup's words into LDS ----
    // (A wave reads a bank only between this exchange's barrier and the next
    // pass's first barrier, and the poll wave refills the bank two exchanges
    // later, after that barrier.)
    if (wave == kPollWave) {
      bool to = false;
      if (pass == P_RESID && (MULTI || lane < N) && ((U >> lane) & 1ull)) {
        uint32_t v[kHdr] = {0u, 0u, 0u, 0u};
        if (!take_tagged<1>(kid + par * 64 + lane, tag, v, a.spin_limit)) to = true;
        s_rx2[par][lane] = __uint_as_float(v[0]);
      }
      for (int gg = lane; gg < G; gg += 64) {
        uint32_t v[kHdr] = {0u, 0u, 0u, 0u};
        const bool okp = pass == P_ENTER ? take_tagged<4>(bank + static_cast<size_t>(gg) * kHdr, tag, v, a.spin_limit)
                                         : take_tagged<3>(bank + static_cast<size_t>(gg) * kHdr, tag, v, a.spin_limit);
        if (!okp) to = true;
        if (pass == P_ENTER) {
          s_gm[par][gg] = __uint_as_float(v[0]);
          s_gs[par][gg] = join64(v[1], v[2]);
          s_ga[par][gg] = static_cast<int>(v[3]);
        } else {
          s_gs[par][gg] = join64(v[0], v[1]);
          s_ga[par][gg] = static_cast<int>(v[2]);
        }
      }
      if (__any(to) && lane == 0) s_timeout = 1;
    }
    if (mss && cand >= 0 && t == 0) {
      s_lxq[par][0] = lx_c;
      s_lxq[par][1] = qx_c;
    }
    __syncthreads();
    if (mss && cand >= 0 && wave == kPollWave) {
      lx_c = s_lxq[par][0];
      qx_c = s_lxq[par][1];
    }
    if (speculate && wave == kPollWave) {
#pragma unroll
      for (int i = 0; i < 8; ++i) spec[i] = s_spec[par][lane < 2 ? lane : 1][i];
    }
    ++ex_no;
    if (s_timeout) {
      timed_out = true;
      break;
    }

    // ---- merge the slices and decide (every wave, same values) ----
    bool fail = false;
    if (pass == P_ENTER) {
      // max with the lowest index on ties, flags, then the normaliser
      float mm = -INFINITY;
      int am = 0x7FFFFFFF, fl = 0;
      for (int gg = lane; gg < G; gg += 64) {
        fl |= static_cast<int>(static_cast<uint32_t>(s_ga[par][gg]) >> 24);
        tv::argmax_merge(mm, am, s_gm[par][gg], s_ga[par][gg] & 0xFFFFFF);
      }
      tv::wave_argmax_dpp(mm, am);
      fl = tv::wave_or_dpp(fl);
      fail = (fl & (FLAG_NAN | FLAG_PINF)) || !(fl & FLAG_FINITE);
      if (!fail && MODE == MODE_GREEDY) {
        // greedy: the child whose token is the argmax, lowest node first
        const uint64_t hit = __ballot(lane < N && ((U >> lane) & 1ull) && s_tok[lane] == am);
        if (hit) {
          const int nxt = __builtin_ctzll(hit);
          if (t == 0) s_acc[k] = nxt;
          ++k;
          u = nxt;
          U = s_child[nxt + 1];
          pre = nxt == c1 ? 1 : (nxt == c2 ? 2 : 0);
          pass = P_ENTER;
        } else {
          bonus = am;
          pass = P_DONE;
        }
      } else if (!fail) {
        double part = 0.0;
        for (int gg = lane; gg < G; gg += 64) {
          const float mg = s_gm[par][gg];
          const double tg = mg == -INFINITY ? 0.0 : s_gs[par][gg] * static_cast<double>(tv::exp_acc(mg - mm));
          s_gt[wave][gg] = tg;
          part += tg;
        }
        Z = tv::wave_sum_dpp(part);
        m = mm;
        mode = 0;
      }
    } else {
      double part = 0.0;
      int ab = 0;
      for (int gg = lane; gg < G; gg += 64) {
        part += s_gs[par][gg];
        ab |= s_ga[par][gg];
      }
      const double Znew = tv::wave_sum_dpp(part);
      fail = tv::wave_or_dpp(ab) != 0;
      if (!fail && Znew > 0.0) {       // else the distribution stays (zero-normaliser guard)
        for (int gg = lane; gg < G; gg += 64) s_gt[wave][gg] = s_gs[par][gg];
        if ((MULTI || lane < N) && ((U >> lane) & 1ull)) rx = s_rx2[par][lane];
#pragma unroll
        for (int e = 0; e < kElem; ++e) cv[e] = rn[e];
        Z = Znew;
        mode = 1;
      }
    }
    if (fail) {
      status = TV_REQ_NONFINITE;
    } else if (mss && cand >= 0) {   // (cand >= 0 only in MSS)
      {
        // ratio test: u1 <= p(x) / q(x) with p(x) = e / Z, tested as
        // u1 * q(x) * Z <= e (no division); q(x) = 0 accepts exactly when p(x) > 0
        if (q_bad(qx_c)) {
          status = TV_REQ_NONFINITE;
        } else {
          const double e = mode == 0 ? (lx_c == -INFINITY ? 0.0 : static_cast<double>(tv::exp_acc(lx_c - m)))
                                     : static_cast<double>(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(rx), cand)));
          const bool accept = qx_c > 0.f ? tv::unit_open0(w.y) * static_cast<double>(qx_c) * Z <= e : e > 0.0;
          ++rounds;
          if (accept) {
            const int node = MULTI ? s_node[cand] : cand;   // the proposal's node
            if (t == 0) s_acc[k] = node;
            ++k;
            u = node;
            U = s_child[node + 1];
            j = 0;
            pass = P_ENTER;
          } else {
            U &= ~(1ull << cand);
            ++j;
            pass = P_RESID;
          }
          const int from = accept ? 0 : 1;
          w_next.x = __builtin_amdgcn_readlane(spec[0], from);
          w_next.y = __builtin_amdgcn_readlane(spec[1], from);
          w_next.z = __builtin_amdgcn_readlane(spec[2], from);
          w_next.w = __builtin_amdgcn_readlane(spec[3], from);
          c_next = static_cast<int>(__builtin_amdgcn_readlane(spec[4], from));
          node_next = static_cast<int>(__builtin_amdgcn_readlane(spec[5], from));
          tok_next = static_cast<int>(__builtin_amdgcn_readlane(spec[6], from));
          qr_next = static_cast<int>(__builtin_amdgcn_readlane(spec[7], from));
          have_next = true;
        }
      }
    } else if (need_z) {
      // MSS with no child left, or naive having entered u: locate the slice
      // of the draw (the next pass makes it)
      locate(mss ? zdraw : __builtin_amdgcn_readlane(spec[2], 0));
      pass = mss ? P_FINAL : P_NSAMPLE;
    }
  }
  if constexpr (COMMIT)
    if (wave == kPollWave && lane < tv::kMaxTreeBlocks) s_tblk[lane] = tblk;
  __syncthreads();
  const bool ok = status == TV_REQ_OK && !s_timeout;

  // ---- MSS's final sample: the owner slice's workgroup finds the token.
  // Workgroup 0 writes every output of the request, so an owner other than
  // workgroup 0 hands the token over in a tagged word of the request's
  // workspace line (workgroup 0 waits for it below). ----
  uint64_t* const xword = reinterpret_cast<uint64_t*>(done + 2);
  const bool final_draw = mss && ok && pass == P_FINAL;
  if (final_draw && g == owner) {
    const int x = slice_search();
    if (g == 0) bonus = x;
    else if (t == 0) put_tagged(xword, 1u, static_cast<uint32_t>(x));
  }

  int stt = status;
  if (stt == TV_REQ_OK && s_timeout) stt = TV_REQ_TIMEOUT;

  // ---- verify + commit: every workgroup compacts the accepted path of its
  // own block of heads, [g H / G, (g + 1) H / G), exactly as
  // kv_commit_accepted would after this call.  Heads occupy disjoint rows,
  // so the workgroups' moves never meet; within one, the batches keep the
  // order kv_move.h describes.  Workgroup 0 decides whether the move is made
  // (its walk, the checks and the final token's hand-over) and posts the
  // decision; the others move only on it and report, and workgroup 0 grows
  // the prefix length only when every report says moved.  Otherwise the
  // request times out with its prefix length unchanged (the rows of its
  // tree's slots may then be partly compacted).  Each workgroup's checks and
  // first batch of row loads go out now, so the loads are in flight during
  // the hand-over. ----
  tv::MovePlan plan;
  int mres = -1;                   // TV_REQ_OK: move; -1: nothing to do; else the status to store
  int mv_begin = 0;                // this workgroup's first item of the move
  uint4 mbuf[kMoveChunks];
  uint64_t* const dword = reinterpret_cast<uint64_t*>(done + 4);   // COMMIT: the decision
  uint32_t* const acks = done + 6;                                  // COMMIT: the reports
  if constexpr (COMMIT) {
    mres = tv::move_prepare<kCoThreads, kMoveChunks, true>(a.kv, b, N, stt, s_L, ok ? k : -1, s_acc, false, s_mv,
                                                            s_tblk, plan);
    if (mres == TV_REQ_OK) {
      mv_begin = (g * a.kv.H) / G * plan.per_head;
      plan.total = ((g + 1) * a.kv.H) / G * plan.per_head;
      if (mv_begin < plan.total) tv::move_load<kCoThreads, kMoveChunks>(a.kv, plan, s_mv, mv_begin, mbuf);
    }
  }

  // ---- MSS's token from another slice arrives in the tagged word; if it
  // does not within the wait bound, the request times out like any other
  // wait (no output, no move), so the outputs always come from one
  // decision. ----
  if (g == 0 && final_draw && owner != 0) {
    if (t == 0) {
      uint32_t v[kHdr] = {0u, 0u, 0u, 0u};
      s_xs = take_tagged<1>(xword, 1u, v, a.spin_limit) ? static_cast<int>(v[0]) : -1;
    }
    __syncthreads();
    if (s_xs >= 0) {
      bonus = s_xs;
    } else {
      stt = TV_REQ_TIMEOUT;
      mres = -1;
    }
  }

  if constexpr (COMMIT) {
    if (g == 0 && t == 0) put_tagged(dword, 1u, mres == TV_REQ_OK ? 1u : 0u);
    if (g != 0 && t == 0) {
      int dec = 0;
      if (mres == TV_REQ_OK) {
        uint32_t v[kHdr] = {0u, 0u, 0u, 0u};
        dec = take_tagged<1>(dword, 1u, v, a.spin_limit) ? static_cast<int>(v[0]) : 0;
      }
      s_dec = dec;
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the first batch have completed
    __syncthreads();
    const bool go = mres == TV_REQ_OK && (g == 0 || s_dec == 1);
    if (go && mv_begin < plan.total) {
      tv::move_store<kCoThreads, kMoveChunks>(a.kv, plan, s_mv, mv_begin, mbuf);
      tv::move_rest<kCoThreads, kMoveChunks>(a.kv, plan, s_mv, mv_begin + plan.step);
    }
    if (g != 0) {
      if (t == 0) __hip_atomic_fetch_add(acks, go ? 1u : 0x10000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (go) {
      // every other workgroup's report: low half moved, high half not
      if (t == 0) {
        int all = 0;
        for (unsigned polls = 0; polls < a.spin_limit; ++polls) {
          const uint32_t x = __hip_atomic_load(acks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (static_cast<int>((x & 0xFFFFu) + (x >> 16)) >= G - 1) {
            all = (x >> 16) == 0u ? 1 : 0;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        s_acks = all;
      }
      __syncthreads();
      if (!s_acks) {
        stt = TV_REQ_TIMEOUT;
        mres = -1;
      }
    }
  }

  // ---- results: workgroup 0 writes the path, the bonus and the status ----
  if (g == 0) {
    if (t == 0) {
      if (stt != TV_REQ_OK) {
        a.status[b] = stt;
        a.num_accepted[b] = -1;
        a.bonus[b] = -1;
        if (a.rounds) a.rounds[b] = -1;
      } else {
        a.num_accepted[b] = k;
        a.bonus[b] = bonus;
        if (a.rounds) a.rounds[b] = rounds;
      }
      if constexpr (COMMIT) {
        if (mres == TV_REQ_OK) a.kv.prefix_len[b] = s_L + k;
        else if (mres >= 0 && mres != stt) a.status[b] = mres;
      }
    }
    const int kk = stt == TV_REQ_OK ? k : 0;
    for (int i = t; i < N; i += kCoThreads) a.accepted[static_cast<size_t>(b) * N + i] = i < kk ? s_acc[i] : -1;
  }

  // ---- leave the workspace zeroed: the last workgroup out clears it ----
  __builtin_amdgcn_s_waitcnt(0);     // this thread's stores have completed
  __syncthreads();
  uint32_t prev = 0;
  if (t == 0) prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == 0) s_last = prev == static_cast<uint32_t>(G - 1);
  __syncthreads();
  if (s_last) {          // every workgroup has finished reading
    for (int i = t; i < 2 * G * kHdr; i += kCoThreads) st_u64(hdr + i, 0ull);
    if (t < 128) st_u64(kid + t, 0ull);
    if (t == 0) {
      st_u32(done, 0u);
      st_u64(xword, 0ull);
      if constexpr (COMMIT) {
        st_u64(dword, 0ull);
        st_u32(acks, 0u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row-resident walk, for V <= kRowThreads * kRowMaxE (16384): one workgroup
// of 512 threads per request holds the whole current distribution in
// registers, so a step of the walk synchronises one workgroup and never waits
// for another.  Up to that size a walk step is cheaper on one CU than an
// exchange between CUs, which costs two memory round trips plus the skew
// between workgroups; beyond it, one CU's share of memory bandwidth (a few
// tens of GB/s) makes streaming a whole row slower than splitting it.  Two
// waves per SIMD leave room for the distribution row, the row being reduced
// and the temporaries; the passes are independent per entry, so two waves
// keep the vector units busy.  Every node's draft probability of its own
// token is loaded while the request is staged, so a ratio test never waits
// for memory.
//
// Entry x of a row lives in thread (x mod 2048) / 4, register
// 4 * (x / 2048) + x mod 4, so each load instruction of a wave reads 1 KB of
// contiguous row, and a thread's registers are in increasing x order.
//
// Loads are issued as soon as their rows are known.  The entered node's row
// and the draft row of its first tested child are fetched together; each
// residual pass first takes the draft row of the rejected child, then starts
// fetching the draft row of the child tested after it (the random choice of
// that child does not depend on any outcome still open), so every draft row
// streams in during a whole pass before it is needed.  Greedy fetches the
// rows of the entered node's first two children while it reduces the node's
// row.  One of the prefetched rows goes to LDS through direct-to-LDS loads,
// which hold no registers while in flight.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 512;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRowQuad = 4 * kRowThreads;        // entries covered by one register quad
constexpr int kRowMaxE = 32;                     // registers per row per thread

template <int E, bool VEC, int MODE, bool COMMIT, bool MULTI = false>
__global__ __launch_bounds__(kRowThreads) void walk_row_kernel(WalkArgs a) {
  static_assert(E % 4 == 0 && E <= kRowMaxE, "row registers");
  constexpr int C = E / 4;
  const int b = a.b0 + static_cast<int>(blockIdx.x);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int N = a.N, V = a.V;
  constexpr bool mss = MODE == MODE_MSS, naive = MODE == MODE_NAIVE;
  const float* lbase = a.logits + static_cast<size_t>(b) * (N + 1) * V;
  const float* sbase = mss ? a.ssm + static_cast<size_t>(b) * a.R * V : nullptr;

  // per child (per proposal slot when MULTI): token, draft row, draft
  // probability of the token; s_node the slot's node (MULTI)
  __shared__ int s_tok[TV_MAX_NODES], s_qrow[TV_MAX_NODES], s_acc[TV_MAX_NODES], s_node[TV_MAX_NODES];
  __shared__ float s_qx[TV_MAX_NODES];
  __shared__ uint64_t s_child[TV_MAX_NODES + 1];
  __shared__ float s_wm[2][kRowWaves];           // per-wave max, two banks
  __shared__ int s_wa[2][kRowWaves], s_wf[2][kRowWaves];
  __shared__ double s_ws[2][kRowWaves];          // per-wave sums, two banks
  __shared__ float s_ex[2][2];                   // the next child's token: old / new residual
  __shared__ double s_scan[C * kRowWaves];       // final sample: wave totals, quad-major
  __shared__ int s_status0, s_found;
  __shared__ int s_L;                            // COMMIT: the request's prefix length
  __shared__ tv::CommitLds s_mv;                 // COMMIT: the move's block offsets
  // the prefetched row (a draft row in MSS, the second child's logits in
  // greedy), in x order, written by direct-to-LDS loads; each wave reads
  // back only what its own loads wrote
  __shared__ float s_row[VEC ? E * kRowThreads : 4];

  // entry held by register e of this thread
  auto xof = [&](int e) { return (e >> 2) * kRowQuad + 4 * t + (e & 3); };
  // Registers past the end of the row get a neutral value (-inf for logits,
  // 0 for draft rows), so the passes over a row need no bounds tests: -inf
  // never wins a max and becomes 0 in the distribution, and a zero draft
  // entry leaves a zero residual.
  // (The quad's offset stays in the scalar base address and the bounds test
  // is uniform except in the one quad that the row's end cuts, so no
  // per-quad vector state lives across the walk.)
  const int t4 = 4 * t;
  auto load_row = [&](const float* row, float (&d)[E], float pad) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const float* rq = row + i * kRowQuad;
      const int lim = V - i * kRowQuad;        // entries of this quad inside the row
#pragma unroll
      for (int r = 0; r < 4; ++r) d[4 * i + r] = pad;
      if constexpr (VEC) {     // V % 4 == 0 and 16-byte aligned rows
        if (lim >= kRowQuad || (lim > 0 && t4 < lim)) {
          const float4 f = *reinterpret_cast<const float4*>(rq + t4);
          d[4 * i] = f.x; d[4 * i + 1] = f.y; d[4 * i + 2] = f.z; d[4 * i + 3] = f.w;
        }
      } else {
        if (lim >= kRowQuad) {
#pragma unroll
          for (int r = 0; r < 4; ++r) d[4 * i + r] = rq[t4 + r];
        } else if (lim > 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (t4 + r < lim) d[4 * i + r] = rq[t4 + r];
        }
      }
    }
  };
  // Start loading a row into s_row (no registers held while it streams).
  // Rows that vector loads cannot read (V % 4 != 0, or unaligned) are read
  // straight into registers when they are taken instead.
  const float* pf_row = nullptr;
  auto dma_row = [&](const float* row) {
    pf_row = row;
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const int lim = V - i * kRowQuad;
        if (lim >= kRowQuad || (lim > 0 && t4 < lim)) {
          const float* src = row + i * kRowQuad + t4;
          // lane l's 16 bytes land at M0 + 16 l: this wave's 1 KB of the quad
          const uint32_t dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s_row + i * kRowQuad + 256 * wave));
          asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(dst) : "memory");
        }
      }
    }
  };
  // take the prefetched row into registers (past the row's end: pad)
  auto lds_row = [&](float (&d)[E], float pad) {
    if constexpr (VEC) {
      // the row's loads have landed (they are this wave's oldest outstanding loads)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const int lim = V - i * kRowQuad;
        float4 f = make_float4(pad, pad, pad, pad);
        if (lim >= kRowQuad || (lim > 0 && t4 < lim))
          f = *reinterpret_cast<const float4*>(s_row + i * kRowQuad + t4);
        d[4 * i] = f.x; d[4 * i + 1] = f.y; d[4 * i + 2] = f.z; d[4 * i + 3] = f.w;
      }
      // every read of s_row is complete before a later load may overwrite it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      load_row(pf_row, d, pad);
    }
  };
  // value of entry x in the thread that holds it
  auto held = [&](const float (&d)[E], int x) {
    const int r = 4 * (x / kRowQuad) + (x & 3);
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) v = e == r ? d[e] : v;
    return v;
  };
  auto holds = [&](int x) { return x >= 0 && ((x % kRowQuad) >> 2) == t; };
  // workgroup sum of a double and OR of an int (one barrier, alternating banks)
  int bank = 0;
  auto block_sum = [&](double v, int f, int* f_out) {
    v = tv::wave_sum_dpp(v);
    f = tv::wave_or_dpp(f);
    if (lane == 0) {
      s_ws[bank][wave] = v;
      s_wf[bank][wave] = f;
    }
    __syncthreads();
    // lanes 0..15 take the wave partials; the same DPP reduction in every
    // wave gives every thread the same sum
    const double s = tv::wave_sum_dpp(lane < kRowWaves ? s_ws[bank][lane] : 0.0);
    const int o = tv::wave_or_dpp(lane < kRowWaves ? s_wf[bank][lane] : 0);
    bank ^= 1;
    *f_out = o;
    return s;
  };
  // workgroup max of the valid entries (lowest index among equal maxima) and
  // whether any is NaN (one barrier)
  auto block_argmax = [&](const float (&d)[E], float* m_out, int* a_out) {
    float mx = -INFINITY;
    int re = -1, nan = 0;          // register of the first maximum
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float f = d[e];
      nan |= f != f;
      if (f > mx || (f == mx && re < 0)) {
        mx = f;
        re = e;
      }
    }
    int arg = (re >> 2) * kRowQuad + 4 * t + (re & 3);
    tv::wave_argmax_dpp(mx, arg);
    nan = tv::wave_or_dpp(nan);
    if (lane == 0) {
      s_wm[bank][wave] = mx;
      s_wa[bank][wave] = arg;
      s_wf[bank][wave] = nan;
    }
    __syncthreads();
    float M = lane < kRowWaves ? s_wm[bank][lane] : -INFINITY;
    int A = lane < kRowWaves ? s_wa[bank][lane] : 0x7FFFFFFF;
    tv::wave_argmax_dpp(M, A);
    const int F = tv::wave_or_dpp(lane < kRowWaves ? s_wf[bank][lane] : 0);
    bank ^= 1;
    *m_out = M;
    *a_out = A;
    return F;     // nonzero: some entry is NaN
  };
  // the same without the index (MSS needs only the maximum)
  auto block_max = [&](const float (&d)[E], float* m_out) {
    float mx = -INFINITY;
    int nan = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      nan |= d[e] != d[e];
      mx = fmaxf(mx, d[e]);
    }
    mx = tv::wave_max_dpp(mx);
    nan = tv::wave_or_dpp(nan);
    if (lane == 0) {
      s_wm[bank][wave] = mx;
      s_wf[bank][wave] = nan;
    }
    __syncthreads();
    const float M = tv::wave_max_dpp(lane < kRowWaves ? s_wm[bank][lane] : -INFINITY);
    const int F = tv::wave_or_dpp(lane < kRowWaves ? s_wf[bank][lane] : 0);
    bank ^= 1;
    *m_out = M;
    return F;
  };

  // ---------------- first loads, staging ----------------
  float lv[E];             // the entered node's logits; then its distribution (unnormalised)
  float qa[E];             // MSS: the rejected child's draft row, then the residual; greedy: first child's row
  load_row(lbase, lv, -INFINITY);
  if (wave == 0) {
    const size_t rb = static_cast<size_t>(b);
    const int st0 = lane == 0 ? a.status[b] : 0;
    const uint64_t cm = lane < N ? a.child[rb * (N + 1) + lane] & later_nodes(lane - 1, N) : 0ull;
    const int tok = lane < N ? a.token[rb * N + lane] : 0;
    const int qr = (mss && !MULTI && lane < N) ? a.q_row[rb * N + lane] : 0;
    const uint64_t real = wave_or64(cm);
    const uint64_t bad_tok = __ballot(lane < N && (tok < 0 || tok >= V));
    uint64_t bad_q = __ballot(mss && !MULTI && lane < N && (qr < 0 || qr >= a.R)) & real;
    // every tested child's ratio needs q(token): load them all now, in parallel
    if constexpr (MULTI) {
      const SlotStage ss = stage_slots(a, b, N, cm, tok, real, &bad_q);
      s_child[lane] = ss.child_slots;
      s_tok[lane] = ss.tok;
      s_qrow[lane] = ss.row;
      s_node[lane] = ss.node;
      const bool ok_q = ss.node >= 0 && ss.tok >= 0 && ss.tok < V;
      s_qx[lane] = ok_q ? sbase[static_cast<size_t>(ss.row) * V + ss.tok] : 0.f;
    } else {
      s_child[lane] = cm;
      s_tok[lane] = tok;
      s_qrow[lane] = qr;
      const bool ok_q = mss && lane < N && tok >= 0 && tok < V && qr >= 0 && qr < a.R;
      s_qx[lane] = ok_q ? sbase[static_cast<size_t>(qr) * V + tok] : 0.f;
    }
    if (lane == 0) {
      s_child[TV_MAX_NODES] = 0ull;
      int st = st0;
      if (st == TV_REQ_OK) {
        if (bad_tok & real) st = TV_REQ_BAD_TOKEN;
        else if (bad_q) st = TV_REQ_BAD_QROW;
      }
      s_status0 = st;
      if constexpr (COMMIT) s_L = a.kv.prefix_len[b];   // nothing writes it before the move
    }
  }
  __syncthreads();

  int status = s_status0;
  int u = -1, k = 0, rounds = 0, bonus = -1;
  uint64_t U = s_child[0];
  double Z = 1.0;
  bool final_sample = false;

  // ---- a sample of the current distribution: smallest x with cumsum >= u * total ----
  // Cumulative sums run in x order: quad by quad, within a quad wave by wave,
  // within a wave lane by lane (four entries per lane).  Every wave publishes
  // its scanned total per quad; a scan over those totals (the same in every
  // wave) finds the (quad, wave) whose range brackets the threshold, and only
  // that wave repeats its lane scan (the same operations on the same values,
  // so the same sums) to find the lane and the entry.  Inside one wave each
  // inclusive sum equals the next lane's exclusive sum bit for bit, so with
  // the threshold clamped to the wave's top exactly one lane brackets it.
  auto sample_lv = [&](uint32_t word) -> int {
    constexpr int K = C * kRowWaves;                 // (quad, wave) ranges
    constexpr int NB = (K + 63) / 64;
    auto quad_sum = [&](int i) {
      double s = 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r) s += static_cast<double>(lv[4 * i + r]);
      return s;
    };
#pragma unroll
    for (int i = 0; i < C; ++i) {
      double ex;
      const double inc = tv::wave_scan_dpp(quad_sum(i), &ex);
      if (lane == 63) s_scan[i * kRowWaves + wave] = inc;
    }
    if (t == 0) s_found = -1;
    __syncthreads();
    // prefix sums over the ranges, 64 per batch (every wave alike)
    double lo[NB], hi[NB], carry = 0.0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int kk = nb * 64 + lane;
      const double v = kk < K ? s_scan[kk] : 0.0;
      double ex;
      const double in = tv::wave_scan_dpp(v, &ex);
      lo[nb] = carry + ex;
      hi[nb] = carry + in;
      carry = tv::readlane_f64(hi[nb], 63);
    }
    const double T = tv::unit_open0(word) * carry;   // in (0, total]
    int kstar = -1;
    double Astar = 0.0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint64_t hit = __ballot(lo[nb] < T && hi[nb] >= T);
      if (kstar < 0 && hit) {
        const int l = __builtin_ctzll(hit);
        kstar = nb * 64 + l;
        Astar = tv::readlane_f64(lo[nb], l);
      }
    }
    if (kstar < 0) {            // rounding left the total short: the last non-empty range
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint64_t pos = __ballot(hi[nb] > lo[nb]);
        if (pos) {
          const int l = 63 - __builtin_clzll(pos);
          kstar = nb * 64 + l;
          Astar = tv::readlane_f64(lo[nb], l);
        }
      }
    }
    const int qi = kstar / kRowWaves, qw = kstar % kRowWaves;
    if (kstar >= 0 && wave == qw) {
      double sq = 0.0;
#pragma unroll
      for (int i = 0; i < C; ++i)
        if (i == qi) sq = quad_sum(i);
      double exl;
      const double inl = tv::wave_scan_dpp(sq, &exl);
      const double Tw = fmin(T, Astar + tv::readlane_f64(inl, 63));
      const double l0 = Astar + exl, l1 = Astar + inl;
      if (l0 < Tw && l1 >= Tw) {
        double accd = l0;
        int xs = -1, last_pos = -1;
#pragma unroll
        for (int i = 0; i < C; ++i) {
          if (i == qi) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float c = lv[4 * i + r];
              if (xs < 0) {
                if (c > 0.f) last_pos = xof(4 * i + r);
                accd += static_cast<double>(c);
                if (accd >= Tw) xs = xof(4 * i + r);
              }
            }
          }
        }
        s_found = xs >= 0 ? xs : last_pos;   // rounding left the lane short: its last positive entry
      }
    }
    __syncthreads();
    return s_found;
  };


  // greedy and naive: the rows of the entered node's first two children
  int c1 = -1, c2 = -1;
  auto fetch_children = [&]() {
    c1 = U ? __builtin_ctzll(U) : -1;
    const uint64_t rest = U & (U - 1);
    c2 = rest ? __builtin_ctzll(rest) : -1;
    if (c1 >= 0) load_row(lbase + static_cast<size_t>(c1 + 1) * V, qa, -INFINITY);
    if (c2 >= 0) dma_row(lbase + static_cast<size_t>(c2 + 1) * V);
  };
  auto enter_child = [&](int nxt) {
    if (t == 0) s_acc[k] = nxt;
    ++k;
    u = nxt;
    U = s_child[nxt + 1];
    if (nxt == c1) {
#pragma unroll
      for (int e = 0; e < E; ++e) lv[e] = qa[e];
    } else if (nxt == c2) {
      lds_row(lv, -INFINITY);
    } else {
      load_row(lbase + static_cast<size_t>(u + 1) * V, lv, -INFINITY);
    }
    fetch_children();
  };

  if (status == TV_REQ_OK && naive) {
    // ---------------- naive sampling: draw, then look for the token ----------------
    fetch_children();
    for (;;) {
      float M;
      const int nan = block_max(lv, &M);
      if (nan || M == INFINITY || M == -INFINITY) {
        status = TV_REQ_NONFINITE;
        break;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) lv[e] = lv[e] != -INFINITY ? tv::exp_acc(lv[e] - M) : 0.f;
      const int x = sample_lv(tv::mss_words(a.seed, a.offset, b, u + 1, 0).z);
      const uint64_t hit = __ballot(lane < N && ((U >> lane) & 1ull) && s_tok[lane] == x);
      if (!hit) {
        bonus = x;
        break;
      }
      enter_child(__builtin_ctzll(hit));
    }
  } else if (status == TV_REQ_OK && !mss) {
    // ---------------- greedy ----------------
    fetch_children();
    for (;;) {
      float M;
      int A;
      const int nan = block_argmax(lv, &M, &A);
      if (nan || M == INFINITY || M == -INFINITY) {
        status = TV_REQ_NONFINITE;
        break;
      }
      const uint64_t hit = __ballot(lane < N && ((U >> lane) & 1ull) && s_tok[lane] == A);
      if (!hit) {
        bonus = A;
        break;
      }
      enter_child(__builtin_ctzll(hit));
    }
  } else if (status == TV_REQ_OK) {
    // ---------------- MSS ----------------
    int j = 0, cand = -1;
    float qx = 0.f;          // draft probability of the candidate's token
    auto choose = [&]() {    // candidate of round j among U; start fetching its draft row
      cand = -1;
      if (U) {
        const tv::u32x4 w = tv::mss_words(a.seed, a.offset, b, u + 1, j);
        cand = nth_bit(U, tv::pick_index(w.x, __builtin_popcountll(U)));
        dma_row(sbase + static_cast<size_t>(s_qrow[cand]) * V);
        qx = s_qx[cand];
      }
    };
    choose();
    float ex = 0.f;          // current distribution at the candidate's token (unnormalised)
    bool enter = true;
    for (;;) {
      if (enter) {
        // ---- statistics of u's row; lv becomes exp(l - max) ----
        float M;
        const int nan = block_max(lv, &M);
        if (nan || M == INFINITY || M == -INFINITY) {
          status = TV_REQ_NONFINITE;
          break;
        }
        double acc = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          lv[e] = lv[e] != -INFINITY ? tv::exp_acc(lv[e] - M) : 0.f;
          acc += static_cast<double>(lv[e]);
        }
        if (cand >= 0 && holds(s_tok[cand])) s_ex[bank][0] = held(lv, s_tok[cand]);
        const int eb = bank;
        int unused;
        Z = block_sum(acc, 0, &unused);
        ex = s_ex[eb][0];
        enter = false;
      }
      if (cand < 0) {
        final_sample = true;
        break;
      }
      // ---- ratio test: u1 <= p(x) / q(x) with p(x) = ex / Z, tested as
      // u1 * q(x) * Z <= ex; q(x) = 0 accepts exactly when p(x) > 0 ----
      if (q_bad(qx)) {
        status = TV_REQ_NONFINITE;
        break;
      }
      const tv::u32x4 w = tv::mss_words(a.seed, a.offset, b, u + 1, j);
      const double e = static_cast<double>(ex);
      const bool accept = qx > 0.f ? tv::unit_open0(w.y) * static_cast<double>(qx) * Z <= e : e > 0.0;
      ++rounds;
      if (accept) {
        const int node = MULTI ? s_node[cand] : cand;   // the proposal's node
        if (t == 0) s_acc[k] = node;
        ++k;
        u = node;
        U = s_child[node + 1];
        j = 0;
        load_row(lbase + static_cast<size_t>(u + 1) * V, lv, -INFINITY);
        choose();
        enter = true;
        continue;
      }
      // ---- rejection: residual max(0, p - q) with the rejected child's draft row ----
      U &= ~(1ull << cand);
      ++j;
      lds_row(qa, 0.f);
      choose();                         // the next candidate's draft row now streams into s_row
      double acc = 0.0;
      int bad = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (q_bad(qa[e])) bad = 1;
        qa[e] = static_cast<float>(fmax(0.0, static_cast<double>(lv[e]) - Z * static_cast<double>(qa[e])));
        acc += static_cast<double>(qa[e]);
      }
      if (cand >= 0 && holds(s_tok[cand])) {
        s_ex[bank][0] = held(lv, s_tok[cand]);
        s_ex[bank][1] = held(qa, s_tok[cand]);
      }
      const int eb = bank;
      int anyb;
      const double Znew = block_sum(acc, bad, &anyb);
      if (anyb) {
        status = TV_REQ_NONFINITE;
        break;
      }
      if (Znew > 0.0) {                 // else the distribution stays (zero-normaliser guard)
#pragma unroll
        for (int e = 0; e < E; ++e) lv[e] = qa[e];
        Z = Znew;
        ex = s_ex[eb][1];
      } else {
        ex = s_ex[eb][0];
      }
    }
  }

  if (final_sample) {
    const tv::u32x4 w0 = tv::mss_words(a.seed, a.offset, b, u + 1, 0);
    bonus = sample_lv(w0.z);
  }

  // ---------------- results ----------------
  // a prefetched row that was never taken may still be landing in LDS: let
  // it land before the workgroup's LDS can go to another workgroup
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();       // s_acc complete
  if (t == 0) {
    if (status != TV_REQ_OK) {
      a.status[b] = status;
      a.num_accepted[b] = -1;
      a.bonus[b] = -1;
      if (a.rounds) a.rounds[b] = -1;
    } else {
      a.num_accepted[b] = k;
      a.bonus[b] = bonus;
      if (a.rounds) a.rounds[b] = rounds;
    }
  }
  const int kk = status == TV_REQ_OK ? k : 0;
  for (int i = t; i < N; i += kRowThreads) a.accepted[static_cast<size_t>(b) * N + i] = i < kk ? s_acc[i] : -1;
  // verify + commit: compact the accepted path, as kv_commit_accepted would
  if constexpr (COMMIT) {
    const int res = tv::commit_request<kRowThreads, kMoveChunks, true>(a.kv, b, N, status, s_L,
                                                                        status == TV_REQ_OK ? k : -1, s_acc, false, s_mv);
    if (t == 0 && res != status) a.status[b] = res;
  }
}

tv_status check_verify_args(int B, int N, int V) {
  if (B < 0 || N < 0 || V < 1 || V > (1 << 20)) return TV_EINVAL;
  if (N > TV_MAX_NODES) return TV_ETOOBIG;
  return TV_OK;
}

// kernel variant: 0 greedy, 1 MSS, 2 naive, 3 MSS + commit, 4 MSS over proposals
template <bool VEC, int E>
const void* walk_kernel_of(int variant) {
  if (variant == 4) return reinterpret_cast<const void*>(walk_kernel<MODE_MSS, VEC, false, true, E>);
  if (variant == 3) return reinterpret_cast<const void*>(walk_kernel<MODE_MSS, VEC, true, false, E>);
  if (variant == MODE_MSS) return reinterpret_cast<const void*>(walk_kernel<MODE_MSS, VEC, false, false, E>);
  if (variant == MODE_NAIVE) return reinterpret_cast<const void*>(walk_kernel<MODE_NAIVE, VEC, false, false, E>);
  return reinterpret_cast<const void*>(walk_kernel<MODE_GREEDY, VEC, false, false, E>);
}

int elem_index(int E) { return E == 4 ? 0 : (E == 8 ? 1 : 2); }

// Compute units of device dev (cached per device).
int device_cus(int dev) {
  static std::atomic<int> cache[64];
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
  if (cached) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Workgroups of a walk variant resident at once on device dev (cached per
// device, variant and slice width; every thread that fills an entry computes
// the same value, so relaxed atomics suffice).
int walk_capacity(int dev, int variant, bool vec, int E) {
  static std::atomic<int> cache[2][5][3][64];
  const int ei = elem_index(E);
  const bool cached = dev >= 0 && dev < 64 && variant >= 0 && variant < 5;
  if (cached) {
    const int c = cache[vec][variant][ei][dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  const int cus = device_cus(dev);
  if (cus <= 0) return 0;
  const void* fn = ei == 0 ? (vec ? walk_kernel_of<true, 4>(variant) : walk_kernel_of<false, 4>(variant))
                 : ei == 1 ? (vec ? walk_kernel_of<true, 8>(variant) : walk_kernel_of<false, 8>(variant))
                           : (vec ? walk_kernel_of<true, 16>(variant) : walk_kernel_of<false, 16>(variant));
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kCoThreads, 0) != hipSuccess) return 0;
  const int cap = cus * std::max(1, per_cu);
  if (cached) cache[vec][variant][ei][dev].store(cap, std::memory_order_relaxed);
  return cap;
}

template <bool VEC, int E>
void launch_sliced_ve(const WalkArgs& a, int grid, hipStream_t stream) {
  if (a.mode == MODE_MSS && a.multi)
    hipLaunchKernelGGL((walk_kernel<MODE_MSS, VEC, false, true, E>), dim3(grid), dim3(kCoThreads), 0, stream, a);
  else if (a.mode == MODE_MSS && a.commit)
    hipLaunchKernelGGL((walk_kernel<MODE_MSS, VEC, true, false, E>), dim3(grid), dim3(kCoThreads), 0, stream, a);
  else if (a.mode == MODE_MSS)
    hipLaunchKernelGGL((walk_kernel<MODE_MSS, VEC, false, false, E>), dim3(grid), dim3(kCoThreads), 0, stream, a);
  else if (a.mode == MODE_NAIVE)
    hipLaunchKernelGGL((walk_kernel<MODE_NAIVE, VEC, false, false, E>), dim3(grid), dim3(kCoThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((walk_kernel<MODE_GREEDY, VEC, false, false, E>), dim3(grid), dim3(kCoThreads), 0, stream, a);
}

void launch_sliced(const WalkArgs& a, int grid, bool vec, int E, hipStream_t stream) {
  if (E == 4) vec ? launch_sliced_ve<true, 4>(a, grid, stream) : launch_sliced_ve<false, 4>(a, grid, stream);
  else if (E == 8) vec ? launch_sliced_ve<true, 8>(a, grid, stream) : launch_sliced_ve<false, 8>(a, grid, stream);
  else vec ? launch_sliced_ve<true, 16>(a, grid, stream) : launch_sliced_ve<false, 16>(a, grid, stream);
}

template <int E, int MODE, bool COMMIT = false, bool MULTI = false>
void launch_row_mode(const WalkArgs& a, int B, bool vec, hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL((walk_row_kernel<E, true, MODE, COMMIT, MULTI>), dim3(B), dim3(kRowThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((walk_row_kernel<E, false, MODE, COMMIT, MULTI>), dim3(B), dim3(kRowThreads), 0, stream, a);
}
template <int E>
void launch_row(const WalkArgs& a, int B, bool vec, hipStream_t stream) {
  if (a.mode == MODE_MSS && a.multi) launch_row_mode<E, MODE_MSS, false, true>(a, B, vec, stream);
  else if (a.mode == MODE_MSS && a.commit) launch_row_mode<E, MODE_MSS, true>(a, B, vec, stream);
  else if (a.mode == MODE_MSS) launch_row_mode<E, MODE_MSS>(a, B, vec, stream);
  else if (a.mode == MODE_NAIVE) launch_row_mode<E, MODE_NAIVE>(a, B, vec, stream);
  else launch_row_mode<E, MODE_GREEDY>(a, B, vec, stream);
}

// Launch the walk in request batches whose workgroups all fit on the device
// at once, so the workgroups of a request never wait for one another's
// residency (the waits are bounded regardless).
tv_status launch_walk(WalkArgs a, int B, hipStream_t stream) {
  const bool vec = (a.V & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0 &&
                   (a.mode != MODE_MSS || (reinterpret_cast<uintptr_t>(a.ssm) & 15) == 0);
  if (a.V <= kRowThreads * kRowMaxE) {     // one workgroup per request
    a.b0 = 0;
    if (a.V <= kRowThreads * 8) launch_row<8>(a, B, vec, stream);
    else if (a.V <= kRowThreads * 16) launch_row<16>(a, B, vec, stream);
    else launch_row<32>(a, B, vec, stream);
    return tv::launch_status();
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TV_EHIP;
  const int cus = device_cus(dev);
  if (cus <= 0) return TV_EHIP;
  const int variant = a.mode != MODE_MSS ? a.mode : (a.multi ? 4 : (a.commit ? 3 : MODE_MSS));
  // Greedy passes are light (a max and an argmax, no normaliser), so its
  // walk keeps 8 entries per thread: measured, 4 or 16 only made it slower.
  int E = a.mode == MODE_GREEDY ? 8 : 0;
  for (int e = 4; e <= 16 && !E; e *= 2) {
    const int g = slice_groups(a.V, e);
    if (g <= kMaxG && static_cast<long>(B) * g <= cus) E = e;
  }
  if (!E) {
    long best = 0;
    for (int e = 16; e >= 4; e /= 2) {
      const int g = slice_groups(a.V, e);
      const int cap = walk_capacity(dev, variant, vec, e);
      if (cap <= 0) return TV_EHIP;
      if (g > kMaxG || g > cap) continue;
      const long per = cap / g, launches = (B + per - 1) / per;
      if (!E || launches < best) {
        E = e;
        best = launches;
      }
    }
    if (!E) return TV_EINVAL;
  }
  const int G = slice_groups(a.V, E);            // <= ws_groups(V): the workspace holds it
  a.G = G;
  const int capacity = walk_capacity(dev, variant, vec, E);
  if (capacity <= 0) return TV_EHIP;
  if (G > capacity) return TV_EINVAL;
  const int per_launch = capacity / G;
  for (int b0 = 0; b0 < B; b0 += per_launch) {
    const int nb = std::min(per_launch, B - b0);
    a.b0 = b0;
    launch_sliced(a, nb * G, vec, E, stream);
    if (hipGetLastError() != hipSuccess) return TV_EHIP;
  }
  return TV_OK;
}

// The wait bound of the sliced walk's exchanges: kSpinLimit polls, or the
// value of TREEVERIFY_WALK_WAIT_POLLS (a decimal count; 0 makes every wait
// give up at once, which tests the time-out path without a hang).
unsigned wait_limit() {
  const char* e = std::getenv("TREEVERIFY_WALK_WAIT_POLLS");
  if (e && *e) {
    char* end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    if (end && *end == '\0') return static_cast<unsigned>(std::min<unsigned long>(v, kSpinLimit));
  }
  return kSpinLimit;
}

WalkArgs make_args(int mode, int N, int V, int R, void* workspace, int B) {
  WalkArgs a{};
  a.mode = mode;
  a.spin_limit = wait_limit();
  a.N = N;
  a.V = V;
  a.R = R;
  a.G = 0;                  // set by launch_walk with the slice width
  const WsLayout w = ws_layout(B, V);
  uint8_t* p = static_cast<uint8_t*>(workspace);
  a.done = reinterpret_cast<uint32_t*>(p);
  a.hdr = reinterpret_cast<uint64_t*>(p + w.off_hdr);
  a.kid = reinterpret_cast<uint64_t*>(p + w.off_kid);
  return a;
}

}  // namespace

extern "C" size_t tree_verify_workspace(int B, int N, int V) {
  if (check_verify_args(B, N, V) != TV_OK || B == 0) return 0;
  return ws_layout(B, V).total;
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
  if (!workspace || ws_bytes < ws_layout(B, V).total) return TV_EWORKSPACE;
  WalkArgs a = make_args(MODE_GREEDY, N, V, 1, workspace, B);
  a.logits = target_logits;
  a.token = token;
  a.child = child;
  a.status = status;
  a.accepted = accepted;
  a.num_accepted = num_accepted;
  a.bonus = bonus;
  return launch_walk(a, B, stream);
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
  if (!workspace || ws_bytes < ws_layout(B, V).total) return TV_EWORKSPACE;
  WalkArgs a = make_args(MODE_MSS, N, V, R, workspace, B);
  a.logits = target_logits;
  a.ssm = ssm_probs;
  a.q_row = q_row;
  a.token = token;
  a.child = child;
  a.status = status;
  a.seed = seed;
  a.offset = offset;
  a.accepted = accepted;
  a.num_accepted = num_accepted;
  a.bonus = bonus;
  a.rounds = rounds;
  return launch_walk(a, B, stream);
}

extern "C" tv_status tree_verify_mss_commit(int B, int N, int V, int R, const float* target_logits,
                                            const float* ssm_probs, const int32_t* q_row, const int32_t* token,
                                            const uint64_t* child, int32_t* status, uint64_t seed,
                                            uint64_t offset, int32_t* accepted, int32_t* num_accepted,
                                            int32_t* bonus, int32_t* rounds, void* workspace, size_t ws_bytes,
                                            tv_dtype kv_dtype, int H, int D, void* k_cache, void* v_cache,
                                            int num_blocks, int block_size, const int32_t* block_table,
                                            int max_blocks, int32_t* prefix_len, hipStream_t stream) {
  const tv_status c = check_verify_args(B, N, V);
  if (c != TV_OK) return c;
  if (kv_dtype != TV_F32 && kv_dtype != TV_BF16) return TV_EDTYPE;
  if (R < 1 || H < 1 || (D != 64 && D != 128) || block_size != TV_BLOCK || max_blocks < 1 || num_blocks < 1)
    return TV_EINVAL;
  if (B == 0) return TV_OK;
  if (!target_logits || !ssm_probs || !child || !status || !num_accepted || !bonus ||
      (N > 0 && (!token || !accepted || !q_row)))
    return TV_EINVAL;
  if (!k_cache || !v_cache || !block_table || !prefix_len) return TV_EINVAL;
  if (!workspace || ws_bytes < ws_layout(B, V).total) return TV_EWORKSPACE;
  WalkArgs a = make_args(MODE_MSS, N, V, R, workspace, B);
  a.logits = target_logits;
  a.ssm = ssm_probs;
  a.q_row = q_row;
  a.token = token;
  a.child = child;
  a.status = status;
  a.seed = seed;
  a.offset = offset;
  a.accepted = accepted;
  a.num_accepted = num_accepted;
  a.bonus = bonus;
  a.rounds = rounds;
  a.commit = true;
  a.kv.H = H;
  a.kv.D = D;
  a.kv.elem = kv_dtype == TV_BF16 ? 2 : 4;
  a.kv.kc = static_cast<uint8_t*>(k_cache);
  a.kv.vc = static_cast<uint8_t*>(v_cache);
  a.kv.num_blocks = num_blocks;
  a.kv.block_table = block_table;
  a.kv.max_blocks = max_blocks;
  a.kv.prefix_len = prefix_len;
  return launch_walk(a, B, stream);
}

extern "C" tv_status tree_verify_mss_multi(int B, int N, int S, int V, int R, const float* target_logits,
                                           const float* ssm_probs, const int32_t* prop_node,
                                           const int32_t* prop_row, const int32_t* token, const uint64_t* child,
                                           int32_t* status, uint64_t seed, uint64_t offset, int32_t* accepted,
                                           int32_t* num_accepted, int32_t* bonus, int32_t* rounds, void* workspace,
                                           size_t ws_bytes, hipStream_t stream) {
  const tv_status c = check_verify_args(B, N, V);
  if (c != TV_OK) return c;
  if (S < 0 || S > TV_MAX_NODES) return S < 0 ? TV_EINVAL : TV_ETOOBIG;
  if (R < 1) return TV_EINVAL;
  if (B == 0) return TV_OK;
  if (!target_logits || !ssm_probs || !child || !status || !num_accepted || !bonus ||
      (N > 0 && (!token || !accepted)) || (S > 0 && (!prop_node || !prop_row)))
    return TV_EINVAL;
  if (!workspace || ws_bytes < ws_layout(B, V).total) return TV_EWORKSPACE;
  WalkArgs a = make_args(MODE_MSS, N, V, R, workspace, B);
  a.logits = target_logits;
  a.ssm = ssm_probs;
  a.token = token;
  a.child = child;
  a.status = status;
  a.seed = seed;
  a.offset = offset;
  a.accepted = accepted;
  a.num_accepted = num_accepted;
  a.bonus = bonus;
  a.rounds = rounds;
  a.multi = true;
  a.S = S;
  a.prop_node = prop_node;
  a.prop_row = prop_row;
  return launch_walk(a, B, stream);
}

extern "C" tv_status tree_verify_naive(int B, int N, int V, const float* target_logits,
                                       const int32_t* token, const uint64_t* child, int32_t* status,
                                       uint64_t seed, uint64_t offset, int32_t* accepted,
                                       int32_t* num_accepted, int32_t* bonus, void* workspace,
                                       size_t ws_bytes, hipStream_t stream) {
  const tv_status c = check_verify_args(B, N, V);
  if (c != TV_OK) return c;
  if (B == 0) return TV_OK;
  if (!target_logits || !child || !status || !num_accepted || !bonus ||
      (N > 0 && (!token || !accepted)))
    return TV_EINVAL;
  if (!workspace || ws_bytes < ws_layout(B, V).total) return TV_EWORKSPACE;
  WalkArgs a = make_args(MODE_NAIVE, N, V, 1, workspace, B);
  a.logits = target_logits;
  a.token = token;
  a.child = child;
  a.status = status;
  a.seed = seed;
  a.offset = offset;
  a.accepted = accepted;
  a.num_accepted = num_accepted;
  a.bonus = bonus;
  return launch_walk(a, B, stream);
}

// ---------------------------------------------------------------------------
// tree_verify_mss_noalloc: tree_verify_mss with its workspace in a fixed
// device array of the library instead of a caller's buffer.
//
// `scratch` holds the exchange words of the sliced walk exactly as a caller's
// workspace would (same layout, same all-zero rule between calls).  Each
// device holds its own copy at its own address, so host code never passes the
// array's name to a kernel: the first call on a device (that device current)
// looks its address up with hipGetSymbolAddress and keeps it for the device,
// and launches a zero fill of the array on the call's stream ahead of the
// walk.  From then on every completed walk leaves the words zero, as with a
// caller's workspace.  A first call made while its stream is being captured
// records the fill in the graph and is not counted as the clearing one, so
// the next call outside a capture clears again.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[TV_NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void __launch_bounds__(256) scratch_fill_zero(uint4* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];       // the array's device address, per device
bool scratch_clear[kMaxDevices];      // a zero fill has run outside a capture

tv_status scratch_for_device(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TV_EINVAL;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TV_EHIP;
    scratch_ptr[dev] = p;
  }
  if (!scratch_clear[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return TV_EHIP;
    const size_t n = TV_NOALLOC_SCRATCH_BYTES / sizeof(uint4);
    hipLaunchKernelGGL(scratch_fill_zero, dim3(256), dim3(256), 0, stream,
                       static_cast<uint4*>(scratch_ptr[dev]), n);
    if (hipGetLastError() != hipSuccess) return TV_EHIP;
    scratch_clear[dev] = cs == hipStreamCaptureStatusNone;
  }
  *out = scratch_ptr[dev];
  return TV_OK;
}

}  // namespace

extern "C" tv_status tree_verify_mss_noalloc(int B, int N, int V, int R, const float* target_logits,
                                             const float* ssm_probs, const int32_t* q_row, const int32_t* token,
                                             const uint64_t* child, int32_t* status, uint64_t seed,
                                             uint64_t offset, int32_t* accepted, int32_t* num_accepted,
                                             int32_t* bonus, int32_t* rounds, hipStream_t stream) {
  const tv_status c = check_verify_args(B, N, V);
  if (c != TV_OK) return c;
  if (R < 1) return TV_EINVAL;
  if (B == 0) return TV_OK;
  if (!target_logits || !ssm_probs || !child || !status || !num_accepted || !bonus ||
      (N > 0 && (!token || !accepted || !q_row)))
    return TV_EINVAL;
  const size_t need = ws_layout(B, V).total;
  if (need > TV_NOALLOC_SCRATCH_BYTES) return TV_ESCRATCH;
  void* ws = nullptr;
  const tv_status s = scratch_for_device(stream, &ws);
  if (s != TV_OK) return s;
  return tree_verify_mss(B, N, V, R, target_logits, ssm_probs, q_row, token, child, status, seed, offset,
                         accepted, num_accepted, bonus, rounds, ws, need, stream);
}
