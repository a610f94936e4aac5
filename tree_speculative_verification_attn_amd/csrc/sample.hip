// tree_logits_transform: temperature, top-k and top-p on rows of logits.
//
// Wiki concept page "Speculative decoding", "Implementation sketch": the
// lossless acceptance rule holds for the sampling distributions, so
// temperature, top-k and top-p are applied to both the target's and the
// draft's distribution before verification.  The scaled logit of entry x is
// the fp32 product l'(x) = l(x) * fp32(1/T); top-k keeps the k largest l'
// (ties to the lower index), top-p then keeps the smallest prefix of that
// order whose mass reaches p times the mass top-k kept.  The kept set is
// therefore {x : l'(x) > v} plus {x : l'(x) = v, x <= c} for a cut value v and
// index c.
//
// One workgroup per row, in three layouts: rows of up to 32768 entries in
// the registers of 512 threads; such rows staged in LDS by 1024 threads where
// the register kernel has no short path; longer rows read from memory on
// every pass.  Top-k first bounds its cut from below with no pass of its own:
// in each wave, the ceil(k/8)-th largest of the lanes' maxima has ceil(k/8)
// entries at or above it (one per lane), so the smallest of these over the 8
// waves of a 512-thread workgroup (16 of a 1024-thread one, with ceil(k/16))
// has at least k entries at or above it and cannot exceed the cut value.  The
// entries above the bound go to a list of (index, value) pairs in LDS.  A list
// of at most 512 kept entries is cut exactly by ranking: each entry's rank in
// the order (value descending, index ascending), counted by all threads at
// once, and the first rank whose count or prefix of masses reaches the
// target.  Otherwise (top-p alone, a large k, a list that overflows) each cut
// is found without sorting: a pass histograms the candidates into 256 bins
// that are linear in the value over the current value range, the bin where
// the cumulative weight (count, or mass in fixed point) crosses the target
// becomes the next range, and a few such levels isolate the cut value; ties at
// the cut are split by bisection over the index.  Bins linear in the value
// spread logits over many bins, so the LDS atomics rarely collide (bins over
// the key bits would put almost every logit into a handful of exponent bins).
// Once such a search's candidates fit the list, its later levels scan the
// list instead of the row.  Masses are accumulated as 32.32 fixed point
// integers, so every sum, and every decision taken from one, is the same on
// every run.
#include "tv_common.h"

#include <atomic>

namespace {

// Rows are read and written once in the hot passes: those accesses carry the
// non-temporal hint (measured 4-8% faster on the LLaMA-65B layer's rows).
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTfBins = 256;
constexpr int kTfList = 4096;                 // candidate list capacity (32 KB of LDS)
constexpr int kRgThreads = 512;               // threads of the register kernel
constexpr int kRgQuad = 4 * kRgThreads;       // entries per register quad (2048)
constexpr int kRgMaxE = 64;                   // registers per thread: rows up to 32768 entries
constexpr int kStThreads = 1024;              // threads of the streaming and staged kernels
constexpr int kStaged = -1;                   // E of the kernel that stages the row in LDS
constexpr int kStagedMax = 32768;             // its longest row (128 KB of LDS)
constexpr int kTfLevels = 6;                  // linear-bin levels before exact bisection
constexpr double kFix = 4294967296.0;         // masses in [0, 1] as multiples of 2^-32

struct TfArgs {
  int V;
  const float* in;
  float* out;
  float inv_t;
  int top_k;
  double top_p;
  int probs;
  int vec;                    // V % 4 == 0 and both arrays 16-byte aligned: 16-byte accesses
};

// Order-preserving key of a float (-0 is taken as +0).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// E > 0: the row in registers, E entries per thread of 512 (entry x in
// thread (x mod 2048) / 4, register 4 (x / 2048) + x mod 4, so each load or
// store instruction of a wave covers 1 KB of contiguous row); entries past V
// hold -inf, which no step keeps or counts.  Only the hot passes read the
// registers (the load, the listing above the top-k bound, the output); a
// search that needs the whole row again first writes the scaled row to the
// output row, which the output pass overwrites at the end, and reads it from
// there.  E = 0: 1024 threads, thread t owns entries t, t + 1024, ..., read
// from the input row and scaled on every full pass.  E = kStaged: the same
// threads, with the scaled row staged in LDS once (for the searches the
// register kernel does not shortcut: top-p alone, top-k above 256, a whole
// row of probabilities); the list then keeps only indices.  Either way the
// code of the searches exists once, so the kernel fits the instruction cache.
template <int E>
__global__ __launch_bounds__(E > 0 ? kRgThreads : kStThreads) __attribute__((amdgpu_waves_per_eu(E == 0 ? 8 : 4)))
void transform_kernel(TfArgs a) {
  constexpr int NT = E > 0 ? kRgThreads : kStThreads;
  constexpr int NW = NT / 64;
  constexpr int kLV = E < 0 ? 1 : kTfList;           // list values kept (E < 0: read from the row)
  constexpr int kSmall = E < 0 ? 512 : NT;           // longest list the ranking search takes
  static_assert(E == kStaged || (E >= 0 && E % 4 == 0 && E <= kRgMaxE), "entries per thread");
  extern __shared__ float s_row[];                   // E < 0: the scaled row
  __shared__ uint32_t s_cnt[kTfBins];
  __shared__ unsigned long long s_mass[kTfBins];
  __shared__ double s_rd[2][NW];
  __shared__ float s_rmx[2][NW], s_rmn[2][NW];
  __shared__ int s_ri[2][NW];
  __shared__ int s_bin, s_inbin, s_n;
  __shared__ double s_above;
  __shared__ int s_lx[kTfList];               // candidate list: entry indices
  __shared__ float s_lv[kLV];                 //   and their scaled logits
  __shared__ int s_sx[kSmall];                // a short list in rank order: indices
  __shared__ float s_sv[kSmall];              //   and values
  __shared__ int s_rk[kSmall];                // ranks being summed
  __shared__ double s_wsum[NW];
  __shared__ int s_first;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int V = a.V;
  const float* src = a.in + static_cast<size_t>(blockIdx.x) * V;
  float* dst = a.out + static_cast<size_t>(blockIdx.x) * V;
  int bank = 0;

  float r[E > 0 ? E : 1];                     // E > 0: the row's scaled logits
  auto xof = [&](int e) __attribute__((always_inline)) { return (e >> 2) * kRgQuad + 4 * t + (e & 3); };
  // A register pass reads each entry and its index through an empty asm:
  // values derived from them then cannot be shared with another pass, which
  // would keep E of each alive.
  auto fresh = [](auto v) {
    asm volatile("" : "+v"(v));
    return v;
  };
  // Full passes over memory read row[x] * scale: the input row and 1/T, or
  // (E > 0, once written) the output row, which holds the scaled logits.
  const float* row = src;
  float scale = E < 0 ? 1.0f : a.inv_t;
  auto L = [&](int x) __attribute__((always_inline)) {
    if constexpr (E < 0) return s_row[x];
    else return row[x] * scale;
  };

  // ---- workgroup reductions (one barrier each, alternating banks) ----
  auto bsum = [&](double v) __attribute__((always_inline)) {
    v = tv::wave_sum_dpp(v);
    if (lane == 0) s_rd[bank][wave] = v;
    __syncthreads();
    const double s = tv::wave_sum_dpp(lane < NW ? s_rd[bank][lane] : 0.0);
    bank ^= 1;
    return s;
  };
  auto bminmax = [&](float& mn, float& mx, int& f) __attribute__((always_inline)) {
    mx = tv::wave_max_dpp(mx);
    mn = -tv::wave_max_dpp(-mn);
    f = tv::wave_or_dpp(f);
    if (lane == 0) {
      s_rmx[bank][wave] = mx;
      s_rmn[bank][wave] = mn;
      s_ri[bank][wave] = f;
    }
    __syncthreads();
    mx = tv::wave_max_dpp(lane < NW ? s_rmx[bank][lane] : -INFINITY);
    mn = -tv::wave_max_dpp(lane < NW ? -s_rmn[bank][lane] : -INFINITY);
    f = tv::wave_or_dpp(lane < NW ? s_ri[bank][lane] : 0);
    bank ^= 1;
  };

  // ---- load, range, validity ----
  float mn = INFINITY, mx = -INFINITY;
  int bad = 0;
  double nfin = 0.0;
  auto see = [&](float l) __attribute__((always_inline)) {
    if (l != l || l == INFINITY) {
      bad = 1;
    } else if (l != -INFINITY) {
      mx = fmaxf(mx, l);
      mn = fminf(mn, l);
      nfin += 1.0;
    }
  };
  if constexpr (E > 0) {
    if (a.vec) {
#pragma unroll
      for (int j = 0; j < E / 4; ++j) {
        const int x = j * kRgQuad + 4 * t;
        v4f f = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (x < V) f = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + x));
        r[4 * j] = f.x * a.inv_t;
        r[4 * j + 1] = f.y * a.inv_t;
        r[4 * j + 2] = f.z * a.inv_t;
        r[4 * j + 3] = f.w * a.inv_t;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int x = xof(e);
        r[e] = x < V ? src[x] * a.inv_t : -INFINITY;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) see(r[e]);
  } else if (a.vec) {
#pragma unroll 4
    for (int x = 4 * t; x < V; x += 4 * NT) {
      float4 f = *reinterpret_cast<const float4*>(src + x);
      f.x *= a.inv_t;
      f.y *= a.inv_t;
      f.z *= a.inv_t;
      f.w *= a.inv_t;
      if constexpr (E < 0) *reinterpret_cast<float4*>(s_row + x) = f;
      see(f.x);
      see(f.y);
      see(f.z);
      see(f.w);
    }
  } else {
#pragma unroll 4
    for (int x = t; x < V; x += NT) {
      const float l = src[x] * a.inv_t;
      if constexpr (E < 0) s_row[x] = l;
      see(l);
    }
  }
  const float tmax = mx;         // this thread's largest finite entry (-inf if none)
  bminmax(mn, mx, bad);
  nfin = bsum(nfin);
  if (bad || nfin == 0.0) {      // invalid row: every entry NaN
    for (int x = t; x < V; x += NT) dst[x] = __builtin_nanf("");
    return;
  }
  const float row_lo = mn, row_hi = mx;

  // kept set: finite l' and (l' > cut_v or (l' == cut_v and x <= cut_x))
  float cut_v = -INFINITY;
  int cut_x = V;
  auto kept = [&](float l, int x) __attribute__((always_inline)) { return l != -INFINITY && (l > cut_v || (l == cut_v && x <= cut_x)); };
  auto mass = [&](float l) __attribute__((always_inline)) { return tv::exp_acc(l - mx); };
  auto mfix = [&](float l) __attribute__((always_inline)) { return static_cast<unsigned long long>(static_cast<double>(mass(l)) * kFix); };

  // E > 0: the scaled row goes to the output row when the general path
  // takes over (every thread calls this at the same point).
  auto spill = [&]() __attribute__((always_inline)) {
    if constexpr (E > 0) {
      if (a.vec) {
#pragma unroll
        for (int j = 0; j < E / 4; ++j) {
          const int x = fresh(j * kRgQuad + 4 * t);
          if (x < V) *reinterpret_cast<float4*>(dst + x) = make_float4(r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int x = fresh(xof(e));
          if (x < V) dst[x] = r[e];
        }
      }
      __syncthreads();                       // the workgroup's writes are visible to it from here
      row = dst;
      scale = 1.0f;
    }
  };

  // Candidates: either every kept entry (full passes over the row) or the
  // kept entries among a list of at most kTfList (index, value) pairs in LDS.
  bool listed = false;        // candidates are the listed entries
  bool list_all = false;      // ... and the list holds every kept entry
  bool list_exact = false;    // ... every listed entry is kept, and every kept entry
                              //     above the cut being searched is listed
  int nlist = 0;
  auto lv = [&](int i) __attribute__((always_inline)) {    // value of list entry i
    if constexpr (E < 0) return s_row[s_lx[i]];
    else return s_lv[i];
  };
  auto for_cands = [&](auto&& fn) __attribute__((always_inline)) {
    if (listed) {
      for (int i = t; i < nlist; i += NT) {
        const int x = s_lx[i];
        const float l = lv(i);
        if (kept(l, x)) fn(l, x);
      }
    } else {                                  // (E > 0: after the spill)
#pragma unroll 4
      for (int x = t; x < V; x += NT) {
        const float l = L(x);
        if (kept(l, x)) fn(l, x);
      }
    }
  };
  // Wave-aggregated append of (x, l) to the list where c holds (every lane
  // of the wave calls it; appends past kTfList only count).
  auto append = [&](bool c, int x, float l) __attribute__((always_inline)) {
    const uint64_t m = __ballot(c);
    if (m) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_n, __builtin_popcountll(m));
      base = __shfl(base, 0);
      const int i = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
      if (c && i < kTfList) {
        s_lx[i] = x;
        if constexpr (E >= 0) s_lv[i] = l;
      }
    }
  };
  auto list_begin = [&]() __attribute__((always_inline)) {
    __syncthreads();                          // every read of the last list is done
    if (t == 0) s_n = 0;
    __syncthreads();
  };
  auto list_end = [&]() __attribute__((always_inline)) {
    __syncthreads();
    nlist = s_n;
    listed = nlist <= kTfList;                // if more qualify, the candidates stay the row
  };
  // List the row's entries with pred(l, x) (a pass over memory; E > 0:
  // after the spill).
  auto make_list = [&](auto&& pred) __attribute__((always_inline)) {
    list_begin();
    for (int x0 = t - lane; x0 < V; x0 += NT) {       // wave-uniform trip count
      const int x = x0 + lane;
      bool c = false;
      float l = 0.f;
      if (x < V) {
        l = L(x);
        c = pred(l, x);
      }
      append(c, x, l);
    }
    list_end();
  };
  // Drop the listed entries that are no longer kept (the list shrinks in
  // place: every thread reads its entries before any is rewritten).
  auto compact_list = [&]() __attribute__((always_inline)) {
    constexpr int PER = kTfList / NT;
    int xs[PER];
    float vs[PER];
    bool ks[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = q * NT + t;
      xs[q] = i < nlist ? s_lx[i] : 0;
      vs[q] = i < nlist ? lv(i) : -INFINITY;
      ks[q] = i < nlist && kept(vs[q], xs[q]);
    }
    list_begin();
#pragma unroll
    for (int q = 0; q < PER; ++q) append(ks[q], xs[q], vs[q]);
    list_end();
  };
  // Exact cut over a list of at most NT entries that are all kept: each
  // entry's rank in the order (value descending, index ascending), which is
  // the order the kept prefix follows, places it in s_sx/s_sv; the cut is the
  // first rank whose inclusive weight (count, or fixed-point mass) reaches
  // need.  The same cut as the bin search finds, in one pass over the list.
  auto select_small = [&](double need, bool use_mass) __attribute__((always_inline)) {
    const bool mine = t < nlist;
    if (mine) s_rk[t] = 0;
    if (t == 0) s_first = INT_MAX;
    __syncthreads();
    {
      // Candidate ci = t mod CW against part t / CW of the list: the
      // candidates padded to whole waves (CW), the list split into the
      // NT / CW parts the threads cover, so every wave works.  Each part is
      // read in chunks of 64, one entry per lane, every entry of a chunk
      // taken across lanes (no memory round trip per comparison).
      const int CW = (nlist + 63) & ~63;
      const int parts = NT / CW;
      const int part = t / CW, ci = t - part * CW;
      if (part < parts) {                     // (wave-uniform: CW is a multiple of 64)
        const int len = (nlist + parts - 1) / parts;
        const int j0 = part * len, j1 = min(nlist, j0 + len);
        const bool cand = ci < nlist;
        const int xi = cand ? s_lx[ci] : 0;
        const float vi = cand ? lv(ci) : -INFINITY;
        int rank = 0;
        for (int c0 = j0; c0 < j1; c0 += 64) {
          const int jj = c0 + lane;
          const float vc = jj < j1 ? lv(jj) : -INFINITY;
          const int xc = jj < j1 ? s_lx[jj] : 0;
          const int cnt = min(64, j1 - c0);
          for (int j = 0; j < cnt; ++j) {
            const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vc), j));
            const int xj = __builtin_amdgcn_readlane(xc, j);
            rank += (vj > vi || (vj == vi && xj < xi)) ? 1 : 0;
          }
        }
        if (cand && rank > 0) atomicAdd(&s_rk[ci], rank);
      }
    }
    __syncthreads();
    if (mine) {
      const int rank = s_rk[t];
      s_sx[rank] = s_lx[t];
      s_sv[rank] = lv(t);
    }
    __syncthreads();
    int r_cut = static_cast<int>(need) - 1;     // count: need = k <= nlist
    if (use_mass) {
      // inclusive prefix of the masses in rank order, rank t in thread t
      const double m = mine ? static_cast<double>(mfix(s_sv[t])) : 0.0;
      double excl;
      const double incl = tv::wave_scan_dpp(m, &excl);
      if (lane == 63) s_wsum[wave] = incl;
      __syncthreads();
      double base = 0.0;
      for (int w = 0; w < wave; ++w) base += s_wsum[w];
      const uint64_t hit = __ballot(mine && base + incl >= need);
      if (hit && lane == 0) atomicMin(&s_first, wave * 64 + __builtin_ctzll(hit));
      __syncthreads();
      r_cut = min(s_first, nlist - 1);          // (need <= the total: the last rank reaches it)
    }
    return r_cut;
  };

  // The cut where the weight (use_mass: fixed-point mass, else count) of the
  // candidates, taken in order, first reaches `need`; narrows the kept set.
  auto select = [&](double need, bool use_mass) __attribute__((always_inline)) {
    float v;
    int cx;
    if (listed && list_exact && nlist <= kSmall) {
      const int rc = select_small(need, use_mass);
      v = s_sv[rc];
      cx = s_sx[rc];
    } else {
      float lo = row_lo, hi = row_hi;       // with nothing cut, the candidates span the row
      if (listed || cut_v != -INFINITY) {
        float l0 = INFINITY, h0 = -INFINITY;
        int unused = 0;
        for_cands([&](float l, int) {
          l0 = fminf(l0, l);
          h0 = fmaxf(h0, l);
        });
        bminmax(l0, h0, unused);
        lo = l0;
        hi = h0;
      }
      double above = 0.0;            // weight of candidates above the range [lo, hi]
      for (int level = 0; level < kTfLevels && lo < hi; ++level) {
        const float s = static_cast<float>(kTfBins) / (hi - lo);
        if (!(s > 0.f) || s == INFINITY) break;
        for (int i = t; i < kTfBins; i += NT) {
          s_cnt[i] = 0u;
          s_mass[i] = 0ull;
        }
        __syncthreads();
        auto bin_of = [&](float l) __attribute__((always_inline)) { return min(kTfBins - 1, static_cast<int>((hi - l) * s)); };
        // (the choice is made outside the pass, so each pass is specialised)
        if (use_mass) {
          for_cands([&](float l, int) {
            if (l >= lo && l <= hi) {
              const int b = bin_of(l);
              atomicAdd(&s_cnt[b], 1u);
              atomicAdd(&s_mass[b], mfix(l));
            }
          });
        } else {
          for_cands([&](float l, int) {
            if (l >= lo && l <= hi) atomicAdd(&s_cnt[bin_of(l)], 1u);
          });
        }
        __syncthreads();
        if (wave == 0) {
          // bins in order (0 = largest values): the first whose inclusive
          // cumulative weight reaches need - above; else the last nonempty one
          double run = 0.0;
          int pick = -1, last = -1;
          double ex_pick = 0.0, ex_last = 0.0;
          for (int base = 0; base < kTfBins && pick < 0; base += 64) {
            const int b = base + lane;
            const double wgt = use_mass ? static_cast<double>(s_mass[b]) : static_cast<double>(s_cnt[b]);
            double excl;
            const double incl = run + tv::wave_scan_dpp(wgt, &excl);
            excl += run;
            const uint64_t hit = __ballot(s_cnt[b] > 0u && above + incl >= need);
            const uint64_t nz = __ballot(s_cnt[b] > 0u);
            if (hit) {
              const int l2 = __builtin_ctzll(hit);
              pick = base + l2;
              ex_pick = tv::readlane_f64(excl, l2);
            } else if (nz) {
              const int l2 = 63 - __builtin_clzll(nz);
              last = base + l2;
              ex_last = tv::readlane_f64(excl, l2);
            }
            run = tv::readlane_f64(incl, 63);
          }
          if (pick < 0) {
            pick = last;
            ex_pick = ex_last;
          }
          if (lane == 0) {
            s_bin = pick;
            s_above = above + ex_pick;
            s_inbin = static_cast<int>(s_cnt[pick]);
          }
        }
        __syncthreads();
        const int pb = s_bin;
        const int in_bin = s_inbin;
        above = s_above;
        // from the full row, a bin small enough goes to the candidate list
        if (!listed && in_bin <= kTfList) {
          const float lo0 = lo, hi0 = hi;
          make_list([&](float l, int x) { return kept(l, x) && l >= lo0 && l <= hi0 && bin_of(l) == pb; });
          list_exact = false;
          list_all = false;
        }
        // the picked bin's value range becomes the next range
        float l0 = INFINITY, h0 = -INFINITY;
        int unused = 0;
        for_cands([&](float l, int) {
          if (l >= lo && l <= hi && bin_of(l) == pb) {
            l0 = fminf(l0, l);
            h0 = fmaxf(h0, l);
          }
        });
        bminmax(l0, h0, unused);
        lo = l0;
        hi = h0;
      }
      auto weight_ge = [&](float v, float top) __attribute__((always_inline)) {       // candidates in [v, top]
        double c = 0.0;
        if (use_mass) {
          for_cands([&](float l, int) {
            if (l >= v && l <= top) c += static_cast<double>(mfix(l));
          });
        } else {
          for_cands([&](float l, int) {
            if (l >= v && l <= top) c += 1.0;
          });
        }
        return bsum(c);
      };
      if (lo < hi) {
        // exact bisection over the keys of [lo, hi]: the largest v with
        // above + weight(candidates in [v, hi]) >= need
        uint32_t klo = fkey(lo), khi = fkey(hi);
        while (klo < khi) {
          const uint32_t mid = klo + (khi - klo + 1) / 2;
          if (above + weight_ge(fkey_inv(mid), hi) >= need) klo = mid;
          else khi = mid - 1;
        }
        const float vk = fkey_inv(klo);
        if (vk < hi) above += weight_ge(fkey_inv(klo + 1), hi);
        lo = hi = vk;
      }
      // ties at the cut value: the lowest indices first
      v = lo;
      double c_eq = 0.0;
      for_cands([&](float l, int) {
        if (l == v) c_eq += 1.0;
      });
      c_eq = bsum(c_eq);
      double n_keep;
      if (use_mass) {
        const double m1 = static_cast<double>(mfix(v));
        n_keep = m1 > 0.0 ? ceil((need - above) / m1) : c_eq;
      } else {
        n_keep = need - above;
      }
      n_keep = fmin(fmax(n_keep, 1.0), c_eq);
      cx = V;                              // every tied entry kept, unless split below
      if (n_keep < c_eq) {
        int xlo = 0, xhi = V - 1;          // smallest X with n_keep tied candidates at or below it
        while (xlo < xhi) {
          const int mid = (xlo + xhi) / 2;
          double c = 0.0;
          for_cands([&](float l, int x) {
            if (l == v && x <= mid) c += 1.0;
          });
          if (bsum(c) >= n_keep) xhi = mid;
          else xlo = mid + 1;
        }
        cx = xlo;
      }
    }
    if (v == cut_v) cut_x = min(cut_x, cx);
    else cut_x = cx;
    cut_v = v;
  };

  // ---- top-k, then top-p over what top-k kept ----
  const bool do_k = a.top_k > 0 && static_cast<double>(a.top_k) < nfin;
  const bool do_p = a.top_p < 1.0;
  if (do_k) {
    const int kw = (a.top_k + NW - 1) / NW;     // entries each wave vouches for
    // (the list above the bound holds about twice top_k entries: used when
    // the ranking search can take it)
    if (kw <= 64 && 2 * a.top_k <= kSmall) {
      // this wave's kw-th largest lane maximum
      float t0;
      if (kw <= 16) {
        // take the wave maximum kw times, retiring one lane holding it each time
        float cur = tmax;
        for (int i = 0; i < kw; ++i) {
          t0 = tv::wave_max_dpp(cur);
          const uint64_t h = __ballot(cur == t0);
          if (lane == __builtin_ctzll(h)) cur = -INFINITY;
        }
      } else {
        // the lane of rank kw - 1 in the order (value descending, lane
        // ascending), which is a permutation
        int rank = 0;
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tmax), j));
          rank += (v > tmax || (v == tmax && j < lane)) ? 1 : 0;
        }
        const uint64_t hit = __ballot(rank == kw - 1);
        t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tmax), __builtin_ctzll(hit)));
      }
      float unused_hi = t0;
      int unused = 0;
      bminmax(t0, unused_hi, unused);            // t0: the smallest over the waves
      if (t0 > -INFINITY) {
        // nothing is cut yet, so the entries at or above t0 are kept ones
        if constexpr (E > 0) {
          list_begin();
#pragma unroll
          for (int j = 0; j < E / 4; ++j) {
            // one vote per 4 entries; the entries are appended only where one passes
            const float a0 = fresh(r[4 * j]), a1 = fresh(r[4 * j + 1]), a2 = fresh(r[4 * j + 2]),
                        a3 = fresh(r[4 * j + 3]);
            if (__any(a0 >= t0 || a1 >= t0 || a2 >= t0 || a3 >= t0)) {
              const int x = fresh(xof(4 * j));
              append(a0 >= t0, x, a0);
              append(a1 >= t0, x + 1, a1);
              append(a2 >= t0, x + 2, a2);
              append(a3 >= t0, x + 3, a3);
            }
          }
          list_end();
        } else {
          make_list([&](float l, int) { return l >= t0; });
        }
        list_exact = listed;
      }
    }
  }
  if constexpr (E > 0) {
    // The short path, with the row still in registers: top-k (and top-p on
    // what it kept) over the bound's list, or nothing to cut.
    const bool from_list = do_k && listed && list_exact && nlist <= NT;
    if (from_list || (!do_k && !do_p && !a.probs)) {
      if (from_list) {
        int rc = select_small(static_cast<double>(a.top_k), false);
        cut_v = s_sv[rc];
        cut_x = s_sx[rc];
        if (do_p) {
          compact_list();                        // the top_k kept entries (top_k <= NT)
          double zp = 0.0;
          for_cands([&](float l, int) { zp += static_cast<double>(mfix(l)); });
          rc = select_small(a.top_p * bsum(zp), true);
          const float v = s_sv[rc];
          const int cx = s_sx[rc];
          if (v == cut_v) cut_x = min(cut_x, cx);
          else cut_x = cx;
          cut_v = v;
        }
      }
      const bool nocut = cut_v == -INFINITY;
      if (!a.probs) {
        // scaled logits of the kept entries, -inf elsewhere
        auto write_logits = [&](auto&& keep) __attribute__((always_inline)) {
          if (a.vec) {
#pragma unroll
            for (int j = 0; j < E / 4; ++j) {
              const int x = fresh(j * kRgQuad + 4 * t);
              if (x < V) {
                float4 f;
                f.x = keep(fresh(r[4 * j]), x) ? r[4 * j] : -INFINITY;
                f.y = keep(fresh(r[4 * j + 1]), x + 1) ? r[4 * j + 1] : -INFINITY;
                f.z = keep(fresh(r[4 * j + 2]), x + 2) ? r[4 * j + 2] : -INFINITY;
                f.w = keep(fresh(r[4 * j + 3]), x + 3) ? r[4 * j + 3] : -INFINITY;
                __builtin_nontemporal_store(v4f{f.x, f.y, f.z, f.w}, reinterpret_cast<v4f*>(dst + x));
              }
            }
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const int x = fresh(xof(e));
              if (x < V) dst[x] = keep(fresh(r[e]), x) ? r[e] : -INFINITY;
            }
          }
        };
        if (nocut) write_logits([](float, int) __attribute__((always_inline)) { return true; });   // (-inf stays -inf)
        else write_logits([&](float l, int x) __attribute__((always_inline)) { return l > cut_v || (l == cut_v && x <= cut_x); });
        return;
      }
      // probabilities: zeros, then the kept entries, all of which are listed
      double z = 0.0;
      for_cands([&](float l, int) { z += static_cast<double>(mass(l)); });
      z = bsum(z);
      if (a.vec) {
#pragma unroll
        for (int j = 0; j < E / 4; ++j) {
          const int x = fresh(j * kRgQuad + 4 * t);
          if (x < V) *reinterpret_cast<float4*>(dst + x) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int x = fresh(xof(e));
          if (x < V) dst[x] = 0.f;
        }
      }
      __syncthreads();                           // the zeros land before the entries that replace them
      for (int i = t; i < nlist; i += NT) {
        const int x = s_lx[i];
        const float l = s_lv[i];
        if (kept(l, x)) dst[x] = static_cast<float>(static_cast<double>(mass(l)) / z);
      }
      return;
    }
    spill();                                     // from here on the row is read from memory
  }

  // The general path (over memory).  One search serves both stages (its
  // code exists once).
#pragma nounroll
  for (int stage = do_k ? 0 : 1; stage < (do_p ? 2 : 1); ++stage) {
    double need = static_cast<double>(a.top_k);
    if (stage == 1) {
      if (do_k) {
        // the kept set is now top_k entries: list them
        if (a.top_k <= kTfList) {
          if (listed && list_exact) compact_list();      // they are all in the list
          else make_list([&](float l, int x) __attribute__((always_inline)) { return kept(l, x); });
          list_all = listed;
          list_exact = listed;
        } else {
          listed = false;
        }
      }
      double z = 0.0;
      for_cands([&](float l, int) { z += static_cast<double>(mfix(l)); });
      need = a.top_p * bsum(z);
    }
    select(need, stage == 1);
  }

  // ---- output ----
  if (!list_all) listed = false;     // the normaliser needs every kept entry
  double z = 1.0;
  if (a.probs) {
    z = 0.0;
    for_cands([&](float l, int) { z += static_cast<double>(mass(l)); });
    z = bsum(z);
  }
  const bool nocut = cut_v == -INFINITY;
  // from memory: each thread reads and writes the same entries
  auto out_of = [&](float l, int x) __attribute__((always_inline)) {
    const bool k = nocut ? l != -INFINITY : (l > cut_v || (l == cut_v && x <= cut_x));
    if (a.probs) return k ? static_cast<float>(static_cast<double>(mass(l)) / z) : 0.f;
    return k ? l : -INFINITY;
  };
  if (a.vec) {
#pragma unroll 4
    for (int x = 4 * t; x < V; x += 4 * NT) {
      float4 f = E < 0 ? *reinterpret_cast<const float4*>(s_row + x) : *reinterpret_cast<const float4*>(row + x);
      f.x = out_of(f.x * scale, x);
      f.y = out_of(f.y * scale, x + 1);
      f.z = out_of(f.z * scale, x + 2);
      f.w = out_of(f.w * scale, x + 3);
      __builtin_nontemporal_store(v4f{f.x, f.y, f.z, f.w}, reinterpret_cast<v4f*>(dst + x));
    }
  } else {
#pragma unroll 4
    for (int x = t; x < V; x += NT) dst[x] = out_of(L(x), x);
  }
}

}  // namespace

extern "C" tv_status tree_logits_transform(int rows, int V, const float* in, float* out,
                                           float temperature, int top_k, float top_p, int out_kind,
                                           hipStream_t stream) {
  if (rows < 0 || V < 1 || V > (1 << 20) || !(temperature > 0.f) || temperature == INFINITY ||
      top_k < 0 || !(top_p > 0.f && top_p <= 1.f) || (out_kind != TV_OUT_LOGITS && out_kind != TV_OUT_PROBS))
    return TV_EINVAL;
  if (rows == 0) return TV_OK;
  if (!in || !out) return TV_EINVAL;
  TfArgs a;
  a.V = V;
  a.in = in;
  a.out = out;
  a.inv_t = 1.0f / temperature;
  a.top_k = top_k;
  a.top_p = static_cast<double>(top_p);
  a.probs = out_kind == TV_OUT_PROBS;
  a.vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(in) & 15) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  // The register kernel where its short path applies (top-k of at most 256,
  // whose list above the bound the ranking search takes, or no cut at all),
  // and for rows of up to 8192 entries, whose spill to memory costs less than
  // staging; else the row staged in LDS; else (longer rows) streamed.
  const bool short_path = (top_k >= 1 && 2 * top_k <= kRgThreads) || (top_k == 0 && top_p >= 1.f && !a.probs);
  const dim3 grid(rows), rg(kRgThreads), st(kStThreads);
  if ((short_path || V <= 4 * kRgQuad) && V <= 16 * kRgQuad) {
    if (V <= 2 * kRgQuad) hipLaunchKernelGGL(transform_kernel<8>, grid, rg, 0, stream, a);
    else if (V <= 4 * kRgQuad) hipLaunchKernelGGL(transform_kernel<16>, grid, rg, 0, stream, a);
    else if (V <= 8 * kRgQuad) hipLaunchKernelGGL(transform_kernel<32>, grid, rg, 0, stream, a);
    else hipLaunchKernelGGL(transform_kernel<64>, grid, rg, 0, stream, a);
  } else if (V <= kStagedMax) {
    // the kernel's dynamic LDS limit is raised once per device (a repeated
    // call from another thread sets the same value)
    static std::atomic<bool> lds_ok[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TV_EHIP;
    if (dev < 0 || dev >= 64 || !lds_ok[dev].load(std::memory_order_acquire)) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(transform_kernel<kStaged>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(kStagedMax * sizeof(float))) != hipSuccess)
        return TV_EHIP;
      if (dev >= 0 && dev < 64) lds_ok[dev].store(true, std::memory_order_release);
    }
    const size_t row_bytes = static_cast<size_t>((V + 3) / 4 * 4) * sizeof(float);
    hipLaunchKernelGGL(transform_kernel<kStaged>, grid, st, row_bytes, stream, a);
  } else {
    hipLaunchKernelGGL(transform_kernel<0>, grid, st, 0, stream, a);
  }
  return tv::launch_status();
}
