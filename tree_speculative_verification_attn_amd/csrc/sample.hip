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
// One workgroup of 1024 threads per row; a row of up to 32768 entries is
// staged in LDS as scaled logits once, a longer one is re-read from memory on
// every pass.  After the first histogram level the candidates (the picked
// bin's entries, or the top-k survivors for the top-p stage) usually fit a
// list of 4096 indices in LDS, and the remaining levels, tie counts and the
// top-p stage scan that list instead of the row.  Each cut is found without sorting: a pass histograms the
// candidates into 256 bins that are linear in the value over the current
// value range, the bin where the cumulative weight (count, or mass in fixed
// point) crosses the target becomes the next range, and a few such levels
// isolate the cut value; ties at the cut are split by bisection over the
// index.  Bins linear in the value spread logits over many bins, so the LDS
// atomics rarely collide (bins over the key bits would put almost every logit
// into a handful of exponent bins).  Masses are accumulated as 32.32 fixed
// point integers, so every sum, and every decision taken from one, is the same
// on every run.
#include "tv_common.h"

namespace {

constexpr int kTfThreads = 1024;
constexpr int kTfWaves = kTfThreads / 64;
constexpr int kTfBins = 256;
constexpr int kTfLdsMax = 32768;              // floats staged in LDS (128 KB)
constexpr int kTfList = 4096;                 // candidate list capacity (16 KB of LDS)
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

template <bool LDS>
__global__ __launch_bounds__(kTfThreads) void transform_kernel(TfArgs a) {
  // dynamic LDS: the staged row (LDS = true, V floats rounded up to 4) and
  // then the candidate list (kTfList entry indices)
  extern __shared__ float s_dyn[];
  __shared__ uint32_t s_cnt[kTfBins];
  __shared__ unsigned long long s_mass[kTfBins];
  __shared__ double s_rd[2][kTfWaves];
  __shared__ float s_rmx[2][kTfWaves], s_rmn[2][kTfWaves];
  __shared__ int s_ri[2][kTfWaves];
  __shared__ int s_bin, s_inbin, s_n;
  __shared__ double s_above;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int V = a.V;
  const float* src = a.in + static_cast<size_t>(blockIdx.x) * V;
  float* dst = a.out + static_cast<size_t>(blockIdx.x) * V;
  float* s_row = s_dyn;
  int* s_list = reinterpret_cast<int*>(s_dyn + (LDS ? (V + 3) / 4 * 4 : 0));
  int bank = 0;

  auto L = [&](int x) -> float { return LDS ? s_row[x] : src[x] * a.inv_t; };

  // ---- workgroup reductions (one barrier each, alternating banks) ----
  auto bsum = [&](double v) {
    v = tv::wave_sum_dpp(v);
    if (lane == 0) s_rd[bank][wave] = v;
    __syncthreads();
    const double s = tv::wave_sum_dpp(lane < kTfWaves ? s_rd[bank][lane] : 0.0);
    bank ^= 1;
    return s;
  };
  auto bminmax = [&](float& mn, float& mx, int& f) {
    mx = tv::wave_max_dpp(mx);
    mn = -tv::wave_max_dpp(-mn);
    f = tv::wave_or_dpp(f);
    if (lane == 0) {
      s_rmx[bank][wave] = mx;
      s_rmn[bank][wave] = mn;
      s_ri[bank][wave] = f;
    }
    __syncthreads();
    mx = tv::wave_max_dpp(lane < kTfWaves ? s_rmx[bank][lane] : -INFINITY);
    mn = -tv::wave_max_dpp(lane < kTfWaves ? -s_rmn[bank][lane] : -INFINITY);
    f = tv::wave_or_dpp(lane < kTfWaves ? s_ri[bank][lane] : 0);
    bank ^= 1;
  };

  // ---- load (and stage), range, validity ----
  float mn = INFINITY, mx = -INFINITY;
  int bad = 0;
  double nfin = 0.0;
  auto see = [&](float l) {
    if (l != l || l == INFINITY) {
      bad = 1;
    } else if (l != -INFINITY) {
      mx = fmaxf(mx, l);
      mn = fminf(mn, l);
      nfin += 1.0;
    }
  };
  if (a.vec) {
#pragma unroll 4
    for (int x = 4 * t; x < V; x += 4 * kTfThreads) {
      float4 f = *reinterpret_cast<const float4*>(src + x);
      f.x *= a.inv_t;
      f.y *= a.inv_t;
      f.z *= a.inv_t;
      f.w *= a.inv_t;
      if (LDS) *reinterpret_cast<float4*>(s_row + x) = f;
      see(f.x);
      see(f.y);
      see(f.z);
      see(f.w);
    }
  } else {
#pragma unroll 4
    for (int x = t; x < V; x += kTfThreads) {
      const float l = src[x] * a.inv_t;
      if (LDS) s_row[x] = l;
      see(l);
    }
  }
  bminmax(mn, mx, bad);
  nfin = bsum(nfin);
  if (bad || nfin == 0.0) {      // invalid row: every entry NaN
    for (int x = t; x < V; x += kTfThreads) dst[x] = __builtin_nanf("");
    return;
  }

  // kept set: finite l' and (l' > cut_v or (l' == cut_v and x <= cut_x))
  float cut_v = -INFINITY;
  int cut_x = V;
  auto kept = [&](float l, int x) { return l != -INFINITY && (l > cut_v || (l == cut_v && x <= cut_x)); };
  auto mass = [&](float l) { return tv::exp_acc(l - mx); };
  auto mfix = [&](float l) { return static_cast<unsigned long long>(static_cast<double>(mass(l)) * kFix); };

  // Candidates: either every kept entry (full scans of the row) or the kept
  // entries among a list of at most kTfList indices in LDS.
  bool listed = false;        // candidates are the listed entries
  bool list_all = false;      // ... and the list holds every kept entry
  int nlist = 0;
  auto for_cands = [&](auto&& fn) {
    if (listed) {
      for (int i = t; i < nlist; i += kTfThreads) {
        const int x = s_list[i];
        const float l = L(x);
        if (kept(l, x)) fn(l, x);
      }
    } else {
#pragma unroll 4
      for (int x = t; x < V; x += kTfThreads) {
        const float l = L(x);
        if (kept(l, x)) fn(l, x);
      }
    }
  };
  // List the kept entries with pred(l) (a full scan; wave-aggregated appends).
  // If more than kTfList qualify, the candidates stay the full row.
  auto make_list = [&](auto&& pred) {
    __syncthreads();                          // every read of the last list length is done
    if (t == 0) s_n = 0;
    __syncthreads();
    for (int x0 = t - lane; x0 < V; x0 += kTfThreads) {     // wave-uniform trip count
      const int x = x0 + lane;
      bool c = false;
      if (x < V) {
        const float l = L(x);
        c = kept(l, x) && pred(l);
      }
      const uint64_t m = __ballot(c);
      if (m) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_n, __builtin_popcountll(m));
        base = __shfl(base, 0);
        const int i = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
        if (c && i < kTfList) s_list[i] = x;
      }
    }
    __syncthreads();
    nlist = s_n;
    listed = nlist <= kTfList;
  };

  // The cut where the weight (use_mass: fixed-point mass, else count) of the
  // candidates, taken in order, first reaches `need`; narrows the kept set.
  auto select = [&](double need, bool use_mass) {
    float lo, hi;
    {
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
      for (int i = t; i < kTfBins; i += kTfThreads) {
        s_cnt[i] = 0u;
        s_mass[i] = 0ull;
      }
      __syncthreads();
      auto bin_of = [&](float l) { return min(kTfBins - 1, static_cast<int>((hi - l) * s)); };
      for_cands([&](float l, int) {
        if (l >= lo && l <= hi) {
          const int b = bin_of(l);
          atomicAdd(&s_cnt[b], 1u);
          if (use_mass) atomicAdd(&s_mass[b], mfix(l));
        }
      });
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
        make_list([&](float l) { return l >= lo0 && l <= hi0 && bin_of(l) == pb; });
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
    auto weight_ge = [&](float v, float top) {       // candidates in [v, top]
      double c = 0.0;
      for_cands([&](float l, int) {
        if (l >= v && l <= top) c += use_mass ? static_cast<double>(mfix(l)) : 1.0;
      });
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
      const float v = fkey_inv(klo);
      if (v < hi) above += weight_ge(fkey_inv(klo + 1), hi);
      lo = hi = v;
    }
    // ties at the cut value: the lowest indices first
    const float v = lo;
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
    int cx = V;                          // every tied entry kept, unless split below
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
    if (v == cut_v) cut_x = min(cut_x, cx);
    else cut_x = cx;
    cut_v = v;
  };

  if (a.top_k > 0 && static_cast<double>(a.top_k) < nfin) {
    select(static_cast<double>(a.top_k), false);
    // the kept set is now top_k entries: list them for the top-p stage
    if (a.top_p < 1.0 && a.top_k <= kTfList) {
      make_list([](float) { return true; });
      list_all = listed;
    } else {
      listed = false;
    }
  }
  if (a.top_p < 1.0) {
    double z = 0.0;
    for_cands([&](float l, int) { z += static_cast<double>(mfix(l)); });
    z = bsum(z);
    select(a.top_p * z, true);
  }

  // ---- output ----
  if (!list_all) listed = false;     // the normaliser needs every kept entry
  double z = 1.0;
  if (a.probs) {
    z = 0.0;
    for_cands([&](float l, int) { z += static_cast<double>(mass(l)); });
    z = bsum(z);
  }
  auto out_of = [&](float l, int x) {
    if (a.probs) return kept(l, x) ? static_cast<float>(static_cast<double>(mass(l)) / z) : 0.f;
    return kept(l, x) ? l : -INFINITY;
  };
  if (a.vec) {
#pragma unroll 4
    for (int x = 4 * t; x < V; x += 4 * kTfThreads) {
      float4 f;
      if (LDS) {
        f = *reinterpret_cast<const float4*>(s_row + x);
      } else {
        f = *reinterpret_cast<const float4*>(src + x);
        f.x *= a.inv_t;
        f.y *= a.inv_t;
        f.z *= a.inv_t;
        f.w *= a.inv_t;
      }
      f.x = out_of(f.x, x);
      f.y = out_of(f.y, x + 1);
      f.z = out_of(f.z, x + 2);
      f.w = out_of(f.w, x + 3);
      *reinterpret_cast<float4*>(dst + x) = f;
    }
  } else {
#pragma unroll 4
    for (int x = t; x < V; x += kTfThreads) dst[x] = out_of(L(x), x);
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
  const size_t list_bytes = kTfList * sizeof(int);
  if (V <= kTfLdsMax) {
    static bool lds_ok = false;          // a function attribute: set once per process
    if (!lds_ok) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(transform_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(kTfLdsMax * sizeof(float) + list_bytes)) != hipSuccess)
        return TV_EHIP;
      lds_ok = true;
    }
    const size_t row_bytes = static_cast<size_t>((V + 3) / 4 * 4) * sizeof(float);
    hipLaunchKernelGGL(transform_kernel<true>, dim3(rows), dim3(kTfThreads), row_bytes + list_bytes, stream, a);
  } else {
    hipLaunchKernelGGL(transform_kernel<false>, dim3(rows), dim3(kTfThreads), list_bytes, stream, a);
  }
  return tv::launch_status();
}
