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
// One workgroup of 512 threads per row; a row of up to 36864 entries is
// staged in LDS as scaled logits once, a longer one is re-read from memory on
// every pass.  Each cut is found without sorting: a pass histograms the
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

constexpr int kTfThreads = 512;
constexpr int kTfWaves = kTfThreads / 64;
constexpr int kTfBins = 256;
constexpr int kTfLdsMax = 36864;              // floats staged in LDS (144 KB)
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
  extern __shared__ float s_row[];            // scaled logits (LDS = true)
  __shared__ uint32_t s_cnt[kTfBins];
  __shared__ unsigned long long s_mass[kTfBins];
  __shared__ double s_rd[2][kTfWaves];
  __shared__ float s_rmx[2][kTfWaves], s_rmn[2][kTfWaves];
  __shared__ int s_ri[2][kTfWaves];
  __shared__ int s_bin;
  __shared__ double s_above;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int V = a.V;
  const float* src = a.in + static_cast<size_t>(blockIdx.x) * V;
  float* dst = a.out + static_cast<size_t>(blockIdx.x) * V;
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
  for (int x = t; x < V; x += kTfThreads) {
    const float l = src[x] * a.inv_t;
    if (LDS) s_row[x] = l;
    if (l != l || l == INFINITY) {
      bad = 1;
    } else if (l != -INFINITY) {
      mx = fmaxf(mx, l);
      mn = fminf(mn, l);
      nfin += 1.0;
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

  // The cut where the weight (use_mass: fixed-point mass, else count) of the
  // kept entries, taken in order, first reaches `need`; narrows the kept set.
  auto select = [&](double need, bool use_mass) {
    float lo = mn, hi = mx;
    {
      float l0 = INFINITY, h0 = -INFINITY;
      int unused = 0;
      for (int x = t; x < V; x += kTfThreads) {
        const float l = L(x);
        if (kept(l, x)) {
          l0 = fminf(l0, l);
          h0 = fmaxf(h0, l);
        }
      }
      bminmax(l0, h0, unused);
      lo = l0;
      hi = h0;
    }
    double above = 0.0;            // weight of kept entries above the range [lo, hi]
    for (int level = 0; level < kTfLevels && lo < hi; ++level) {
      const float s = static_cast<float>(kTfBins) / (hi - lo);
      if (!(s > 0.f) || s == INFINITY) break;
      for (int i = t; i < kTfBins; i += kTfThreads) {
        s_cnt[i] = 0u;
        s_mass[i] = 0ull;
      }
      __syncthreads();
      auto bin_of = [&](float l) { return min(kTfBins - 1, static_cast<int>((hi - l) * s)); };
      for (int x = t; x < V; x += kTfThreads) {
        const float l = L(x);
        if (l >= lo && l <= hi && kept(l, x)) {
          const int b = bin_of(l);
          atomicAdd(&s_cnt[b], 1u);
          if (use_mass) atomicAdd(&s_mass[b], mfix(l));
        }
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
        }
      }
      __syncthreads();
      const int pb = s_bin;
      above = s_above;
      // the picked bin's value range becomes the next range
      float l0 = INFINITY, h0 = -INFINITY;
      int unused = 0;
      for (int x = t; x < V; x += kTfThreads) {
        const float l = L(x);
        if (l >= lo && l <= hi && kept(l, x) && bin_of(l) == pb) {
          l0 = fminf(l0, l);
          h0 = fmaxf(h0, l);
        }
      }
      bminmax(l0, h0, unused);
      lo = l0;
      hi = h0;
    }
    auto weight_ge = [&](float v, float top) {       // kept entries in [v, top]
      double c = 0.0;
      for (int x = t; x < V; x += kTfThreads) {
        const float l = L(x);
        if (l >= v && l <= top && kept(l, x)) c += use_mass ? static_cast<double>(mfix(l)) : 1.0;
      }
      return bsum(c);
    };
    if (lo < hi) {
      // exact bisection over the keys of [lo, hi]: the largest v with
      // above + weight(kept in [v, hi]) >= need
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
    for (int x = t; x < V; x += kTfThreads) {
      const float l = L(x);
      if (l == v && kept(l, x)) c_eq += 1.0;
    }
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
      int xlo = 0, xhi = V - 1;          // smallest X with n_keep tied kept entries at or below it
      while (xlo < xhi) {
        const int mid = (xlo + xhi) / 2;
        double c = 0.0;
        for (int x = t; x <= mid && x < V; x += kTfThreads) {
          const float l = L(x);
          if (l == v && kept(l, x)) c += 1.0;
        }
        if (bsum(c) >= n_keep) xhi = mid;
        else xlo = mid + 1;
      }
      cx = xlo;
    }
    if (v == cut_v) cut_x = min(cut_x, cx);
    else cut_x = cx;
    cut_v = v;
  };

  if (a.top_k > 0 && static_cast<double>(a.top_k) < nfin) select(static_cast<double>(a.top_k), false);
  if (a.top_p < 1.0) {
    double z = 0.0;
    for (int x = t; x < V; x += kTfThreads) {
      const float l = L(x);
      if (kept(l, x)) z += static_cast<double>(mfix(l));
    }
    z = bsum(z);
    select(a.top_p * z, true);
  }

  // ---- output ----
  if (a.probs) {
    double z = 0.0;
    for (int x = t; x < V; x += kTfThreads) {
      const float l = L(x);
      if (kept(l, x)) z += static_cast<double>(mass(l));
    }
    z = bsum(z);
    for (int x = t; x < V; x += kTfThreads) {
      const float l = L(x);
      dst[x] = kept(l, x) ? static_cast<float>(static_cast<double>(mass(l)) / z) : 0.f;
    }
  } else {
    for (int x = t; x < V; x += kTfThreads) {
      const float l = L(x);
      dst[x] = kept(l, x) ? l : -INFINITY;
    }
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
  if (V <= kTfLdsMax) {
    static bool lds_ok = false;          // a function attribute: set once per process
    if (!lds_ok) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(transform_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              kTfLdsMax * static_cast<int>(sizeof(float))) != hipSuccess)
        return TV_EHIP;
      lds_ok = true;
    }
    hipLaunchKernelGGL(transform_kernel<true>, dim3(rows), dim3(kTfThreads), V * sizeof(float), stream, a);
  } else
    hipLaunchKernelGGL(transform_kernel<false>, dim3(rows), dim3(kTfThreads), 0, stream, a);
  return tv::launch_status();
}
