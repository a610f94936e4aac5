// Shared device/host helpers of the treeverify library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/treeverify.h"

#define TV_BLOCK 16          // paged-cache block size (tokens)
#define TV_MAX_NODES 64      // tree nodes per request (one uint64 mask)

namespace tv {

// ---------------------------------------------------------------------------
// Host-side launch checks
// ---------------------------------------------------------------------------
inline tv_status launch_status() {
  return hipGetLastError() == hipSuccess ? TV_OK : TV_EHIP;
}

// ---------------------------------------------------------------------------
// bfloat16 <-> float
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; inputs here are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of the S-P
// network; each round multiplies words 0 and 2 by the two round constants,
// mixes the high halves with words 1/3 and the key, and the key advances by
// the two Weyl increments between rounds.
// ---------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

// Words of round `rnd` at node slot `slot` (0 = root, i + 1 = node i) of request b.
__device__ __forceinline__ u32x4 mss_words(uint64_t seed, uint64_t offset, int b, int slot, int rnd) {
  u32x4 c{static_cast<uint32_t>(64 * slot + rnd), static_cast<uint32_t>(b),
          static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32)};
  return philox4x32_10(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

// Uniform in (0, 1] from the top 24 bits (exact in fp32 and fp64).
__device__ __forceinline__ double unit_open0(uint32_t w) {
  return static_cast<double>((w >> 8) + 1u) * (1.0 / 16777216.0);
}

// Uniform integer in [0, m) by multiply-shift of the top 24 bits.
__device__ __forceinline__ int pick_index(uint32_t w, int m) {
  return static_cast<int>((static_cast<uint64_t>(w >> 8) * static_cast<uint64_t>(m)) >> 24);
}

// ---------------------------------------------------------------------------
// exp with a split log2(e): exp(x) = 2^(x*log2e).  The product x*log2e is
// carried as y + err (y = fp32 product, err = its rounding error plus the
// low part of log2e) and 2^err ~ 1 + err*ln2 corrects the hardware exp2 of y.
// Accurate to a couple of ulp for x <= 0, which is all this library needs.
// Arguments below -200 give 0 (fp32 exp underflows long before), which also
// keeps the split product finite for arguments near -FLT_MAX.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_acc(float x) {
  const float L2E_HI = 1.44269502162933349609375f;        // fp32(log2 e)
  const float L2E_LO = 1.925963033500011079e-8f;          // log2 e - L2E_HI
  x = fmaxf(x, -200.f);
  const float y = x * L2E_HI;
  const float err = fmaf(x, L2E_HI, -y) + x * L2E_LO;
  const float e = __builtin_amdgcn_exp2f(y);
  return fmaf(e, err * 0.693147180559945309f, e);
}

// Fast exp for attention probabilities (argument already scaled by log2 e).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Wave64 reductions through DPP-free shuffles (compiled to ds_swizzle/dpp).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Wave64 reductions and scans on DPP lane moves (VALU, no LDS round trip).
// gfx9 DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes 1 and 2
// apart, row_half_mirror / row_mirror pair lanes across 8- and 16-lane
// groups, row_bcast:15 / row_bcast:31 carry a row's last lane into the next
// row(s), row_shr:n shifts within a row, wave_shr:1 shifts the whole wave.
// Reductions leave the result in lane 63 and return it to every lane.
// ---------------------------------------------------------------------------
namespace dpp {
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowMirror = 0x140, kRowHalfMirror = 0x141,
              kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;
}

template <int ctrl, int row_mask = 0xF>
__device__ __forceinline__ int dpp_mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, ctrl, row_mask, 0xF, false);
}
template <int ctrl, int row_mask = 0xF>
__device__ __forceinline__ double dpp_mov_f64(double old, double v) {
  const int lo = dpp_mov<ctrl, row_mask>(__double2loint(old), __double2loint(v));
  const int hi = dpp_mov<ctrl, row_mask>(__double2hiint(old), __double2hiint(v));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}

// sum of a double over the wave (same value, bit for bit, in every lane)
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_mov_f64<dpp::kQuadXor1>(0.0, v);
  v += dpp_mov_f64<dpp::kQuadXor2>(0.0, v);
  v += dpp_mov_f64<dpp::kRowHalfMirror>(0.0, v);
  v += dpp_mov_f64<dpp::kRowMirror>(0.0, v);
  v += dpp_mov_f64<dpp::kRowBcast15, 0xA>(0.0, v);
  v += dpp_mov_f64<dpp::kRowBcast31, 0xC>(0.0, v);
  return readlane_f64(v, 63);
}

// max of a float over the wave (NaN inputs lose to any number)
__device__ __forceinline__ float wave_max_dpp(float v) {
  auto step = [](float x, float y) { return fmaxf(x, y); };
  v = step(v, __int_as_float(dpp_mov<dpp::kQuadXor1>(__float_as_int(-INFINITY), __float_as_int(v))));
  v = step(v, __int_as_float(dpp_mov<dpp::kQuadXor2>(__float_as_int(-INFINITY), __float_as_int(v))));
  v = step(v, __int_as_float(dpp_mov<dpp::kRowHalfMirror>(__float_as_int(-INFINITY), __float_as_int(v))));
  v = step(v, __int_as_float(dpp_mov<dpp::kRowMirror>(__float_as_int(-INFINITY), __float_as_int(v))));
  v = step(v, __int_as_float(dpp_mov<dpp::kRowBcast15, 0xA>(__float_as_int(-INFINITY), __float_as_int(v))));
  v = step(v, __int_as_float(dpp_mov<dpp::kRowBcast31, 0xC>(__float_as_int(-INFINITY), __float_as_int(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// OR of an int over the wave
__device__ __forceinline__ int wave_or_dpp(int v) {
  v |= dpp_mov<dpp::kQuadXor1>(0, v);
  v |= dpp_mov<dpp::kQuadXor2>(0, v);
  v |= dpp_mov<dpp::kRowHalfMirror>(0, v);
  v |= dpp_mov<dpp::kRowMirror>(0, v);
  v |= dpp_mov<dpp::kRowBcast15, 0xA>(0, v);
  v |= dpp_mov<dpp::kRowBcast31, 0xC>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}

// max over the wave with the lowest index among equal maxima; NaN values
// never win (callers flag them separately)
__device__ __forceinline__ void argmax_merge(float& m, int& a, float m2, int a2) {
  if (m2 > m || (m2 == m && a2 < a)) {
    m = m2;
    a = a2;
  }
}
template <int ctrl, int row_mask = 0xF>
__device__ __forceinline__ void argmax_step(float& m, int& a) {
  const float m2 = __int_as_float(dpp_mov<ctrl, row_mask>(__float_as_int(-INFINITY), __float_as_int(m)));
  const int a2 = dpp_mov<ctrl, row_mask>(0x7FFFFFFF, a);
  argmax_merge(m, a, m2, a2);
}
__device__ __forceinline__ void wave_argmax_dpp(float& m, int& a) {
  argmax_step<dpp::kQuadXor1>(m, a);
  argmax_step<dpp::kQuadXor2>(m, a);
  argmax_step<dpp::kRowHalfMirror>(m, a);
  argmax_step<dpp::kRowMirror>(m, a);
  argmax_step<dpp::kRowBcast15, 0xA>(m, a);
  argmax_step<dpp::kRowBcast31, 0xC>(m, a);
  m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
  a = __builtin_amdgcn_readlane(a, 63);
}

// inclusive prefix sum of a double over the wave (lane order); *excl gets
// the previous lane's inclusive value, bit for bit (0 in lane 0)
__device__ __forceinline__ double wave_scan_dpp(double v, double* excl) {
  v += dpp_mov_f64<0x111>(0.0, v);        // row_shr:1
  v += dpp_mov_f64<0x112>(0.0, v);        // row_shr:2
  v += dpp_mov_f64<0x114>(0.0, v);        // row_shr:4
  v += dpp_mov_f64<0x118>(0.0, v);        // row_shr:8
  v += dpp_mov_f64<dpp::kRowBcast15, 0xA>(0.0, v);
  v += dpp_mov_f64<dpp::kRowBcast31, 0xC>(0.0, v);
  *excl = dpp_mov_f64<dpp::kWaveShr1>(0.0, v);
  return v;
}

}  // namespace tv
