// Device helpers shared by the pair-Gram kernels (fp64 tiles in kh.hip, exact
// integer tiles in gram8.hip): raw feature access, fp64 exponentials, and the
// thresholds of the kernel-halving walk.
#pragma once

#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace thin {

namespace {

constexpr int kThrCap = 2048;          // pairs whose b^2 and u a threshold workgroup keeps in LDS

// 8 consecutive features of one point, kept raw until they are staged.
struct Raw8 {
  uint4 w[2];   // fp32: two float4; bf16: w[0] only; fp8: w[0].x, w[0].y
};

template <int ET>
__device__ __forceinline__ void load8(const void* base, int64_t off, Raw8& r) {
  if constexpr (ET == kFP8) {
    const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + off);
    r.w[0].x = x.x;
    r.w[0].y = x.y;
  } else if constexpr (ET == kBF16) {
    r.w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
}

template <int ET>
__device__ __forceinline__ double raw8_at(const Raw8& r, int j) {
  if constexpr (ET == kFP8) {
    return fp8_byte_to_float(j < 4 ? r.w[0].x : r.w[0].y, j & 3);
  } else if constexpr (ET == kBF16) {
    const uint32_t word = (j < 2 ? r.w[0].x : j < 4 ? r.w[0].y : j < 6 ? r.w[0].z : r.w[0].w);
    return bf16_bits_to_float(static_cast<uint16_t>((j & 1) ? (word >> 16) : (word & 0xffffu)));
  } else {
    const uint4& q = r.w[j >> 2];
    const uint32_t word = ((j & 3) == 0 ? q.x : (j & 3) == 1 ? q.y : (j & 3) == 2 ? q.z : q.w);
    return __uint_as_float(word);
  }
}

// e^x in fp64 for finite x: Cody-Waite reduction x = n ln2 + r (ln2 split into
// a double and its remainder, so r is exact to far below an ulp), |r| <= ln2/2,
// the Taylor series of e^r through r^13 (truncation < 5e-18 relative), then a
// scaling by 2^n (overflow gives inf, underflow 0 or a subnormal).
__device__ __forceinline__ double exp_f64(double x) {
  const double n = __builtin_rint(x * 1.4426950408889634);
  double r = fma(-n, 0x1.62e42fefa39efp-1, x);
  r = fma(-n, 0x1.abc9e3b39803fp-56, r);
  double p = 1.6059043836821613e-10;
  p = fma(p, r, 2.08767569878681e-09);
  p = fma(p, r, 2.505210838544172e-08);
  p = fma(p, r, 2.755731922398589e-07);
  p = fma(p, r, 2.7557319223985893e-06);
  p = fma(p, r, 2.48015873015873e-05);
  p = fma(p, r, 0.0001984126984126984);
  p = fma(p, r, 0.001388888888888889);
  p = fma(p, r, 0.008333333333333333);
  p = fma(p, r, 0.041666666666666664);
  p = fma(p, r, 0.16666666666666666);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return __builtin_amdgcn_ldexp(p, static_cast<int>(fmax(fmin(n, 2100.0), -2100.0)));
}

// ---------------------------------------------------------------------------
// Thresholds of the walk.  For pair i: b_i^2 = G_ii,
// a_i = max(b_i sigma_{i-1} c_N, b_i^2) with c_N = sqrt(2 ln(2N / delta)), and
// the first point is kept iff u_i < (1 - alpha_i / a_i) / 2, i.e. iff
// alpha_i < a_i (1 - 2 u_i) (a_i = 0: iff u_i < 1/2).  a_i and sigma_i depend
// only on the b's, so the thresholds thr_i = a_i (1 - 2 u_i) are formed ahead
// of the walk.  Bins of more than 64 pairs get them from extra workgroups of
// the pair-Gram launch (one wave per bin, overlapping the tiles), stored in the
// lower triangle of the bin's G, which the walk does not otherwise read: pair
// i >= 1 at G[i][i-1], pair 0 at G[P-1][0].  The one-wave walk of smaller bins
// forms its own.
//
// sigma recursion without a division: with sigma = sqrt(sigma^2),
//   if b sigma c >= b^2 (a = b sigma c):
//     sigma^2 += max(0, b^2 (1 + 1/c^2) - 2 sigma b / c)
//   else (a = b^2):  sigma^2 = max(sigma^2, b^2)
// which is the published update b^2 max(0, 1 + (b^2 - 2a) sigma^2 / a^2)
// written out for the two cases of a.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t thr_slot(int i, int P) {
  return i >= 1 ? static_cast<int64_t>(i) * P + (i - 1) : static_cast<int64_t>(P - 1) * P;
}

__device__ __forceinline__ double readlane_f64(double x, int i) {
  const uint64_t bits = __double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(bits), i);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(bits >> 32), i);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Steps 0 .. n-1 of the sigma recursion on the pairs held by the lanes of one
// wave (lane i: b_i^2 and b_i), from sigma^2 = s2; lane i receives
// a_i = max(b_i sigma_{i-1} c, b_i^2).  The values depending on b alone are
// formed lane-parallel first; on the serial path stay one square root, one
// multiply, one fma, two max, one add and selects (no branches).
__device__ __forceinline__ double sigma_steps(double& s2, double b2l, double bl, int n, double c, double k1, double k2) {
  const int lane = threadIdx.x & 63;
  const double cbl = c * bl, b2k1l = b2l * k1, k2bl = k2 * bl;
  double al = 0.0;
  for (int i = 0; i < n; ++i) {
    const double b2 = readlane_f64(b2l, i);
    const double cb = readlane_f64(cbl, i);
    const double b2k1 = readlane_f64(b2k1l, i);
    const double k2b = readlane_f64(k2bl, i);
    const double sg = __builtin_amdgcn_sqrt(s2);
    const double bsc = cb * sg;
    const double grow = s2 + fmax(0.0, fma(-k2b, sg, b2k1));
    const double keep = fmax(s2, b2);
    al = lane == i ? fmax(bsc, b2) : al;
    s2 = bsc >= b2 ? grow : keep;
  }
  return al;
}

// Threshold of a pair: a (1 - 2 u), or +-inf by u < 1/2 when a = 0.
__device__ __forceinline__ double threshold(double al, double u) {
  return al > 0.0 ? al * (1.0 - 2.0 * u) : (u < 0.5 ? INFINITY : -INFINITY);
}

// The threshold a walk step compares alpha with: greedy signs keep the first
// point exactly when alpha < 0, whatever a and u are.
__device__ __forceinline__ double step_threshold(int greedy, double al, double u) {
  return greedy ? 0.0 : threshold(al, u);
}

// b_i^2 of pair i (its two points: fp64 dot products, the same kernel as the
// Gram, four partial sums per product) and u_i (Philox).
template <int ET>
__device__ void pair_b2_u(const GramLaunch& a, int z, int i, double& b2, double& u) {
  const int unit = z / a.bins_per_unit, lb = z % a.bins_per_unit;
  const int b = unit / a.src.H_kv, h = unit % a.src.H_kv;
  const int32_t* list = a.idx + static_cast<int64_t>(unit) * a.idx_unit_stride + static_cast<int64_t>(lb) * a.idx_stride;
  auto dots = [&](const void* base, int F, int64_t re, int64_t ro, double& xx, double& xy, double& yy) {
    double sxx[4] = {0.0, 0.0, 0.0, 0.0}, sxy[4] = {0.0, 0.0, 0.0, 0.0}, syy[4] = {0.0, 0.0, 0.0, 0.0};
    for (int f = 0; f < F; f += 8) {
      Raw8 e8, o8;
      load8<ET>(base, re * F + f, e8);
      load8<ET>(base, ro * F + f, o8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double x = raw8_at<ET>(e8, j), y = raw8_at<ET>(o8, j);
        sxx[j & 3] = fma(x, x, sxx[j & 3]);
        sxy[j & 3] = fma(x, y, sxy[j & 3]);
        syy[j & 3] = fma(y, y, syy[j & 3]);
      }
    }
    xx = (sxx[0] + sxx[1]) + (sxx[2] + sxx[3]);
    xy = (sxy[0] + sxy[1]) + (sxy[2] + sxy[3]);
    yy = (syy[0] + syy[1]) + (syy[2] + syy[3]);
  };
  const int32_t te = list[2 * i], to = list[2 * i + 1];
  if ((static_cast<uint32_t>(te) >= static_cast<uint32_t>(a.src.S) ||
       static_cast<uint32_t>(to) >= static_cast<uint32_t>(a.src.S)) && a.err)
    __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const int64_t S1 = a.src.S - 1;
  const int64_t ce = te < 0 ? 0 : (te > S1 ? S1 : te), co = to < 0 ? 0 : (to > S1 ? S1 : to);
  const int64_t re = (static_cast<int64_t>(b) * a.src.S + ce) * a.src.H_kv + h;
  const int64_t ro = (static_cast<int64_t>(b) * a.src.S + co) * a.src.H_kv + h;
  double kee, keo, koo, vee, veo, voo;
  dots(a.src.k, a.src.E, re, ro, kee, keo, koo);
  dots(a.src.v, a.src.D, re, ro, vee, veo, voo);
  const double xee = exp_f64(a.scale * kee) * (vee + 1.0);
  const double xeo = exp_f64(a.scale * keo) * (veo + 1.0);
  const double xoo = exp_f64(a.scale * koo) * (voo + 1.0);
  b2 = fmax((xee - xeo) - (xeo - xoo), 0.0);
  u = philox_uniform(static_cast<uint64_t>(i), a.bin_base + lb, static_cast<uint64_t>(unit), a.tag, a.seed);
}

// The sigma recursion of bin z by one wave, 64 pairs at a time, and the
// thresholds into the lower triangle.  s_b2 / s_u: the bin's b^2 and u already
// formed (by the whole workgroup), or nullptr to form them here per chunk.
template <int ET>
__device__ void bin_thresholds(const GramLaunch& a, int z, const double* s_b2, const double* s_u) {
  const int P = a.N / 2;
  const int lane = threadIdx.x & 63;
  double* G = a.G + static_cast<int64_t>(z) * P * P;
  const double c = sqrt(2.0 * log(2.0 * a.N / a.delta));
  const double k1 = 1.0 + 1.0 / (c * c);
  const double k2 = 2.0 / c;
  double s2 = 0.0;
  for (int i0 = 0; i0 < P; i0 += 64) {
    const int i = i0 + lane;
    const bool mine = i < P;
    double b2 = 0.0, u = 0.0;
    if (mine) {
      if (s_b2) {
        b2 = s_b2[i];
        u = s_u[i];
      } else {
        pair_b2_u<ET>(a, z, i, b2, u);
      }
    }
    const double al = sigma_steps(s2, b2, sqrt(b2), min(64, P - i0), c, k1, k2);
    if (mine) G[thr_slot(i, P)] = step_threshold(a.greedy, al, u);
  }
}

// e^x in fp64 for the Gram entries: x = (256 n' + j) ln2 / 256 + r with
// |r| <= ln2 / 512, e^x = 2^n' T[j] (1 + r + r^2/2 + r^3/6 + r^4/24); the
// truncation is below 4e-17 relative, and T[j] = 2^(j/256) comes from exp_f64.
__device__ __forceinline__ double exp_tab(double x, const double* T) {
  double n = __builtin_rint(x * 369.3299304675746);    // 256 / ln 2
  n = fmax(fmin(n, 540000.0), -540000.0);
  double r = fma(-n, 0x1.62e42fefa39efp-9, x);
  r = fma(-n, 0x1.abc9e3b39803fp-64, r);
  double p = fma(r, 0.041666666666666664, 0.16666666666666666);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = static_cast<int>(n);
  return __builtin_amdgcn_ldexp(T[ni & 255] * p, ni >> 8);
}

// Threshold workgroups of a pair-Gram launch (bins of more than 64 pairs; the
// walks of the large sweep kernel read the thresholds).  With few bins
// (per_wave == 0) workgroup w takes bin w: all its waves form b^2 and u into
// LDS (smem: 2 kThrCap doubles), then wave 0 runs the recursion; with many,
// each wave takes bins on its own, (waves per workgroup) nthr apart, so the
// thresholds hold few workgroup slots while the tiles run.
template <int ET>
__device__ void threshold_workgroup(const GramLaunch& a, int w, int nthr, int per_wave, double* smem) {
  if (per_wave) {
    const int waves = blockDim.x >> 6;
    for (int z = waves * w + (threadIdx.x >> 6); z < a.nbins; z += waves * nthr) bin_thresholds<ET>(a, z, nullptr, nullptr);
    return;   // the whole workgroup: no barrier in this mode
  }
  const int z = w;
  if (z >= a.nbins) return;   // the whole workgroup
  const int P = a.N / 2;      // b^2 and u of up to kThrCap pairs
  double* s_b2 = smem;
  double* s_u = smem + kThrCap;
  for (int i = threadIdx.x; i < P; i += blockDim.x) pair_b2_u<ET>(a, z, i, s_b2[i], s_u[i]);
  __syncthreads();
  if (threadIdx.x < 64) bin_thresholds<ET>(a, z, s_b2, s_u);
}

// How many threshold workgroups a pair-Gram launch over `a` carries: one per
// bin while there are at most 64 bins, else at most 64 with a bin per wave at
// a time; a multiple of 8 so that the tiles after them keep their XCD mapping.
inline void threshold_groups(const GramLaunch& a, int& nthr, int& per_wave) {
  const int P = a.N / 2;
  per_wave = (a.nbins > 64 || P > kThrCap) ? 1 : 0;
  nthr = 0;
  if (P > 64) nthr = per_wave ? std::min((a.nbins + 31) / 32 * 8, 64) : (a.nbins + 7) / 8 * 8;
}

}  // namespace

}  // namespace thin
