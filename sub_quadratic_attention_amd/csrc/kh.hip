// Kernel halving on gfx950: fp64 pair Gram under kappa_att and the sequential
// self-balancing walk, plus the index bookkeeping of Compress and EXPRESS.
//
// kappa((k, v), (k', v')) = exp(s <k, k'>) (<v, v'> + 1): the exponential
// dot-product kernel on keys times the linear kernel on (v, 1), whose inner
// products are exactly the two sums softmax attention needs ("Express
// Language Modeling", section "Thinformer Express", names this key-value
// attention kernel).  The walk is kernel halving as published in the
// kernel-thinning papers (Dwivedi and Mackey, "Kernel Thinning"; Shetty,
// Dwivedi and Mackey, "Distribution Compression in Near-linear Time").
//
// Precision: every dot product is accumulated in fp64 (products of fp32 or
// bf16 inputs are exact in fp64) and exp is evaluated in fp64, so that the
// randomised sign decisions agree with a float64 reference except at true
// near-ties.

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace thin {

namespace {

// ---------------------------------------------------------------------------
// Pair Gram.  One workgroup (4 waves) computes a 32 x 32 tile of pairs
// (64 x 64 points) with fp64 MFMA 16x16x4.  Wave (wr, wc) owns the 16 x 16
// pair block (16 wr.., 16 wc..) and keeps four accumulators per pass:
// even-even, even-odd, odd-even and odd-odd point products, so the pair
// combination G = k_ee - k_eo - k_oe + k_oo needs no lane exchange.
// Pass 0 accumulates <k, k'>, pass 1 <v, v'>.
// ---------------------------------------------------------------------------
constexpr int kChunk = 16;             // features staged per step
constexpr int kPad = kChunk + 1;

template <bool BF16>
__device__ __forceinline__ void load4(const void* base, int64_t off, double out[4]) {
  if constexpr (BF16) {
    const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    out[0] = bf16_bits_to_float(static_cast<uint16_t>(raw.x & 0xffffu));
    out[1] = bf16_bits_to_float(static_cast<uint16_t>(raw.x >> 16));
    out[2] = bf16_bits_to_float(static_cast<uint16_t>(raw.y & 0xffffu));
    out[3] = bf16_bits_to_float(static_cast<uint16_t>(raw.y >> 16));
  } else {
    const float4 raw = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    out[0] = raw.x;
    out[1] = raw.y;
    out[2] = raw.z;
    out[3] = raw.w;
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void pair_gram_kernel(GramLaunch a) {
  // blockIdx.x = bin * tiles_per_bin + lower-triangular tile (tr >= tc)
  const int P = a.N / 2;
  const int nt = (P + 31) / 32;
  const int tiles = nt * (nt + 1) / 2;
  const int z = static_cast<int>(blockIdx.x / tiles);
  const int t = static_cast<int>(blockIdx.x % tiles);
  int tr = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
  while (tr * (tr + 1) / 2 > t) --tr;
  while ((tr + 1) * (tr + 2) / 2 <= t) ++tr;
  const int tc = t - tr * (tr + 1) / 2;

  const int unit = z / a.bins_per_unit;
  const int b = unit / a.src.H_kv;
  const int h = unit % a.src.H_kv;
  const int32_t* idx = a.idx + static_cast<int64_t>(unit) * a.idx_unit_stride +
                       static_cast<int64_t>(z % a.bins_per_unit) * a.idx_stride;

  __shared__ double rowF[64][kPad];
  __shared__ double colF[64][kPad];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wr = w >> 1, wc = w & 1;

  // loader role: point lp of the row / column sets, features lf .. lf+3
  const int lp = tid >> 2;
  const int lf = (tid & 3) * 4;
  const int rp = 64 * tr + lp;
  const int cp = 64 * tc + lp;
  const bool rvalid = rp < a.N;
  const bool cvalid = cp < a.N;
  const int64_t rrow = rvalid ? (static_cast<int64_t>(b) * a.src.S + idx[rp]) * a.src.H_kv + h : 0;
  const int64_t crow = cvalid ? (static_cast<int64_t>(b) * a.src.S + idx[cp]) * a.src.H_kv + h : 0;

  f64x4_t acc[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[p][q] = f64x4_t{0.0, 0.0, 0.0, 0.0};

  const int pr = 16 * wr + (lane & 15);   // pair row inside the tile
  const int pc = 16 * wc + (lane & 15);   // pair column inside the tile
  const int kq = lane >> 4;

#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int F = pass ? a.src.D : a.src.E;
    const void* base = pass ? a.src.v : a.src.k;
    double nr[4] = {0, 0, 0, 0}, nc[4] = {0, 0, 0, 0};
    if (rvalid) load4<BF16>(base, rrow * F + lf, nr);
    if (cvalid) load4<BF16>(base, crow * F + lf, nc);
    for (int f0 = 0; f0 < F; f0 += kChunk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rowF[lp][lf + j] = nr[j];
        colF[lp][lf + j] = nc[j];
      }
      __syncthreads();
      if (f0 + kChunk < F) {     // prefetch the next chunk while this one is used
        if (rvalid) load4<BF16>(base, rrow * F + f0 + kChunk + lf, nr);
        if (cvalid) load4<BF16>(base, crow * F + f0 + kChunk + lf, nc);
      }
#pragma unroll
      for (int kk = 0; kk < kChunk / 4; ++kk) {
        const int kf = kk * 4 + kq;
        const double Ae = rowF[2 * pr][kf];
        const double Ao = rowF[2 * pr + 1][kf];
        const double Be = colF[2 * pc][kf];
        const double Bo = colF[2 * pc + 1][kf];
        acc[pass][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(Ae, Be, acc[pass][0], 0, 0, 0);
        acc[pass][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(Ae, Bo, acc[pass][1], 0, 0, 0);
        acc[pass][2] = __builtin_amdgcn_mfma_f64_16x16x4f64(Ao, Be, acc[pass][2], 0, 0, 0);
        acc[pass][3] = __builtin_amdgcn_mfma_f64_16x16x4f64(Ao, Bo, acc[pass][3], 0, 0, 0);
      }
      __syncthreads();
    }
  }

  // fp64 16x16x4 accumulator element i of lane l is (row l / 16 + 4 i, column l % 16)
  double* G = a.G + static_cast<int64_t>(z) * P * P;
  const int col = 32 * tc + 16 * wc + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * tr + 16 * wr + kq + 4 * i;
    const double kee = exp(a.scale * acc[0][0][i]) * (acc[1][0][i] + 1.0);
    const double keo = exp(a.scale * acc[0][1][i]) * (acc[1][1][i] + 1.0);
    const double koe = exp(a.scale * acc[0][2][i]) * (acc[1][2][i] + 1.0);
    const double koo = exp(a.scale * acc[0][3][i]) * (acc[1][3][i] + 1.0);
    if (row < P && col < P) G[static_cast<int64_t>(row) * P + col] = (kee - keo) - (koe - koo);
  }
}

// ---------------------------------------------------------------------------
// Kernel-halving walk of one bin per workgroup.
//
// For pair i: b_i^2 = G_ii, a_i = max(b_i sigma_{i-1} c_N, b_i^2) with
// c_N = sqrt(2 ln(2N / delta)), and the first point is kept iff
// u_i < (1 - alpha_i / a_i) / 2, i.e. iff alpha_i < a_i (1 - 2 u_i)
// (a_i = 0: iff u_i < 1/2).  a_i and sigma_i depend only on the b's, so the
// thresholds thr_i = a_i (1 - 2 u_i) are computed first; alpha_i =
// sum_{j<i} eta_j G_ij is then swept panel by panel: the contribution of
// earlier panels is a matrix-vector product spread over the workgroup, and
// the 64 decisions inside a panel are taken by one wave, lane i holding
// alpha_i and its row of the panel's G block, one ballot per decision.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t dec_offset(const SweepLaunch& a, int lb, int P) {
  if (a.dec_mode == 1) {   // Express batch k = lb: HALVE 0, then (3 batches, HALVE) per epoch
    const int64_t n = P;
    return 3 * n + 6 * n * (lb / 3) + n * (lb % 3);
  }
  return a.dec_base + static_cast<int64_t>(lb) * P;
}

__global__ __launch_bounds__(256) void halving_sweep_kernel(SweepLaunch a) {
  extern __shared__ double smem[];
  const int z = blockIdx.x;
  const int P = a.N / 2;
  const int unit = z / a.bins_per_unit;
  const int lb = z % a.bins_per_unit;
  const double* G = a.G + static_cast<int64_t>(z) * P * P;
  double* s_thr = smem;               // P
  double* s_b2 = s_thr + P;           // P
  double* s_eta = s_b2 + P;           // P
  double* s_alpha = s_eta + P;        // 64
  double* s_G = s_alpha + 64;         // 64 x 65

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  for (int i = tid; i < P; i += 256) {
    s_thr[i] = philox_uniform(static_cast<uint64_t>(i), a.bin_base + lb, static_cast<uint64_t>(unit), a.tag,
                              a.seed);
    s_b2[i] = fmax(G[static_cast<int64_t>(i) * P + i], 0.0);
  }
  __syncthreads();
  if (tid == 0) {
    const double c = sqrt(2.0 * log(2.0 * a.N / a.delta));
    double s2 = 0.0;
    for (int i = 0; i < P; ++i) {
      const double b2 = s_b2[i];
      const double bb = sqrt(b2);
      const double aa = fmax(bb * sqrt(s2) * c, b2);
      const double u = s_thr[i];
      s_thr[i] = aa > 0.0 ? aa * (1.0 - 2.0 * u) : (u < 0.5 ? INFINITY : -INFINITY);
      if (aa > 0.0) s2 = s2 + b2 * fmax(0.0, 1.0 + (b2 - 2.0 * aa) * s2 / (aa * aa));
    }
  }
  __syncthreads();

  const int32_t* in = a.idx_in + static_cast<int64_t>(unit) * a.in_unit_stride + static_cast<int64_t>(lb) * a.in_stride;
  int32_t* out = a.idx_out + static_cast<int64_t>(z) * a.out_stride;
  for (int p0 = 0; p0 < P; p0 += 64) {
    const int rows = min(64, P - p0);
    // contribution of the decided panels
    for (int r = w * 16; r < w * 16 + 16; ++r) {
      double part = 0.0;
      if (r < rows) {
        const double* g = G + static_cast<int64_t>(p0 + r) * P;
        for (int j = lane; j < p0; j += 64) part += s_eta[j] * g[j];
      }
      part = wave_sum(part);
      if (lane == 0) s_alpha[r] = part;
    }
    // this panel's block (lower triangle)
    for (int e = tid; e < 64 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      s_G[r * 65 + c] = (r < rows && c <= r) ? G[static_cast<int64_t>(p0 + r) * P + p0 + c] : 0.0;
    }
    __syncthreads();
    if (w == 0) {
      double alpha = s_alpha[lane];
      const double thr = lane < rows ? s_thr[p0 + lane] : 0.0;
      double g[64];
#pragma unroll
      for (int c = 0; c < 64; ++c) g[c] = s_G[lane * 65 + c];
      uint64_t bits = 0;
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        const uint64_t m = __ballot(alpha < thr);
        const bool first = (m >> j) & 1ull;
        bits |= static_cast<uint64_t>(first) << j;
        alpha += first ? g[j] : -g[j];
      }
      if (lane < rows) {
        const int i = p0 + lane;
        const bool first = (bits >> lane) & 1ull;
        s_eta[i] = first ? 1.0 : -1.0;
        out[i] = in[2 * i + (first ? 0 : 1)];
        if (a.dec) a.dec[static_cast<int64_t>(unit) * a.dec_per_unit + dec_offset(a, lb, P) + i] = first ? 1 : 0;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Index bookkeeping.
// ---------------------------------------------------------------------------
__global__ void iota_kernel(int32_t* out, int64_t units, int64_t n, int64_t stride) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= units * n) return;
  out[(i / n) * stride + (i % n)] = static_cast<int32_t>(i % n);
}

// Uniform subsampling of the thin phase: batch k of epoch e = k / 3 + 1
// (m = 4^e, r = m / 2) covers tokens [4^e n (1 + k % 3), 4^e n (2 + k % 3))
// in 2n aligned groups of r tokens; each group contributes the token at
// offset floor(u r), u from counter (group, log2 r, unit, subsample tag).
__global__ void express_reps_kernel(ExpressView ev, int units, uint64_t seed, int32_t* reps) {
  const int64_t per_unit = static_cast<int64_t>(ev.n_batches_alloc) * 2 * ev.n;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per_unit * units) return;
  const int unit = static_cast<int>(i / per_unit);
  const int64_t rem = i % per_unit;
  const int k = static_cast<int>(rem / (2 * ev.n));
  const int slot = static_cast<int>(rem % (2 * ev.n));
  const int e = k / 3 + 1;
  const int log2m = 2 * e;
  const int log2r = log2m - 1;
  const int64_t start = (static_cast<int64_t>(ev.n) << log2m) * (1 + k % 3);
  const int64_t g = (start >> log2r) + slot;
  const uint64_t word = philox_word0(static_cast<uint64_t>(g), static_cast<uint64_t>(log2r),
                                     static_cast<uint64_t>(unit), kTagSubsample, seed);
  const int64_t off = static_cast<int64_t>(word >> (64 - log2r));
  reps[i] = static_cast<int32_t>((g << log2r) + off);
}

// Input list of HALVE e: the first 4n tokens (e = 0), else the output of
// HALVE e-1 followed by the three batches of epoch e.
__global__ void halve_input_kernel(ExpressView ev, int units, int e, int32_t* halve_in) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per = 4LL * ev.n;
  if (i >= per * units) return;
  const int unit = static_cast<int>(i / per);
  const int j = static_cast<int>(i % per);
  int32_t val;
  if (e == 0) {
    val = j;
  } else if (j < ev.n) {
    val = ev.halve_out[(static_cast<int64_t>(unit) * ev.n_halves + (e - 1)) * ev.n + j];
  } else {
    const int64_t base = (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (e - 1)) * ev.n;
    val = ev.batch_out[base + (j - ev.n)];
  }
  halve_in[i] = val;
}

// Final causal coreset of a unit: the cache and buffer after every full block,
// then the trailing partial block (weight 1), padded with -1 / 0.
__device__ void express_state_after(const ExpressView& ev, int unit, int beta, int& n_halve_pts,
                                    const int32_t*& halve_pts, int& n_batch_pts, const int32_t*& batch_pts,
                                    int& n_rep, const int32_t*& rep_pts, int& raw_prefix, float& wm, float& wr) {
  n_halve_pts = n_batch_pts = n_rep = 0;
  halve_pts = batch_pts = rep_pts = nullptr;
  raw_prefix = 0;
  wm = 1.0f;
  wr = 1.0f;
  if (beta < 4) {
    raw_prefix = beta * ev.n;
    return;
  }
  int E = 1;
  while ((1LL << (2 * (E + 1))) <= beta) ++E;
  const int m = 1 << (2 * E);
  const int since = beta - m;
  const int nbc = since / m;
  const int rem = since % m;
  wm = static_cast<float>(m);
  wr = static_cast<float>(m / 2);
  n_halve_pts = ev.n;
  halve_pts = ev.halve_out + (static_cast<int64_t>(unit) * ev.n_halves + (E - 1)) * ev.n;
  n_batch_pts = nbc * ev.n;
  batch_pts = ev.batch_out + (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (E - 1)) * ev.n;
  n_rep = static_cast<int>((static_cast<int64_t>(rem) * 2 * ev.n) / m);
  rep_pts = ev.reps + (static_cast<int64_t>(unit) * ev.n_batches_alloc + 3 * (E - 1) + nbc) * 2 * ev.n;
}

__global__ void express_final_kernel(ExpressView ev, int units, int S, int32_t* idx, float* w, int32_t* len,
                                     int64_t cap) {
  const int unit = blockIdx.x;
  int nh, nb, nr, raw;
  const int32_t *hp, *bp, *rp;
  float wm, wr;
  express_state_after(ev, unit, ev.nblk, nh, hp, nb, bp, nr, rp, raw, wm, wr);
  const int tail_start = ev.nblk * ev.n;
  const int n_raw = raw + (S - tail_start);   // raw prefix (exact phase) + trailing block
  const int total = nh + nb + nr + n_raw;
  int32_t* oi = idx ? idx + static_cast<int64_t>(unit) * cap : nullptr;
  float* ow = w ? w + static_cast<int64_t>(unit) * cap : nullptr;
  for (int j = threadIdx.x; j < cap; j += blockDim.x) {
    int32_t id = -1;
    float wt = 0.0f;
    if (j < nh) {
      id = hp[j];
      wt = wm;
    } else if (j < nh + nb) {
      id = bp[j - nh];
      wt = wm;
    } else if (j < nh + nb + nr) {
      id = rp[j - nh - nb];
      wt = wr;
    } else if (j < total) {
      const int r = j - nh - nb - nr;
      id = r < raw ? r : tail_start + (r - raw);
      wt = 1.0f;
    }
    if (oi) oi[j] = id;
    if (ow) ow[j] = wt;
  }
  if (len && threadIdx.x == 0) len[unit] = total;
}

__global__ void fill_coreset_kernel(const int32_t* src, int64_t src_stride, int units, int n, float wv,
                                    int32_t* idx, float* w, int32_t* len) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(units) * n) return;
  const int64_t u = i / n, j = i % n;
  if (idx) idx[i] = src ? src[u * src_stride + j] : static_cast<int32_t>(j);
  if (w) w[i] = wv;
  if (len && j == 0) len[u] = n;
}

__global__ void philox_words_kernel(const uint64_t* ctr, int64_t n, uint64_t seed, uint64_t* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t x[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  philox4x64_10(x, seed, 0);
  out[4 * i] = x[0];
  out[4 * i + 1] = x[1];
  out[4 * i + 2] = x[2];
  out[4 * i + 3] = x[3];
}

inline unsigned grid1d(int64_t n, int block) { return static_cast<unsigned>((n + block - 1) / block); }

}  // namespace

hipError_t launch_pair_gram(const GramLaunch& a, hipStream_t s) {
  const int P = a.N / 2;
  const int nt = (P + 31) / 32;
  dim3 grid(static_cast<unsigned>(static_cast<int64_t>(nt) * (nt + 1) / 2 * a.nbins));
  if (a.src.bf16)
    hipLaunchKernelGGL(pair_gram_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(pair_gram_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t sweep_lds_bytes(int N) { return (3 * static_cast<size_t>(N / 2) + 64 + 64 * 65) * sizeof(double); }

hipError_t launch_halving_sweep(const SweepLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(halving_sweep_kernel, dim3(a.nbins), dim3(256), sweep_lds_bytes(a.N), s, a);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* out, int64_t units, int64_t n, int64_t stride, hipStream_t s) {
  if (units * n == 0) return hipSuccess;
  hipLaunchKernelGGL(iota_kernel, dim3(grid1d(units * n, 256)), dim3(256), 0, s, out, units, n, stride);
  return hipGetLastError();
}

hipError_t launch_express_reps(const ExpressView& ev, int units, uint64_t seed, int32_t* reps, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(units) * ev.n_batches_alloc * 2 * ev.n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(express_reps_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, ev, units, seed, reps);
  return hipGetLastError();
}

hipError_t launch_halve_input(const ExpressView& ev, int units, int e, int32_t* halve_in, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(units) * 4 * ev.n;
  hipLaunchKernelGGL(halve_input_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, ev, units, e, halve_in);
  return hipGetLastError();
}

hipError_t launch_express_final(const ExpressView& ev, int units, int S, int32_t* idx, float* w, int32_t* len,
                                int64_t cap, hipStream_t s) {
  if (!idx && !w && !len) return hipSuccess;
  hipLaunchKernelGGL(express_final_kernel, dim3(units), dim3(256), 0, s, ev, units, S, idx, w, len, cap);
  return hipGetLastError();
}

hipError_t launch_fill_coreset(const int32_t* src, int64_t src_stride, int units, int n, float w, int32_t* idx,
                               float* wout, int32_t* len, hipStream_t s) {
  if (!idx && !wout && !len) return hipSuccess;
  const int64_t total = static_cast<int64_t>(units) * n;
  hipLaunchKernelGGL(fill_coreset_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, src, src_stride, units, n, w,
                     idx, wout, len);
  return hipGetLastError();
}

hipError_t launch_philox_words(const uint64_t* ctr, int64_t n, uint64_t seed, uint64_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(philox_words_kernel, dim3(grid1d(n, 256)), dim3(256), 0, s, ctr, n, seed, out);
  return hipGetLastError();
}

ExpressSchedule express_schedule(int64_t S, int n) {
  ExpressSchedule sc{};
  sc.n = n;
  sc.nblk = static_cast<int>(S / n);
  // HALVE e happens after 4^(e+1) blocks; epoch e >= 1 holds three batches of 4^e blocks.
  int halves = 0;
  while ((1LL << (2 * (halves + 1))) <= sc.nblk) ++halves;
  sc.n_halves = halves;
  int done = 0, alloc = 0;
  for (int e = 1;; ++e) {
    const int64_t m = 1LL << (2 * e);
    const int64_t epoch_start = m;            // blocks
    if (epoch_start >= sc.nblk) break;
    for (int j = 0; j < 3; ++j) {
      const int64_t bstart = epoch_start + j * m;
      if (bstart < sc.nblk) ++alloc;
      if (bstart + m <= sc.nblk) ++done;
    }
  }
  sc.n_batches_done = done;
  sc.n_batches_alloc = alloc;
  sc.decisions = static_cast<int64_t>(3) * n * halves + static_cast<int64_t>(n) * done;
  return sc;
}

}  // namespace thin
