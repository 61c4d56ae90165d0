// Host-side helpers shared by the C ABI translation units (not part of the ABI).
#pragma once

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "../../include/thin_attn.h"
#include "internal.hpp"

struct thin_attn {
  thin_attn_config cfg;
  double delta;
  float scale;      // softmax scale of the attention kernels
  double scale64;   // the same scale in fp64 for kappa (decisions must match a float64 reference)
  std::string err;
  // launch timing records (label, start event, end event)
  bool timing = false;
  struct Rec {
    const char* label;
    hipEvent_t start, end;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;   // events not in use
};

namespace thinhost {

inline std::string g_create_error;

inline int fail(thin_attn* h, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (h)
    h->err = buf;
  else
    g_create_error = buf;
  return code;
}

inline bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

inline int64_t default_cache_size(int64_t S) {
  int64_t p = 2;
  while (p * p < S) p *= 2;
  return p;
}

inline int64_t cache_size(const thin_attn* h, int64_t S) { return h->cfg.n_out > 0 ? h->cfg.n_out : default_cache_size(S); }

// Compress depth j and base block s0 for S tokens and oversampling g.
inline void compress_depth(int64_t S, int g, int& j, int64_t& s0) {
  j = 0;
  int64_t four_g = 1;
  for (int i = 0; i < g && four_g <= S; ++i) four_g *= 4;
  while (S % (static_cast<int64_t>(1) << (2 * (j + 1))) == 0 && S / (static_cast<int64_t>(1) << (2 * (j + 1))) >= four_g &&
         j < 30)
    ++j;
  s0 = S >> (2 * j);
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace carve-up (same arithmetic for sizing and for forward).
struct Layout {
  size_t total = 0;
  size_t add(size_t bytes) {
    const size_t off = total;
    total += align256(bytes);
    return off;
  }
};

// Stratum length r of base subsampling (THIN_SUBSAMPLE_BASE) for a list of S
// points: the largest divisor r of the Compress base block s0 with r^2 <= s0
// and s0 / r >= 4^g; 1 without the flag or without a Compress level.
inline int64_t base_stride(const thin_attn* h, int64_t S) {
  if (!(h->cfg.flags & THIN_SUBSAMPLE_BASE)) return 1;
  int j;
  int64_t s0;
  compress_depth(S, h->cfg.g, j, s0);
  if (j == 0) return 1;
  int64_t four_g = 1;
  for (int i = 0; i < h->cfg.g && four_g <= s0; ++i) four_g *= 4;
  int64_t best = 1;
  for (int64_t r = 2; r * r <= s0; ++r)
    if (s0 % r == 0 && s0 / r >= four_g) best = r;
  return best;
}

struct UnmaskedPlan {
  int64_t r, L;   // base stratum length and the thinned list's length S / r
  int j;
  int64_t s0, n_out;
  size_t off_list, off_a, off_b, off_g;
  size_t bytes;
};

inline UnmaskedPlan plan_unmasked(const thin_attn* h, int64_t B, int64_t S0) {
  UnmaskedPlan p{};
  p.r = base_stride(h, S0);
  p.L = S0 / p.r;
  const int64_t S = p.L;
  compress_depth(S, h->cfg.g, p.j, p.s0);
  p.n_out = S >> p.j;
  const int64_t units = B * h->cfg.H_kv;
  Layout L;
  if (p.r > 1) p.off_list = L.add(sizeof(int32_t) * units * S);
  if (p.j > 0) {
    p.off_a = L.add(sizeof(int32_t) * units * S);
    p.off_b = L.add(sizeof(int32_t) * units * S);
    p.off_g = L.add(sizeof(double) * units * S * p.s0);   // every level needs S * s0 per unit
  }
  p.bytes = L.total;
  return p;
}

struct CausalPlan {
  thin::ExpressSchedule sc;
  size_t off_reps, off_bout, off_hin, off_hmid, off_hout, off_g;
  size_t bytes;
};

inline CausalPlan plan_causal(const thin_attn* h, int64_t B, int64_t S, int64_t n) {
  CausalPlan p{};
  p.sc = thin::express_schedule(S, static_cast<int>(n));
  const int64_t units = B * h->cfg.H_kv;
  Layout L;
  p.off_reps = L.add(sizeof(int32_t) * units * p.sc.n_batches_alloc * 2 * n);
  p.off_bout = L.add(sizeof(int32_t) * units * p.sc.n_batches_done * n);
  p.off_hin = L.add(sizeof(int32_t) * units * 4 * n);
  p.off_hmid = L.add(sizeof(int32_t) * units * 2 * n);
  p.off_hout = L.add(sizeof(int32_t) * units * p.sc.n_halves * n);
  int64_t g = 0;
  if (p.sc.n_batches_done) g = units * p.sc.n_batches_done * n * n;
  if (p.sc.n_halves) g = std::max<int64_t>(g, units * 4 * n * n);
  p.off_g = L.add(sizeof(double) * g);
  p.bytes = L.total;
  return p;
}

// Largest subsampling group reached must fit in a block (m / 2 <= n).
inline bool causal_schedule_ok(int64_t S, int64_t n) {
  const int64_t nblk = S / n;
  for (int e = 1; (static_cast<int64_t>(1) << (2 * e)) < nblk; ++e)
    if ((static_cast<int64_t>(1) << (2 * e - 1)) > n) return false;
  return true;
}

inline int check_dims(thin_attn* h, int64_t B, int64_t T, int64_t S, int causal) {
  if (B < 0 || T < 0 || S < 0) return fail(h, THIN_EINVAL, "negative size");
  if (B * h->cfg.H_kv > (1LL << 20)) return fail(h, THIN_ENOTSUP, "too many units (B * H_kv)");
  if (S >= (1LL << 30) || T >= (1LL << 30)) return fail(h, THIN_ENOTSUP, "sequence too long");
  {  // the attention addresses a batch entry's K / V rows with 32-bit byte offsets
    const int64_t row = static_cast<int64_t>(h->cfg.H_kv) * std::max(h->cfg.E, h->cfg.D) * (h->cfg.dtype == THIN_BF16 ? 2 : 4);
    if (row >= (1LL << 24) || S * row >= (1LL << 31))
      return fail(h, THIN_ENOTSUP, "K / V of one batch entry exceed 2 GiB (S * H_kv * max(E, D) * element size)");
  }
  if (causal) {
    if (T != S) return fail(h, THIN_EINVAL, "causal attention needs T == S (got T=%lld, S=%lld)", (long long)T, (long long)S);
    const int64_t n = cache_size(h, S);
    if (!pow2(n) || n < 2) return fail(h, THIN_EINVAL, "n_out must be a power of two >= 2");
    if (!causal_schedule_ok(S, n))
      return fail(h, THIN_ENOTSUP, "subsampling groups would exceed a block (S >= 2 n_out^2)");
  } else if (S == 0 && T > 0) {
    return fail(h, THIN_EINVAL, "S must be positive when T > 0");
  }
  return THIN_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// The pair Gram of the bins a walk is about to halve, with that walk's
// Philox parameters (the Gram launch also forms the walk's thresholds).
inline thin::GramLaunch gram_for(const thin::SweepLaunch& w, const thin::PointSource& src, double scale) {
  thin::GramLaunch g{};
  g.src = src;
  g.idx = w.idx_in;
  g.idx_stride = w.in_stride;
  g.idx_unit_stride = w.in_unit_stride;
  g.N = w.N;
  g.nbins = w.nbins;
  g.bins_per_unit = w.bins_per_unit;
  g.scale = scale;
  g.G = const_cast<double*>(w.G);
  g.seed = w.seed;
  g.tag = w.tag;
  g.bin_base = w.bin_base;
  g.delta = w.delta;
  g.greedy = w.greedy;
  return g;
}

// Sweep over the same bins as a Gram launch; the caller fills the outputs' strides and the log.
inline thin::SweepLaunch make_sweep(const thin_attn* h, const double* G, int N, int units, int bins_per_unit,
                             const int32_t* idx_in, int64_t in_unit_stride, int32_t* idx_out, uint64_t seed,
                             uint32_t tag, uint64_t bin_base) {
  thin::SweepLaunch s{};
  s.G = G;
  s.N = N;
  s.nbins = units * bins_per_unit;
  s.bins_per_unit = bins_per_unit;
  s.idx_in = idx_in;
  s.in_stride = N;
  s.in_unit_stride = in_unit_stride;
  s.idx_out = idx_out;
  s.out_stride = N / 2;
  s.dec = nullptr;
  s.seed = seed;
  s.tag = tag;
  s.bin_base = bin_base;
  s.delta = h->delta;
  s.greedy = (h->cfg.flags & THIN_GREEDY_SIGNS) != 0;
  return s;
}

#define THIN_HIP(call)                                                                 \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(h, THIN_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

inline hipError_t take_event(thin_attn* h, hipEvent_t* e) {
  if (!h->pool.empty()) {
    *e = h->pool.back();
    h->pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Bracket one launch with events when timing is on.
template <class F>
inline hipError_t timed(thin_attn* h, hipStream_t st, const char* label, F&& launch) {
  if (!h->timing) return launch();
  thin_attn::Rec r{label, nullptr, nullptr};
  hipError_t e = take_event(h, &r.start);
  if (e == hipSuccess) e = take_event(h, &r.end);
  if (e == hipSuccess) e = hipEventRecord(r.start, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.end, st);
  if (e == hipSuccess) h->recs.push_back(r);
  return e;
}

inline void release_timing(thin_attn* h) {
  for (auto& r : h->recs) {
    h->pool.push_back(r.start);
    h->pool.push_back(r.end);
  }
  h->recs.clear();
}

// Thinning of the causal path over S tokens of every unit (no attention):
// representatives, all batch halvings at once, then the HALVE chain.  Fills
// `ev` (lists live in `ws` as laid out by plan_causal).
inline int express_thin(thin_attn* h, const thin::PointSource& src, int units, const CausalPlan& p, uint64_t seed,
                        uint8_t* decisions, int64_t ndec, char* ws, hipStream_t st, thin::ExpressView& ev) {
  const int n = p.sc.n;
  ev = thin::ExpressView{};
  ev.n = n;
  ev.nblk = p.sc.nblk;
  ev.n_batches_done = p.sc.n_batches_done;
  ev.n_batches_alloc = p.sc.n_batches_alloc;
  ev.n_halves = p.sc.n_halves;
  int32_t* reps = reinterpret_cast<int32_t*>(ws + p.off_reps);
  int32_t* bout = reinterpret_cast<int32_t*>(ws + p.off_bout);
  int32_t* hin = reinterpret_cast<int32_t*>(ws + p.off_hin);
  int32_t* hmid = reinterpret_cast<int32_t*>(ws + p.off_hmid);
  int32_t* hout = reinterpret_cast<int32_t*>(ws + p.off_hout);
  double* G = reinterpret_cast<double*>(ws + p.off_g);
  ev.reps = reps;
  ev.batch_out = bout;
  ev.halve_out = hout;
  // 1. representatives of every thin-phase batch (data independent)
  THIN_HIP(timed(h, st, "express_reps", [&] { return thin::launch_express_reps(ev, units, seed, reps, st); }));
  // 2. all batch halvings at once: they read only representatives
  if (p.sc.n_batches_done > 0) {
    const int N = 2 * n;
    const int nb = p.sc.n_batches_done;
    const int64_t ustride = static_cast<int64_t>(p.sc.n_batches_alloc) * N;
    thin::SweepLaunch sl = make_sweep(h, G, N, units, nb, reps, ustride, bout, seed, thin::kTagBatch, 0);
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(gram_for(sl, src, h->scale64), st); }));
    sl.out_stride = n;
    sl.dec = decisions;
    sl.dec_per_unit = ndec;
    sl.dec_mode = 1;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, st); }));
  }
  // 3. the HALVE chain: halve twice, 4n -> 2n -> n
  for (int e = 0; e < p.sc.n_halves; ++e) {
    THIN_HIP(timed(h, st, "halve_input", [&] { return thin::launch_halve_input(ev, units, e, hin, st); }));
    thin::SweepLaunch s1 = make_sweep(h, G, 4 * n, units, 1, hin, 4 * n, hmid, seed, thin::kTagHalveFirst,
                                      static_cast<uint64_t>(e));
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(gram_for(s1, src, h->scale64), st); }));
    s1.out_stride = 2 * n;
    s1.dec = decisions;
    s1.dec_per_unit = ndec;
    s1.dec_base = static_cast<int64_t>(6) * n * e;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(s1, st); }));
    thin::SweepLaunch s2 = make_sweep(h, G, 2 * n, units, 1, hmid, 2 * n, hout + static_cast<int64_t>(e) * n, seed,
                                      thin::kTagHalveSecond, static_cast<uint64_t>(e));
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(gram_for(s2, src, h->scale64), st); }));
    s2.out_stride = static_cast<int64_t>(p.sc.n_halves) * n;   // unit u -> row u of [units][halves][n]
    s2.dec = decisions;
    s2.dec_per_unit = ndec;
    s2.dec_base = static_cast<int64_t>(6) * n * e + 2 * n;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(s2, st); }));
  }
  return THIN_OK;
}

}  // namespace thinhost
