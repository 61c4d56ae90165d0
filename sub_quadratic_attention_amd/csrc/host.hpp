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
  // Index errors found on the device: one int of pinned host memory mapped
  // into the device's address space (err_dev); kernels that read a caller's
  // token indices store 1 there when one lies outside [0, S).  Null when no
  // device was present at creation (nothing can be launched then).
  int* err_host = nullptr;
  int* err_dev = nullptr;
  // A second stream (default priority) on the device current at creation: the
  // causal path runs its batch halvings and the attention of finished epochs
  // there, beside the HALVE chain on the caller's stream, joined by events.
  // Null without a device (then everything runs on the caller's stream).
  hipStream_t side = nullptr;
  int dev = -1;
  static constexpr int kSyncEvents = 4;   // fork, batches done, epochs launch, join
  hipEvent_t sync_ev[kSyncEvents] = {};
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

// Bytes of one element of q, k, v.
inline int elt_bytes(int dtype) { return dtype == THIN_F32 ? 4 : (dtype == THIN_BF16 ? 2 : 1); }

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
  size_t off_keys, off_list, off_a, off_b, off_g, off_dig;
  size_t bytes;
};

// LDS one workgroup may hold on gfx950.
constexpr size_t kLdsLimit = 160 * 1024;

// Can the walk of a bin of N points run?  Bins of more than 128 points keep
// their thresholds, running sums and signs in LDS.
inline bool walk_fits(int64_t N) { return N <= 128 || thin::sweep_lds_bytes(static_cast<int>(N)) <= kLdsLimit; }

// Scratch of the exact integer pair Gram over npts points in bins of N (0:
// the fp64 tiles run, for the dtype, the head dims, the bin size or the flag).
inline size_t gram8_bytes(const thin_attn* h, int64_t N, int64_t npts) {
  if ((h->cfg.flags & THIN_FP64_GRAM) || N > (1 << 30) ||
      !thin::gram8_supported(h->cfg.dtype, h->cfg.E, h->cfg.D, static_cast<int>(N)) ||
      !thin::gram8_fits(h->cfg.dtype, npts, h->cfg.E, h->cfg.D))
    return 0;
  return thin::gram8_scratch_bytes(h->cfg.dtype, h->cfg.E, h->cfg.D, npts);
}

inline UnmaskedPlan plan_unmasked(const thin_attn* h, int64_t B, int64_t S0) {
  UnmaskedPlan p{};
  p.r = base_stride(h, S0);
  p.L = S0 / p.r;
  const int64_t S = p.L;
  compress_depth(S, h->cfg.g, p.j, p.s0);
  p.n_out = S >> p.j;
  const int64_t units = B * h->cfg.H_kv;
  Layout L;
  p.off_keys = L.add(sizeof(int32_t) * units * S0);   // a caller's key list, clamped into range
  if (p.r > 1) p.off_list = L.add(sizeof(int32_t) * units * S);
  if (p.j > 0) {
    p.off_a = L.add(sizeof(int32_t) * units * S);
    p.off_b = L.add(sizeof(int32_t) * units * S);
    p.off_g = L.add(sizeof(double) * units * S * p.s0);   // every level needs S * s0 per unit
    size_t dig = 0;   // level l halves bins of s0 2^(l+1) points over the S >> (l-1) points of a unit
    for (int l = 1; l <= p.j; ++l) dig = std::max(dig, gram8_bytes(h, p.s0 << (l + 1), units * (S >> (l - 1))));
    if (dig) p.off_dig = L.add(dig);
  }
  p.bytes = L.total;
  return p;
}

struct CausalPlan {
  thin::ExpressSchedule sc;
  size_t off_reps, off_bout, off_hin, off_hmid, off_hpos, off_hout, off_g, off_gh, off_digb, off_digh;
  size_t off_brow, off_hinrow, off_hrow;
  bool dig_b, dig_h;   // the integer Gram's scratch of the batch and the HALVE Grams
  bool dig_shared;     // one scratch: HALVE 0's points, then the batch points
  int64_t dig_rows;    // its rows
  size_t bytes;
};

// The batch halvings and the HALVE chain may run at once (on two streams).
// When both take the integer Gram they share one digit scratch: rows
// [0, units 4n) hold HALVE 0's points (the first 4n tokens of every unit),
// the batch points follow, each written by its own digit pass, and every
// later HALVE point is one of these (a HALVE's input is the last HALVE's
// output and three batch outputs), so the later HALVEs read their rows through
// the walks' row lists and run no digit pass.  Otherwise each keeps its own
// scratch and a HALVE's second halving reads its first's digits.
inline CausalPlan plan_causal(const thin_attn* h, int64_t B, int64_t S, int64_t n) {
  CausalPlan p{};
  p.sc = thin::express_schedule(S, static_cast<int>(n));
  const int64_t units = B * h->cfg.H_kv;
  Layout L;
  p.off_reps = L.add(sizeof(int32_t) * units * p.sc.n_batches_alloc * 2 * n);
  p.off_bout = L.add(sizeof(int32_t) * units * p.sc.n_batches_done * n);
  p.off_hin = L.add(sizeof(int32_t) * units * 4 * n);
  p.off_hmid = L.add(sizeof(int32_t) * units * 2 * n);
  p.off_hpos = L.add(sizeof(int32_t) * units * 2 * n);
  p.off_hout = L.add(sizeof(int32_t) * units * p.sc.n_halves * n);
  p.off_g = L.add(sizeof(double) * (p.sc.n_batches_done ? units * p.sc.n_batches_done * n * n : 0));
  p.off_gh = L.add(sizeof(double) * (p.sc.n_halves ? units * 4 * n * n : 0));
  const int64_t hrows = units * 4 * n, brows = units * p.sc.n_batches_done * 2 * n;
  const size_t ds = p.sc.n_batches_done && p.sc.n_halves ? gram8_bytes(h, 2 * n, hrows + brows) : 0;
  if (ds && gram8_bytes(h, 4 * n, hrows + brows)) {
    p.dig_shared = p.dig_b = p.dig_h = true;
    p.dig_rows = hrows + brows;
    p.off_digh = p.off_digb = L.add(ds);
    p.off_brow = L.add(sizeof(int32_t) * units * p.sc.n_batches_done * n);
    p.off_hinrow = L.add(sizeof(int32_t) * units * 4 * n);
    p.off_hrow = L.add(sizeof(int32_t) * units * p.sc.n_halves * n);
  } else {
    const size_t db = p.sc.n_batches_done ? gram8_bytes(h, 2 * n, brows) : 0;
    const size_t dh = p.sc.n_halves ? gram8_bytes(h, 4 * n, hrows) : 0;
    p.dig_b = db > 0;
    p.dig_h = dh > 0;
    p.dig_rows = hrows;
    if (db) p.off_digb = L.add(db);
    if (dh) p.off_digh = L.add(dh);
  }
  p.bytes = L.total;
  return p;
}

inline int check_dims(thin_attn* h, int64_t B, int64_t T, int64_t S, int causal) {
  if (B < 0 || T < 0 || S < 0) return fail(h, THIN_EINVAL, "negative size");
  if (B * h->cfg.H_kv > (1LL << 20)) return fail(h, THIN_ENOTSUP, "too many units (B * H_kv)");
  if (S >= (1LL << 30) || T >= (1LL << 30)) return fail(h, THIN_ENOTSUP, "sequence too long");
  {  // the attention addresses a batch entry's K / V rows with 32-bit byte offsets
    const int64_t row = static_cast<int64_t>(h->cfg.H_kv) * std::max(h->cfg.E, h->cfg.D) * elt_bytes(h->cfg.dtype);
    if (row >= (1LL << 24) || S * row >= (1LL << 31))
      return fail(h, THIN_ENOTSUP, "K / V of one batch entry exceed 2 GiB (S * H_kv * max(E, D) * element size)");
  }
  if (causal) {
    if (T != S) return fail(h, THIN_EINVAL, "causal attention needs T == S (got T=%lld, S=%lld)", (long long)T, (long long)S);
    const int64_t n = cache_size(h, S);
    if (!pow2(n) || n < 2) return fail(h, THIN_EINVAL, "n_out must be a power of two >= 2");
    if (S / n >= 4 && !walk_fits(4 * n))
      return fail(h, THIN_ENOTSUP, "n_out = %lld: the halving of a full cache (%lld points) exceeds the walk's LDS",
                  (long long)n, (long long)(4 * n));
  } else if (S == 0 && T > 0) {
    return fail(h, THIN_EINVAL, "S must be positive when T > 0");
  }
  return THIN_OK;
}

// The unmasked Compress of a list of S points: its largest bin must fit the walk.
inline int check_unmasked_plan(thin_attn* h, int64_t S) {
  const UnmaskedPlan p = plan_unmasked(h, 1, S);
  if (p.j > 0 && !walk_fits(p.s0 << (p.j + 1)))
    return fail(h, THIN_ENOTSUP, "S = %lld: the last Compress bin of %lld points exceeds the walk's LDS "
                                 "(base block %lld; choose a length with more factors of 4, or g)",
                (long long)S, (long long)(p.s0 << (p.j + 1)), (long long)p.s0);
  return THIN_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// A caller's index list read by an earlier call held entries outside [0, S):
// report it once (THIN_EINVAL) and clear the flag.  The flag is written by the
// device, so an error becomes visible here once that call's kernels finished.
inline int take_index_error(thin_attn* h) {
  if (!h->err_host) return THIN_OK;
  volatile int* f = h->err_host;
  if (*f == 0) return THIN_OK;
  *f = 0;
  return fail(h, THIN_EINVAL, "an earlier call on this handle read token indices outside [0, S) "
                              "(they were clamped into range; its outputs are not meaningful)");
}

// The pair Gram of the bins a walk is about to halve, with that walk's
// Philox parameters (the Gram launch also forms the walk's thresholds).
// dig: the integer Gram's scratch for these bins, or nullptr (fp64 tiles).
inline thin::GramLaunch gram_for(const thin::SweepLaunch& w, const thin::PointSource& src, double scale,
                                 unsigned char* dig = nullptr) {
  thin::GramLaunch g{};
  g.dig = dig;
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

// The pair Gram of a launch: the integer Gram's digit pass and tiles under
// their own timing labels, or the fp64 tiles; done (optional) is signalled
// when it completes.
inline int run_pair_gram(thin_attn* h, hipStream_t st, const thin::GramLaunch& g, hipEvent_t done = nullptr) {
  if (thin::gram8_runs(g)) {
    if (!g.dig_map) THIN_HIP(timed(h, st, "gram_digits", [&] { return thin::launch_gram8_digits(g, st); }));
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_gram8_tiles(g, st, done); }));
    return THIN_OK;
  }
  THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(g, st); }));
  if (done) THIN_HIP(hipEventRecord(done, st));
  return THIN_OK;
}

// The side stream if this call may use it (created on the current device).
inline hipStream_t side_stream(const thin_attn* h) {
  if (!h->side) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->dev) return nullptr;
  return h->side;
}

// `to` waits for the work enqueued so far on `from` (event k of the handle).
inline hipError_t stream_wait(thin_attn* h, hipStream_t from, hipStream_t to, int k) {
  if (from == to) return hipSuccess;
  hipError_t e = hipEventRecord(h->sync_ev[k], from);
  if (e == hipSuccess) e = hipStreamWaitEvent(to, h->sync_ev[k], 0);
  return e;
}

// Thinning of the causal path over S tokens of every unit: representatives,
// all batch halvings at once, then the HALVE chain; fills `ev` (lists in `ws`
// as laid out by plan_causal).  With `al` the attention runs too, an epoch at a
// time as soon as the state it reads exists: epoch 0 (blocks 0..3, still
// exact), epoch e >= 1 (blocks 4^e .. 4^(e+1) - 1, which read HALVE e - 1 and
// the batches of epoch e).  With H HALVEs, epochs 0 .. H-1 form one launch
// after HALVE H-2 and the last epoch (with the trailing partial block) one
// after HALVE H-1.  With a side stream the batch halvings and the first of
// those launches run there, beside the HALVE chain on `st` (which needs no
// batch before HALVE 1); `st` waits for all of it before the last launch.
inline int express_thin(thin_attn* h, const thin::PointSource& src, int units, const CausalPlan& p, uint64_t seed,
                        uint8_t* decisions, int64_t ndec, char* ws, hipStream_t st, thin::ExpressView& ev,
                        thin::AttnLaunch* al = nullptr) {
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
  int32_t* hpos = reinterpret_cast<int32_t*>(ws + p.off_hpos);
  int32_t* hout = reinterpret_cast<int32_t*>(ws + p.off_hout);
  double* Gb = reinterpret_cast<double*>(ws + p.off_g);
  double* Gh = reinterpret_cast<double*>(ws + p.off_gh);
  unsigned char* digb = p.dig_b ? reinterpret_cast<unsigned char*>(ws + p.off_digb) : nullptr;
  unsigned char* digh = p.dig_h ? reinterpret_cast<unsigned char*>(ws + p.off_digh) : nullptr;
  // digit-scratch rows of the batch outputs, a HALVE's input and the HALVE outputs (shared scratch)
  int32_t* brow = p.dig_shared ? reinterpret_cast<int32_t*>(ws + p.off_brow) : nullptr;
  int32_t* hinrow = p.dig_shared ? reinterpret_cast<int32_t*>(ws + p.off_hinrow) : nullptr;
  int32_t* hrow = p.dig_shared ? reinterpret_cast<int32_t*>(ws + p.off_hrow) : nullptr;
  // the integer Gram's launch of a HALVE's first halving: HALVE 0 (and every
  // HALVE without a shared scratch) writes rows [0, units 4n); the others read
  // their points' rows
  auto first_gram = [&](const thin::SweepLaunch& s1, int e) {
    thin::GramLaunch g = gram_for(s1, src, h->scale64, digh);
    g.dig_npts = p.dig_rows;
    if (p.dig_shared && e > 0) g.dig_map = hinrow;
    return g;
  };
  ev.reps = reps;
  ev.batch_out = bout;
  ev.halve_out = hout;
  const hipStream_t sx0 = side_stream(h);
  const hipStream_t sx = sx0 ? sx0 : st;
  int k = 0;   // next sync event
  const int dt = h->cfg.dtype;
  auto attention = [&](hipStream_t s, int64_t blk0, int64_t blk1) -> int {   // blocks [blk0, blk1) (S rows at the end)
    if (!al) return THIN_OK;
    thin::AttnLaunch a = *al;
    a.causal = 1;
    a.ev = ev;
    a.t0 = static_cast<int>(std::min<int64_t>(blk0 * n, a.T));
    a.t1 = static_cast<int>(std::min<int64_t>(blk1 * n, a.T));
    if (a.t1 <= a.t0) return THIN_OK;
    THIN_HIP(timed(h, s, "attention", [&] { return thin::launch_attention(a, dt, h->cfg.E, h->cfg.D, s); }));
    return THIN_OK;
  };
  const int64_t all_blocks = (static_cast<int64_t>(al ? al->T : 0) + n - 1) / n + 1;   // past every query row
  // 1. representatives of every thin-phase batch (data independent)
  THIN_HIP(timed(h, st, "express_reps", [&] { return thin::launch_express_reps(ev, units, seed, reps, st); }));
  if (p.sc.n_halves == 0) {   // no HALVE: still exact (or only batch halvings past the last block)
    return attention(st, 0, all_blocks);
  }
  // HALVE e halves twice, 4n -> 2n -> n, on st; HALVE e >= 1 reads batches 3(e-1) ..
  auto halve_first_gram = [&](int e, hipEvent_t done) -> int {
    const thin::HalveRows rows{hrow, brow, e > 0 ? hinrow : nullptr};
    THIN_HIP(timed(h, st, "halve_input", [&] { return thin::launch_halve_input(ev, units, e, hin, st, rows); }));
    thin::SweepLaunch s1 = make_sweep(h, Gh, 4 * n, units, 1, hin, 4 * n, hmid, seed, thin::kTagHalveFirst,
                                      static_cast<uint64_t>(e));
    if (const int rg = run_pair_gram(h, st, first_gram(s1, e), done)) return rg;
    return THIN_OK;
  };
  auto halve_rest = [&](int e, hipEvent_t done) -> int {
    thin::SweepLaunch s1 = make_sweep(h, Gh, 4 * n, units, 1, hin, 4 * n, hmid, seed, thin::kTagHalveFirst,
                                      static_cast<uint64_t>(e));
    // the second halving's points are among the first's: with the integer
    // Gram, it reads their digit rows, which the first walk lists
    const thin::GramLaunch g1 = first_gram(s1, e);
    const bool reuse = digh && thin::gram8_runs(g1);
    s1.out_stride = 2 * n;
    s1.row_out = reuse ? hpos : nullptr;
    s1.row_map = g1.dig_map;
    s1.dec = decisions;
    s1.dec_per_unit = ndec;
    s1.dec_base = static_cast<int64_t>(6) * n * e;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(s1, st); }));
    thin::SweepLaunch s2 = make_sweep(h, Gh, 2 * n, units, 1, hmid, 2 * n, hout + static_cast<int64_t>(e) * n, seed,
                                      thin::kTagHalveSecond, static_cast<uint64_t>(e));
    thin::GramLaunch g2 = gram_for(s2, src, h->scale64, digh);
    if (reuse) {
      g2.dig_map = hpos;
      g2.dig_npts = p.dig_rows;
    }
    if (const int rg = run_pair_gram(h, st, g2)) return rg;
    s2.out_stride = static_cast<int64_t>(p.sc.n_halves) * n;   // unit u -> row u of [units][halves][n]
    if (p.dig_shared) {   // the HALVE output's rows, for the next HALVE's input
      s2.row_out = hrow + static_cast<int64_t>(e) * n;
      s2.row_map = hpos;
    }
    s2.dec = decisions;
    s2.dec_per_unit = ndec;
    s2.dec_base = static_cast<int64_t>(6) * n * e + 2 * n;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(s2, st, done); }));
    return THIN_OK;
  };
  // an event for st -> sx dependencies, signalled by the dispatch of the
  // kernel it follows (a separate marker in st's queue delays st's next kernel)
  auto fork_event = [&]() -> hipEvent_t { return sx != st ? h->sync_ev[k++] : nullptr; };
  int rc = THIN_OK;
  // 2. HALVE 0's first Gram, then the fork: the side takes every batch halving
  // (they read only representatives).  Forking after that Gram rather than
  // before it keeps the batch Gram from crowding the small walks of HALVE 0
  // out of the compute units (a walk launched while a large Gram holds every
  // unit waits for it to drain); with a single HALVE, the exact epoch's
  // attention goes to the side first
  {
    const hipEvent_t fork = fork_event();
    if ((rc = halve_first_gram(0, fork))) return rc;
    if (fork) THIN_HIP(hipStreamWaitEvent(sx, fork, 0));
  }
  if (p.sc.n_halves == 1 && (rc = attention(sx, 0, 4))) return rc;
  const int k_batches = k++;   // marks the batch halvings on the side
  const hipEvent_t batches_done = sx != st ? h->sync_ev[k_batches] : nullptr;
  if (p.sc.n_batches_done > 0) {
    const int N = 2 * n;
    const int nb = p.sc.n_batches_done;
    const int64_t ustride = static_cast<int64_t>(p.sc.n_batches_alloc) * N;
    thin::SweepLaunch sl = make_sweep(h, Gb, N, units, nb, reps, ustride, bout, seed, thin::kTagBatch, 0);
    thin::GramLaunch gb = gram_for(sl, src, h->scale64, digb);
    if (p.dig_shared) {   // the batch points' rows follow HALVE 0's
      gb.dig_npts = p.dig_rows;
      gb.dig_row0 = static_cast<int64_t>(units) * 4 * n;
      sl.row_out = brow;
      sl.row0 = gb.dig_row0;
    }
    if (const int rg = run_pair_gram(h, sx, gb)) return rg;
    sl.out_stride = n;
    sl.dec = decisions;
    sl.dec_per_unit = ndec;
    sl.dec_mode = 1;
    THIN_HIP(timed(h, sx, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, sx, batches_done); }));
  } else if (batches_done) {
    THIN_HIP(hipEventRecord(batches_done, sx));
  }
  // 3. the HALVE chain on st
  const int H = p.sc.n_halves;
  for (int e = 0; e < H; ++e) {
    if (e == 1 && sx != st) THIN_HIP(hipStreamWaitEvent(st, h->sync_ev[k_batches], 0));
    if (e > 0 && (rc = halve_first_gram(e, nullptr))) return rc;
    // epoch e + 1 reads HALVE e and the batches of its epoch (done on the side before this
    // point).  Every epoch but the last goes in one launch on the side once the HALVE before
    // the last is done, beside the last HALVE; the last epoch follows that HALVE on st
    const hipEvent_t epochs = e == H - 2 && al ? fork_event() : nullptr;
    if ((rc = halve_rest(e, epochs))) return rc;
    if (e == H - 2 && al) {
      if (epochs) THIN_HIP(hipStreamWaitEvent(sx, epochs, 0));
      if ((rc = attention(sx, 0, static_cast<int64_t>(1) << (2 * H)))) return rc;
    }
    if (e == H - 1) {   // the last epoch on st (beside the side's tail), then st takes in the side's work
      // the last epoch reads the batches of its own epoch: with a single HALVE
      // st has not waited for them yet (with more, HALVE 1 did)
      if (H == 1 && sx != st) THIN_HIP(hipStreamWaitEvent(st, h->sync_ev[k_batches], 0));
      if ((rc = attention(st, static_cast<int64_t>(1) << (2 * H), all_blocks))) return rc;
      THIN_HIP(stream_wait(h, sx, st, k++));
    }
  }
  return THIN_OK;
}

}  // namespace thinhost
