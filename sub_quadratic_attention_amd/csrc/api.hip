// C ABI of the thin-attention library: validation, workspace layout and the
// launch sequence of the unmasked (Compress) and causal (Express) paths.

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

namespace {

std::string g_create_error;

int fail(thin_attn* h, int code, const char* fmt, ...) {
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

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t default_cache_size(int64_t S) {
  int64_t p = 2;
  while (p * p < S) p *= 2;
  return p;
}

int64_t cache_size(const thin_attn* h, int64_t S) { return h->cfg.n_out > 0 ? h->cfg.n_out : default_cache_size(S); }

// Compress depth j and base block s0 for S tokens and oversampling g.
void compress_depth(int64_t S, int g, int& j, int64_t& s0) {
  j = 0;
  int64_t four_g = 1;
  for (int i = 0; i < g && four_g <= S; ++i) four_g *= 4;
  while (S % (static_cast<int64_t>(1) << (2 * (j + 1))) == 0 && S / (static_cast<int64_t>(1) << (2 * (j + 1))) >= four_g &&
         j < 30)
    ++j;
  s0 = S >> (2 * j);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace carve-up (same arithmetic for sizing and for forward).
struct Layout {
  size_t total = 0;
  size_t add(size_t bytes) {
    const size_t off = total;
    total += align256(bytes);
    return off;
  }
};

struct UnmaskedPlan {
  int j;
  int64_t s0, n_out;
  size_t off_a, off_b, off_g;
  size_t bytes;
};

UnmaskedPlan plan_unmasked(const thin_attn* h, int64_t B, int64_t S) {
  UnmaskedPlan p{};
  compress_depth(S, h->cfg.g, p.j, p.s0);
  p.n_out = S >> p.j;
  const int64_t units = B * h->cfg.H_kv;
  Layout L;
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

CausalPlan plan_causal(const thin_attn* h, int64_t B, int64_t S) {
  CausalPlan p{};
  const int64_t n = cache_size(h, S);
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
bool causal_schedule_ok(int64_t S, int64_t n) {
  const int64_t nblk = S / n;
  for (int e = 1; (static_cast<int64_t>(1) << (2 * e)) < nblk; ++e)
    if ((static_cast<int64_t>(1) << (2 * e - 1)) > n) return false;
  return true;
}

int check_dims(thin_attn* h, int64_t B, int64_t T, int64_t S, int causal) {
  if (B < 0 || T < 0 || S < 0) return fail(h, THIN_EINVAL, "negative size");
  if (B * h->cfg.H_kv > (1LL << 20)) return fail(h, THIN_ENOTSUP, "too many units (B * H_kv)");
  if (S >= (1LL << 30) || T >= (1LL << 30)) return fail(h, THIN_ENOTSUP, "sequence too long");
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

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

thin::GramLaunch make_gram(const thin::PointSource& src, const int32_t* idx, int N, int64_t unit_stride, int units,
                           int bins_per_unit, double scale, double* G) {
  thin::GramLaunch g{};
  g.src = src;
  g.idx = idx;
  g.idx_stride = N;
  g.idx_unit_stride = unit_stride;
  g.N = N;
  g.nbins = units * bins_per_unit;
  g.bins_per_unit = bins_per_unit;
  g.scale = scale;
  g.G = G;
  return g;
}

// Sweep over the same bins as a Gram launch; the caller fills the outputs' strides and the log.
thin::SweepLaunch make_sweep(const thin_attn* h, const double* G, int N, int units, int bins_per_unit,
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
  return s;
}

#define THIN_HIP(call)                                                                 \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(h, THIN_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

hipError_t take_event(thin_attn* h, hipEvent_t* e) {
  if (!h->pool.empty()) {
    *e = h->pool.back();
    h->pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Bracket one launch with events when timing is on.
template <class F>
hipError_t timed(thin_attn* h, hipStream_t st, const char* label, F&& launch) {
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

void release_timing(thin_attn* h) {
  for (auto& r : h->recs) {
    h->pool.push_back(r.start);
    h->pool.push_back(r.end);
  }
  h->recs.clear();
}

}  // namespace

extern "C" {

int thin_attn_create(const thin_attn_config* cfg, thin_attn_t** out) {
  if (!cfg || !out) return fail(nullptr, THIN_EINVAL, "null argument");
  const thin_attn_config& c = *cfg;
  if (c.dtype != THIN_F32 && c.dtype != THIN_BF16) return fail(nullptr, THIN_EINVAL, "unknown dtype %d", c.dtype);
  if (c.E <= 0 || c.D <= 0 || c.H <= 0 || c.H_kv <= 0) return fail(nullptr, THIN_EINVAL, "dims must be positive");
  if (c.H % c.H_kv != 0) return fail(nullptr, THIN_EINVAL, "H %% H_kv != 0");
  if (c.g < 0) return fail(nullptr, THIN_EINVAL, "g must be >= 0");
  if (c.n_out < 0 || (c.n_out > 0 && (!pow2(c.n_out) || c.n_out < 2)))
    return fail(nullptr, THIN_EINVAL, "n_out must be 0 or a power of two >= 2");
  if (c.flags != 0) return fail(nullptr, THIN_EINVAL, "flags must be 0");
  if (!(c.scale >= 0.0f) || !std::isfinite(c.scale)) return fail(nullptr, THIN_EINVAL, "scale must be finite and >= 0");
  if (!thin::attention_supported(c.dtype == THIN_BF16, c.E, c.D))
    return fail(nullptr, THIN_ENOTSUP, "head dims E=%d D=%d not built for this dtype", c.E, c.D);
  thin_attn* h = new thin_attn();
  h->cfg = c;
  h->delta = c.delta > 0.0 ? c.delta : 0.5;
  h->scale64 = c.scale > 0.0f ? static_cast<double>(c.scale) : 1.0 / sqrt(static_cast<double>(c.E));
  h->scale = static_cast<float>(h->scale64);
  *out = h;
  return THIN_OK;
}

int thin_attn_destroy(thin_attn_t* h) {
  if (!h) return THIN_OK;
  release_timing(h);
  for (auto e : h->pool) (void)hipEventDestroy(e);
  delete h;
  return THIN_OK;
}

const char* thin_attn_last_error(const thin_attn_t* h) { return h ? h->err.c_str() : g_create_error.c_str(); }

int64_t thin_attn_coreset_size(const thin_attn_t* h, int64_t S, int causal) {
  if (!h || S < 0) return THIN_EINVAL;
  if (causal) return cache_size(h, S);
  int j;
  int64_t s0;
  compress_depth(S, h->cfg.g, j, s0);
  return S >> j;
}

int64_t thin_attn_coreset_capacity(const thin_attn_t* h, int64_t S, int causal) {
  const int64_t n = thin_attn_coreset_size(h, S, causal);
  if (n < 0) return n;
  return causal ? 6 * n : n;
}

int64_t thin_attn_decision_count(const thin_attn_t* h, int64_t S, int causal) {
  if (!h || S < 0) return THIN_EINVAL;
  if (causal) {
    const int64_t n = cache_size(h, S);
    if (!causal_schedule_ok(S, n)) return THIN_ENOTSUP;
    return thin::express_schedule(S, static_cast<int>(n)).decisions;
  }
  int j;
  int64_t s0;
  compress_depth(S, h->cfg.g, j, s0);
  int64_t total = 0;
  for (int l = 1; l <= j; ++l) total += (S / (s0 << (2 * l))) * (s0 << l);
  return total;
}

size_t thin_attn_workspace_size(const thin_attn_t* h, int64_t B, int64_t T, int64_t S, int causal) {
  if (!h || B < 0 || T < 0 || S < 0) return 0;
  (void)T;
  if (causal) {
    const int64_t n = cache_size(h, S);
    if (!causal_schedule_ok(S, n)) return 0;
    return std::max<size_t>(plan_causal(h, B, S).bytes, 256);
  }
  return std::max<size_t>(plan_unmasked(h, B, S).bytes, 256);
}

int thin_attn_set_timing(thin_attn_t* h, int enable) {
  if (!h) return THIN_EINVAL;
  release_timing(h);
  if (!enable) {
    for (auto e : h->pool) (void)hipEventDestroy(e);
    h->pool.clear();
  }
  h->timing = enable != 0;
  return THIN_OK;
}

int64_t thin_attn_timing_count(const thin_attn_t* h) { return h ? static_cast<int64_t>(h->recs.size()) : THIN_EINVAL; }

int thin_attn_timing_read(thin_attn_t* h, int64_t i, char* label, size_t label_len, float* ms) {
  if (!h) return THIN_EINVAL;
  if (i < 0 || i >= static_cast<int64_t>(h->recs.size())) return fail(h, THIN_EINVAL, "no timing record %lld", (long long)i);
  const auto& r = h->recs[static_cast<size_t>(i)];
  THIN_HIP(hipEventSynchronize(r.end));
  float t = 0.f;
  THIN_HIP(hipEventElapsedTime(&t, r.start, r.end));
  if (ms) *ms = t;
  if (label && label_len) {
    snprintf(label, label_len, "%s", r.label);
  }
  return THIN_OK;
}

int thin_attn_forward(thin_attn_t* h, const void* q, const void* k, const void* v, int64_t B, int64_t T, int64_t S,
                      int causal, uint64_t seed, void* out, int32_t* coreset_idx, float* coreset_w,
                      int32_t* coreset_len, uint8_t* decisions, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  if (causal != 0 && causal != 1) return fail(h, THIN_EINVAL, "causal must be 0 or 1");
  int rc = check_dims(h, B, T, S, causal);
  if (rc) return rc;
  if (B * T == 0) return THIN_OK;
  if (!q || !k || !v || !out) return fail(h, THIN_EINVAL, "null q, k, v or out");
  const size_t need = thin_attn_workspace_size(h, B, T, S, causal);
  if (need > 256 && (!workspace || workspace_bytes < need))
    return fail(h, THIN_ENOMEM, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(h, THIN_EINVAL, "workspace must be 256-byte aligned");
  const hipStream_t st = as_stream(stream);
  const thin_attn_config& c = h->cfg;
  const int units = static_cast<int>(B * c.H_kv);
  char* ws = static_cast<char*>(workspace);
  const int bf16 = c.dtype == THIN_BF16;
  thin::PointSource src{k, v, S, c.H_kv, c.E, c.D, bf16};
  const int64_t ndec = thin_attn_decision_count(h, S, causal);

  thin::AttnLaunch al{};
  al.q = q;
  al.k = k;
  al.v = v;
  al.out = out;
  al.B = static_cast<int>(B);
  al.T = static_cast<int>(T);
  al.S = static_cast<int>(S);
  al.H = c.H;
  al.H_kv = c.H_kv;
  al.scale = h->scale;

  if (!causal) {
    const UnmaskedPlan p = plan_unmasked(h, B, S);
    const int32_t* coreset = nullptr;
    if (p.j > 0) {
      int32_t* a = reinterpret_cast<int32_t*>(ws + p.off_a);
      int32_t* b = reinterpret_cast<int32_t*>(ws + p.off_b);
      double* G = reinterpret_cast<double*>(ws + p.off_g);
      THIN_HIP(timed(h, st, "iota", [&] { return thin::launch_iota(a, units, S, S, st); }));
      int64_t dec_base = 0;
      for (int l = 1; l <= p.j; ++l) {
        // level l: bins of N = s0 2^(l+1) points; every level's lists are dense [unit][S >> (l-1)]
        const int N = static_cast<int>(p.s0 << (l + 1));
        const int bins = static_cast<int>(S / (p.s0 << (2 * l)));
        const int64_t in_unit = S >> (l - 1);
        THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(make_gram(src, a, N, in_unit, units, bins, h->scale64, G), st); }));
        thin::SweepLaunch sl = make_sweep(h, G, N, units, bins, a, in_unit, b, seed, thin::kTagCompress,
                                          static_cast<uint64_t>(l) << 20);
        sl.out_stride = N / 2;
        sl.dec = decisions;
        sl.dec_per_unit = ndec;
        sl.dec_base = dec_base;
        THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, st); }));
        dec_base += static_cast<int64_t>(bins) * (N / 2);
        std::swap(a, b);
      }
      coreset = a;   // the last level's output: dense [unit][n_out]
    }
    const float w = static_cast<float>(static_cast<int64_t>(1) << p.j);
    al.causal = 0;
    al.cs_idx = coreset;
    al.cs_w = nullptr;
    al.cs_n = static_cast<int>(coreset ? p.n_out : S);
    al.cs_stride = coreset ? p.n_out : 0;
    al.cs_lnw = coreset ? logf(w) : 0.f;
    THIN_HIP(timed(h, st, "attention", [&] { return thin::launch_attention(al, bf16, c.E, c.D, st); }));
    THIN_HIP(thin::launch_fill_coreset(coreset, al.cs_stride, units, static_cast<int>(p.n_out), w, coreset_idx,
                                       coreset_w, coreset_len, st));
    return THIN_OK;
  }

  // ---- causal: Thinformer Express ----
  const CausalPlan p = plan_causal(h, B, S);
  const int n = p.sc.n;
  thin::ExpressView ev{};
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
    thin::GramLaunch gl = make_gram(src, reps, N, static_cast<int64_t>(p.sc.n_batches_alloc) * N, units, nb,
                                    h->scale64, G);
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(gl, st); }));
    thin::SweepLaunch sl = make_sweep(h, G, N, units, nb, reps, static_cast<int64_t>(p.sc.n_batches_alloc) * N, bout,
                                      seed, thin::kTagBatch, 0);
    sl.out_stride = n;
    sl.dec = decisions;
    sl.dec_per_unit = ndec;
    sl.dec_mode = 1;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, st); }));
  }
  // 3. the HALVE chain: halve twice, 4n -> 2n -> n
  for (int e = 0; e < p.sc.n_halves; ++e) {
    THIN_HIP(timed(h, st, "halve_input", [&] { return thin::launch_halve_input(ev, units, e, hin, st); }));
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(make_gram(src, hin, 4 * n, 4 * n, units, 1, h->scale64, G), st); }));
    thin::SweepLaunch s1 = make_sweep(h, G, 4 * n, units, 1, hin, 4 * n, hmid, seed, thin::kTagHalveFirst,
                                      static_cast<uint64_t>(e));
    s1.out_stride = 2 * n;
    s1.dec = decisions;
    s1.dec_per_unit = ndec;
    s1.dec_base = static_cast<int64_t>(6) * n * e;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(s1, st); }));
    THIN_HIP(timed(h, st, "pair_gram", [&] { return thin::launch_pair_gram(make_gram(src, hmid, 2 * n, 2 * n, units, 1, h->scale64, G), st); }));
    thin::SweepLaunch s2 = make_sweep(h, G, 2 * n, units, 1, hmid, 2 * n, hout + static_cast<int64_t>(e) * n, seed,
                                      thin::kTagHalveSecond, static_cast<uint64_t>(e));
    s2.out_stride = static_cast<int64_t>(p.sc.n_halves) * n;   // one bin per unit: unit u -> row u of [units][halves][n]
    s2.dec = decisions;
    s2.dec_per_unit = ndec;
    s2.dec_base = static_cast<int64_t>(6) * n * e + 2 * n;
    THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(s2, st); }));
  }
  al.causal = 1;
  al.ev = ev;
  THIN_HIP(timed(h, st, "attention", [&] { return thin::launch_attention(al, bf16, c.E, c.D, st); }));
  THIN_HIP(thin::launch_express_final(ev, units, static_cast<int>(S), coreset_idx, coreset_w, coreset_len, 6LL * n,
                                      st));
  return THIN_OK;
}

int thin_attn_coreset_attention(thin_attn_t* h, const void* q, const void* k, const void* v, int64_t B, int64_t T,
                                int64_t S, const int32_t* idx, const float* w, int64_t n, void* out, void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  int rc = check_dims(h, B, T, S, 0);
  if (rc) return rc;
  if (B * T == 0) return THIN_OK;
  if (!q || !k || !v || !out) return fail(h, THIN_EINVAL, "null q, k, v or out");
  if (n <= 0 || n > S) return fail(h, THIN_EINVAL, "coreset size must be in [1, S]");
  if (!idx && n != S) return fail(h, THIN_EINVAL, "idx may be NULL only with n == S");
  const thin_attn_config& c = h->cfg;
  thin::AttnLaunch al{};
  al.q = q;
  al.k = k;
  al.v = v;
  al.out = out;
  al.B = static_cast<int>(B);
  al.T = static_cast<int>(T);
  al.S = static_cast<int>(S);
  al.H = c.H;
  al.H_kv = c.H_kv;
  al.scale = h->scale;
  al.causal = 0;
  al.cs_idx = idx;
  al.cs_w = w;
  al.cs_n = static_cast<int>(n);
  al.cs_stride = idx ? n : 0;
  al.cs_lnw = 0.f;
  THIN_HIP(thin::launch_attention(al, c.dtype == THIN_BF16, c.E, c.D, as_stream(stream)));
  return THIN_OK;
}

int thin_attn_halving(thin_attn_t* h, const void* k, const void* v, int64_t B, int64_t S, const int32_t* points,
                      int64_t N, uint64_t seed, uint32_t tag, uint64_t bin, int32_t* kept, uint8_t* decisions,
                      double* gram, void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  if (B < 0 || S <= 0) return fail(h, THIN_EINVAL, "bad B or S");
  if (N < 2 || N > 2048 || (N & 1)) return fail(h, THIN_EINVAL, "N must be even and in [2, 2048]");
  if (tag > 4) return fail(h, THIN_EINVAL, "unknown tag %u", tag);
  if (B == 0) return THIN_OK;
  if (!k || !v || !points || !kept || !gram) return fail(h, THIN_EINVAL, "null k, v, points, kept or gram");
  const thin_attn_config& c = h->cfg;
  const int units = static_cast<int>(B * c.H_kv);
  const hipStream_t st = as_stream(stream);
  thin::PointSource src{k, v, S, c.H_kv, c.E, c.D, c.dtype == THIN_BF16};
  const int n = static_cast<int>(N);
  THIN_HIP(thin::launch_pair_gram(make_gram(src, points, n, n, units, 1, h->scale64, gram), st));
  thin::SweepLaunch sl = make_sweep(h, gram, n, units, 1, points, n, kept, seed, tag, bin);
  sl.dec = decisions;
  sl.dec_per_unit = n / 2;
  THIN_HIP(thin::launch_halving_sweep(sl, st));
  return THIN_OK;
}

int thin_attn_philox(const uint64_t* counters, int64_t n, uint64_t seed, uint64_t* out, void* stream) {
  thin_attn* h = nullptr;
  if (n < 0 || (n > 0 && (!counters || !out))) return THIN_EINVAL;
  THIN_HIP(thin::launch_philox_words(counters, n, seed, out, as_stream(stream)));
  return THIN_OK;
}

}  // extern "C"
