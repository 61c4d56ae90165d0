// C ABI of the thin-attention library: validation, workspace layout and the
// launch sequence of the unmasked (Compress) and causal (Express) paths.

#include <mutex>

#include "host.hpp"

using namespace thinhost;

// ---- thin_attn_forward_static: thin_attn_forward on a library-owned scratch ----
//
// The scratch lives in this file's device array (one copy per GPU, resident
// until the process ends).  Its name is only a host-side stand-in: the device
// address of each GPU's copy is looked up once per device, with that device
// current, and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = THIN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null: not looked up yet)

int static_scratch(thin_attn* h, void** out) {
  int dev = -1;
  THIN_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(h, THIN_ENOTSUP, "device %d beyond the static scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    THIN_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255))
      return fail(h, THIN_EHIP, "static scratch of device %d has no usable address", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return THIN_OK;
}
}  // namespace

extern "C" {

int thin_attn_create(const thin_attn_config* cfg, thin_attn_t** out) {
  if (!cfg || !out) return fail(nullptr, THIN_EINVAL, "null argument");
  const thin_attn_config& c = *cfg;
  if (c.dtype != THIN_F32 && c.dtype != THIN_BF16 && c.dtype != THIN_FP8_E4M3)
    return fail(nullptr, THIN_EINVAL, "unknown dtype %d", c.dtype);
  if (c.E <= 0 || c.D <= 0 || c.H <= 0 || c.H_kv <= 0) return fail(nullptr, THIN_EINVAL, "dims must be positive");
  if (c.H % c.H_kv != 0) return fail(nullptr, THIN_EINVAL, "H %% H_kv != 0");
  if (c.g < 0) return fail(nullptr, THIN_EINVAL, "g must be >= 0");
  if (c.n_out < 0 || (c.n_out > 0 && (!pow2(c.n_out) || c.n_out < 2)))
    return fail(nullptr, THIN_EINVAL, "n_out must be 0 or a power of two >= 2");
  if (c.flags & ~static_cast<uint32_t>(THIN_GREEDY_SIGNS | THIN_SUBSAMPLE_BASE | THIN_ONE_STREAM | THIN_FP64_GRAM))
    return fail(nullptr, THIN_EINVAL, "unknown flags 0x%x", c.flags);
  if (!(c.scale >= 0.0f) || !std::isfinite(c.scale)) return fail(nullptr, THIN_EINVAL, "scale must be finite and >= 0");
  if (!thin::attention_supported(c.dtype, c.E, c.D))
    return fail(nullptr, THIN_ENOTSUP, "head dims E=%d D=%d not built for this dtype", c.E, c.D);
  thin_attn* h = new thin_attn();
  h->cfg = c;
  // the device-visible index-error flag (pinned host memory); without a device
  // there is none, and nothing can be launched anyway
  void* flag = nullptr;
  if (hipHostMalloc(&flag, sizeof(int), hipHostMallocMapped | hipHostMallocPortable | hipHostMallocCoherent) ==
      hipSuccess) {
    void* dflag = nullptr;
    if (hipHostGetDevicePointer(&dflag, flag, 0) == hipSuccess) {
      h->err_host = static_cast<int*>(flag);
      h->err_dev = static_cast<int*>(dflag);
      *h->err_host = 0;
    } else {
      (void)hipHostFree(flag);
    }
  }
  {  // the side stream of the causal path and its events, on the current device
    int dev = -1;
    hipStream_t side = nullptr;
    if (!(c.flags & THIN_ONE_STREAM) && hipGetDevice(&dev) == hipSuccess &&
        hipStreamCreateWithFlags(&side, hipStreamNonBlocking) == hipSuccess) {
      bool ok = true;
      for (int i = 0; i < thin_attn::kSyncEvents && ok; ++i)
        ok = hipEventCreateWithFlags(&h->sync_ev[i], hipEventDisableTiming) == hipSuccess;
      if (ok) {
        h->side = side;
        h->dev = dev;
      } else {
        for (auto& e : h->sync_ev)
          if (e) (void)hipEventDestroy(e), e = nullptr;
        (void)hipStreamDestroy(side);
      }
    }
  }
  {  // the static scratch's address on the current device (thin_attn_forward_static)
    void* sp = nullptr;
    if (static_scratch(h, &sp) != THIN_OK) h->err.clear();
  }
  (void)hipGetLastError();   // a failed probe above leaves no error behind
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
  if (h->err_host) (void)hipHostFree(h->err_host);
  if (h->side) {   // the side stream's work was joined into the caller's stream by every call
    (void)hipStreamSynchronize(h->side);
    (void)hipStreamDestroy(h->side);
  }
  for (auto e : h->sync_ev)
    if (e) (void)hipEventDestroy(e);
  delete h;
  return THIN_OK;
}

const char* thin_attn_last_error(const thin_attn_t* h) { return h ? h->err.c_str() : g_create_error.c_str(); }

int thin_attn_status(thin_attn_t* h, void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  THIN_HIP(hipStreamSynchronize(as_stream(stream)));
  return take_index_error(h);
}

int64_t thin_attn_coreset_size(const thin_attn_t* h, int64_t S, int causal) {
  if (!h || S < 0) return THIN_EINVAL;
  if (causal) return cache_size(h, S);
  const int64_t Lp = S / base_stride(h, S);
  int j;
  int64_t s0;
  compress_depth(Lp, h->cfg.g, j, s0);
  return Lp >> j;
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
    return thin::express_schedule(S, static_cast<int>(n)).decisions;
  }
  const int64_t Lp = S / base_stride(h, S);
  int j;
  int64_t s0;
  compress_depth(Lp, h->cfg.g, j, s0);
  int64_t total = 0;
  for (int l = 1; l <= j; ++l) total += (Lp / (s0 << (2 * l))) * (s0 << l);
  return total;
}

size_t thin_attn_workspace_size(const thin_attn_t* h, int64_t B, int64_t T, int64_t S, int causal) {
  if (!h || B < 0 || T < 0 || S < 0) return 0;
  (void)T;
  if (causal) {
    const int64_t n = cache_size(h, S);
    return std::max<size_t>(plan_causal(h, B, S, n).bytes, 256);
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

// Unmasked path: the Compress recursion over a key list per unit (keys ==
// nullptr: tokens 0 .. L-1 in order, L == S), then coreset attention.
static int unmasked_path(thin_attn_t* h, const thin::PointSource& src, thin::AttnLaunch& al, const int32_t* keys,
                         int64_t L, int units, uint64_t seed, uint8_t* decisions, int64_t ndec, char* ws,
                         hipStream_t st, int32_t* coreset_idx, float* coreset_w, int32_t* coreset_len) {
  const thin_attn_config& c = h->cfg;
  const int dt = c.dtype;
  const int64_t B = al.B;
  const UnmaskedPlan p = plan_unmasked(h, B, L);
  if (p.r > 1) {   // base subsampling: one point per stratum of r; the Compress runs on L / r points
    int32_t* list = reinterpret_cast<int32_t*>(ws + p.off_list);
    THIN_HIP(timed(h, st, "base_sample", [&] { return thin::launch_base_sample(keys, L, units, p.r, seed, list, st); }));
    keys = list;
    L = p.L;
  }
  const int32_t* coreset = keys;   // no thinning: the list itself (nullptr: all keys in order)
  if (p.j > 0) {
    int32_t* a = reinterpret_cast<int32_t*>(ws + p.off_a);
    int32_t* b = reinterpret_cast<int32_t*>(ws + p.off_b);
    double* G = reinterpret_cast<double*>(ws + p.off_g);
    unsigned char* dig = p.off_dig ? reinterpret_cast<unsigned char*>(ws + p.off_dig) : nullptr;
    const int32_t* in = keys;
    if (!keys) {
      THIN_HIP(timed(h, st, "iota", [&] { return thin::launch_iota(a, units, L, L, st); }));
      in = a;
    }
    int32_t* outl = b;
    int64_t dec_base = 0;
    for (int l = 1; l <= p.j; ++l) {
      // level l: bins of N = s0 2^(l+1) points; every level's lists are dense [unit][L >> (l-1)]
      const int N = static_cast<int>(p.s0 << (l + 1));
      const int bins = static_cast<int>(L / (p.s0 << (2 * l)));
      const int64_t in_unit = L >> (l - 1);
      thin::SweepLaunch sl = make_sweep(h, G, N, units, bins, in, in_unit, outl, seed, thin::kTagCompress,
                                        static_cast<uint64_t>(l) << 20);
      sl.out_stride = N / 2;
      sl.dec = decisions;
      sl.dec_per_unit = ndec;
      sl.dec_base = dec_base;
      if (thin::small_halving_supported(N, c.E, c.D)) {   // small bins: Gram and walk in one kernel
        THIN_HIP(timed(h, st, "small_halving",
                       [&] { return thin::launch_small_halving(gram_for(sl, src, h->scale64), sl, st); }));
      } else if (thin::medium_halving_supported(N, c.E, c.D, dt)) {   // one workgroup per bin
        THIN_HIP(timed(h, st, "medium_halving",
                       [&] { return thin::launch_medium_halving(gram_for(sl, src, h->scale64), sl, st); }));
      } else {
        if (const int rg = run_pair_gram(h, st, gram_for(sl, src, h->scale64, dig))) return rg;
        THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, st); }));
      }
      dec_base += static_cast<int64_t>(bins) * (N / 2);
      in = outl;
      outl = outl == b ? a : b;
    }
    coreset = in;   // the last level's output: dense [unit][n_out]
  }
  const int64_t n_cs = p.j > 0 ? p.n_out : L;
  const float w = static_cast<float>(p.r * (static_cast<int64_t>(1) << p.j));
  al.causal = 0;
  al.cs_idx = coreset;
  al.cs_w = nullptr;
  al.cs_n = static_cast<int>(n_cs);
  al.cs_stride = coreset ? n_cs : 0;
  al.cs_lnw = coreset ? logf(w) : 0.f;
  THIN_HIP(timed(h, st, "attention", [&] { return thin::launch_attention(al, dt, c.E, c.D, st); }));
  THIN_HIP(thin::launch_fill_coreset(coreset, al.cs_stride, units, static_cast<int>(n_cs), w, coreset_idx, coreset_w,
                                     coreset_len, st));
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
  if (!causal && (rc = check_unmasked_plan(h, S))) return rc;
  if ((rc = take_index_error(h))) return rc;
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
  const int dt = c.dtype;
  thin::PointSource src{k, v, S, c.H_kv, c.E, c.D, dt};
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

  if (!causal)
    return unmasked_path(h, src, al, nullptr, S, units, seed, decisions, ndec, ws, st, coreset_idx, coreset_w,
                         coreset_len);

  // ---- causal: Thinformer Express ----
  const int64_t nn = cache_size(h, S);
  const CausalPlan p = plan_causal(h, B, S, nn);
  const int n = p.sc.n;
  thin::ExpressView ev{};
  al.causal = 1;
  rc = express_thin(h, src, units, p, seed, decisions, ndec, ws, st, ev, &al);   // thinning and attention
  if (rc) return rc;
  THIN_HIP(thin::launch_express_final(ev, units, static_cast<int>(S), coreset_idx, coreset_w, coreset_len, 6LL * n,
                                      st));
  return THIN_OK;
}


int thin_attn_forward_static(thin_attn_t* h, const void* q, const void* k, const void* v, int64_t B, int64_t T,
                             int64_t S, int causal, uint64_t seed, void* out, int32_t* coreset_idx, float* coreset_w,
                             int32_t* coreset_len, uint8_t* decisions, void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  if (causal != 0 && causal != 1) return fail(h, THIN_EINVAL, "causal must be 0 or 1");
  int rc = check_dims(h, B, T, S, causal);
  if (rc) return rc;
  const size_t need = thin_attn_workspace_size(h, B, T, S, causal);
  if (need > kStaticScratchBytes)
    return fail(h, THIN_ENOMEM, "these sizes need %zu bytes of scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  if (B * T == 0) return thin_attn_forward(h, q, k, v, B, T, S, causal, seed, out, coreset_idx, coreset_w,
                                           coreset_len, decisions, nullptr, 0, stream);
  void* ws = nullptr;
  if ((rc = static_scratch(h, &ws))) return rc;
  const bool timing = h->timing;   // launch timing would create events: off for this call
  h->timing = false;
  rc = thin_attn_forward(h, q, k, v, B, T, S, causal, seed, out, coreset_idx, coreset_w, coreset_len, decisions, ws,
                         kStaticScratchBytes, stream);
  h->timing = timing;
  return rc;
}

int thin_attn_forward_subset(thin_attn_t* h, const void* q, const void* k, const void* v, const int32_t* key_idx,
                             int64_t B, int64_t T, int64_t S, int64_t L, uint64_t seed, void* out,
                             int32_t* coreset_idx, float* coreset_w, int32_t* coreset_len, uint8_t* decisions,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  int rc = check_dims(h, B, T, S, 0);
  if (rc) return rc;
  if (L < 1 || L >= (1LL << 30)) return fail(h, THIN_EINVAL, "key list length L must be in [1, 2^30) (got %lld)", (long long)L);
  if ((rc = check_unmasked_plan(h, L))) return rc;
  if ((rc = take_index_error(h))) return rc;
  if (B * T == 0) return THIN_OK;
  if (S == 0) return fail(h, THIN_EINVAL, "S must be positive");
  if (!q || !k || !v || !out || !key_idx) return fail(h, THIN_EINVAL, "null q, k, v, out or key_idx");
  const size_t need = thin_attn_workspace_size(h, B, T, L, 0);
  if (need > 256 && (!workspace || workspace_bytes < need))
    return fail(h, THIN_ENOMEM, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(h, THIN_EINVAL, "workspace must be 256-byte aligned");
  const thin_attn_config& c = h->cfg;
  const int units = static_cast<int>(B * c.H_kv);
  thin::PointSource src{k, v, S, c.H_kv, c.E, c.D, c.dtype};
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
  // the caller's list is read from a copy clamped into [0, S) (entries outside are reported)
  char* ws = static_cast<char*>(workspace);
  int32_t* keys = reinterpret_cast<int32_t*>(ws + plan_unmasked(h, B, L).off_keys);
  const hipStream_t st = as_stream(stream);
  THIN_HIP(timed(h, st, "sanitize_indices", [&] {
    return thin::launch_sanitize_indices(key_idx, static_cast<int64_t>(units) * L, static_cast<int32_t>(S), keys,
                                         h->err_dev, st);
  }));
  return unmasked_path(h, src, al, keys, L, units, seed, decisions, thin_attn_decision_count(h, L, 0), ws, st,
                       coreset_idx, coreset_w, coreset_len);
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
  if ((rc = take_index_error(h))) return rc;
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
  al.err = h->err_dev;
  THIN_HIP(thin::launch_attention(al, c.dtype, c.E, c.D, as_stream(stream)));
  return THIN_OK;
}

size_t thin_attn_halving_workspace_size(const thin_attn_t* h, int64_t B, int64_t N) {
  if (!h || B < 0 || N < 2 || N > 2048) return 0;
  return gram8_bytes(h, N, B * h->cfg.H_kv * N);
}

int thin_attn_halving(thin_attn_t* h, const void* k, const void* v, int64_t B, int64_t S, const int32_t* points,
                      int64_t N, uint64_t seed, uint32_t tag, uint64_t bin, int32_t* kept, uint8_t* decisions,
                      double* gram, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h) return THIN_EINVAL;
  h->err.clear();
  if (B < 0 || S <= 0) return fail(h, THIN_EINVAL, "bad B or S");
  if (N < 2 || N > 2048 || (N & 1)) return fail(h, THIN_EINVAL, "N must be even and in [2, 2048]");
  if (tag > 4) return fail(h, THIN_EINVAL, "unknown tag %u", tag);
  int rc = take_index_error(h);
  if (rc) return rc;
  if (B == 0) return THIN_OK;
  if (!k || !v || !points || !kept || !gram) return fail(h, THIN_EINVAL, "null k, v, points, kept or gram");
  const thin_attn_config& c = h->cfg;
  const int units = static_cast<int>(B * c.H_kv);
  const hipStream_t st = as_stream(stream);
  thin::PointSource src{k, v, S, c.H_kv, c.E, c.D, c.dtype};
  const int n = static_cast<int>(N);
  thin::SweepLaunch sl = make_sweep(h, gram, n, units, 1, points, n, kept, seed, tag, bin);
  const size_t need = thin_attn_halving_workspace_size(h, B, N);
  if (workspace && need > 0 && workspace_bytes < need)
    return fail(h, THIN_ENOMEM, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(h, THIN_EINVAL, "workspace must be 256-byte aligned");
  thin::GramLaunch gl = gram_for(sl, src, h->scale64, need > 0 ? static_cast<unsigned char*>(workspace) : nullptr);
  gl.err = h->err_dev;   // the caller's points are clamped into [0, S) and reported
  if (const int rg = run_pair_gram(h, st, gl)) return rg;
  sl.dec = decisions;
  sl.dec_per_unit = n / 2;
  THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, st); }));
  return THIN_OK;
}

int thin_attn_philox(const uint64_t* counters, int64_t n, uint64_t seed, uint64_t* out, void* stream) {
  thin_attn* h = nullptr;
  if (n < 0 || (n > 0 && (!counters || !out))) return THIN_EINVAL;
  THIN_HIP(thin::launch_philox_words(counters, n, seed, out, as_stream(stream)));
  return THIN_OK;
}

}  // extern "C"
