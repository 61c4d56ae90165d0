// C ABI of the streaming Express state (decode): creation, ingest of tokens
// (block by block, or in bulk from an empty state), one-token decode steps.
//
// The schedule is the one of the causal forward ("Express Language
// Modeling", "The EXPRESS Meta-Procedure"): blocks of n tokens; while m = 1
// blocks enter the cache unchanged; while m >= 4 each aligned group of
// r = m / 2 tokens of a finished block gives one representative to the
// buffer, and a full buffer (2n representatives) is halved into the cache;
// a cache of 4n points is halved twice and m becomes 4m.  All units share
// the counters (they ingest the same tokens), so the host tracks them.

#include <cstring>

#include "host.hpp"

using namespace thinhost;

struct thin_kv {
  thin_attn* h;
  char* state;
  size_t bytes;
  int B, units, n;
  uint64_t seed;
  int64_t tokens;   // tokens ingested
  int64_t m;        // inflation factor
  int nC, nBf, nRaw, nb, nh;
  bool cnt_ready;   // the decode's per-unit split counters are known to be zero
};

namespace {

struct KvLayout {
  size_t off_k, off_v, off_tok, off_cnt, bytes;
};

int elt_of(const thin_attn* h) { return thinhost::elt_bytes(h->cfg.dtype); }

// Slots per unit: cache 4n, buffer 2n, raw block n, one held representative.
inline int kv_slots(int64_t n) { return static_cast<int>(7 * n + 1); }

KvLayout kv_layout(const thin_attn* h, int64_t units, int64_t n) {
  KvLayout k{};
  Layout L;
  const int64_t rows = units * kv_slots(n);
  k.off_k = L.add(static_cast<size_t>(rows) * h->cfg.E * elt_of(h));
  k.off_v = L.add(static_cast<size_t>(rows) * h->cfg.D * elt_of(h));
  k.off_tok = L.add(static_cast<size_t>(rows) * sizeof(int32_t));
  k.off_cnt = L.add(static_cast<size_t>(units) * sizeof(int32_t));   // decode split counters (zero between calls)
  k.bytes = L.total;
  return k;
}

struct KvWs {
  size_t off_la, off_lb, off_lc, off_g, off_dig, off_part, bytes;
};

KvWs kv_ws(const thin_attn* h, int64_t units, int64_t n) {
  KvWs w{};
  Layout L;
  w.off_la = L.add(sizeof(int32_t) * units * 4 * n);
  w.off_lb = L.add(sizeof(int32_t) * units * 4 * n);
  w.off_lc = L.add(sizeof(int32_t) * units * 4 * n);
  w.off_g = L.add(sizeof(double) * units * 4 * n * n);
  const size_t dig = thinhost::gram8_bytes(h, 4 * n, units * 4 * n);   // covers the 2n halvings
  w.off_dig = dig ? L.add(dig) : 0;
  const int G = h->cfg.H / h->cfg.H_kv;
  w.off_part = L.add(sizeof(float) * units * thin::kv_decode_splits(static_cast<int>(n)) * G * (h->cfg.D + 4));
  w.bytes = L.total;
  return w;
}

// Decisions an ingest of n_new tokens makes (per unit): the schedule is fixed by
// the token count, so it is the difference of the static schedule's counts over
// the full blocks before and after.
int64_t decisions_for(const thin_kv& kv, int64_t n_new) {
  const int64_t n = kv.n;
  const int64_t before = (kv.tokens / n) * n, after = ((kv.tokens + n_new) / n) * n;
  return thin::express_schedule(after, static_cast<int>(n)).decisions -
         thin::express_schedule(before, static_cast<int>(n)).decisions;
}

// Streams stay below 2^30 tokens (32-bit token indices).
bool kv_range_ok(const thin_kv& kv, int64_t n_new) { return n_new >= 0 && kv.tokens + n_new < (1LL << 30); }

int log2_of(int64_t r) {
  int l = 0;
  while ((1LL << l) < r) ++l;
  return l;
}

thin::PointSource state_source(const thin_kv& kv) {
  const thin_attn* h = kv.h;
  const KvLayout L = kv_layout(h, kv.units, kv.n);
  // rows of unit u are [u][7n]: present the state as a [units, 7n, 1, *] tensor
  return thin::PointSource{kv.state + L.off_k, kv.state + L.off_v, kv_slots(kv.n), 1, h->cfg.E, h->cfg.D,
                           h->cfg.dtype};
}

thin::KvRowsLaunch rows_base(const thin_kv& kv) {
  const thin_attn* h = kv.h;
  const KvLayout L = kv_layout(h, kv.units, kv.n);
  thin::KvRowsLaunch r{};
  r.state_k = kv.state + L.off_k;
  r.state_v = kv.state + L.off_v;
  r.state_tok = reinterpret_cast<const int32_t*>(kv.state + L.off_tok);
  r.state_tok_out = reinterpret_cast<int32_t*>(kv.state + L.off_tok);
  r.units = kv.units;
  r.slots = kv_slots(kv.n);
  r.E = h->cfg.E;
  r.D = h->cfg.D;
  r.elt = elt_of(h);
  r.H_kv = h->cfg.H_kv;
  return r;
}

// state slots listed in `list` ([units][stride]) -> slots [dst, dst + cnt)
int move_slots(thin_kv& kv, const int32_t* list, int64_t stride, int cnt, int dst, hipStream_t st) {
  thin_attn* h = kv.h;
  thin::KvRowsLaunch r = rows_base(kv);
  r.src_list = list;
  r.list_stride = stride;
  r.cnt = cnt;
  r.dst_first = dst;
  THIN_HIP(timed(h, st, "kv_rows", [&] { return thin::launch_kv_rows(r, st); }));
  return THIN_OK;
}

// tokens [first, first + cnt) of a [B, S_src, H_kv, *] chunk (stream position tok_base) -> slots dst..
int put_tokens(thin_kv& kv, const void* k, const void* v, int64_t S_src, int64_t first, int cnt, int dst,
               int64_t tok_base, const int32_t* tok_list, int64_t list_stride, hipStream_t st) {
  thin_attn* h = kv.h;
  thin::KvRowsLaunch r = rows_base(kv);
  r.src_k = k;
  r.src_v = v;
  r.S_src = S_src;
  r.src_first = first;
  r.tok_list = tok_list;
  r.list_stride = list_stride;
  r.tok_base = tok_base;
  r.cnt = cnt;
  r.dst_first = dst;
  THIN_HIP(timed(h, st, "kv_rows", [&] { return thin::launch_kv_rows(r, st); }));
  return THIN_OK;
}

// One kernel halving per unit over the state slots in `in` ([units][N]); kept slots -> out.
int halve_slots(thin_kv& kv, const int32_t* in, int N, int32_t* out, uint32_t tag, uint64_t bin, uint8_t* dec,
                int64_t dec_per_unit, int64_t dec_base, double* G, unsigned char* dig, hipStream_t st) {
  thin_attn* h = kv.h;
  const thin::PointSource src = state_source(kv);
  thin::SweepLaunch sl = make_sweep(h, G, N, kv.units, 1, in, N, out, kv.seed, tag, bin);
  if (const int rg = run_pair_gram(h, st, gram_for(sl, src, h->scale64, dig))) return rg;
  sl.dec = dec;
  sl.dec_per_unit = dec_per_unit;
  sl.dec_base = dec_base;
  THIN_HIP(timed(h, st, "halving_sweep", [&] { return thin::launch_halving_sweep(sl, st); }));
  return THIN_OK;
}

// The raw block is full: move it into the cache (m = 1) or take its
// representatives (m >= 4), halve a full buffer, HALVE a full cache.
int ingest_block(thin_kv& kv, char* ws, uint8_t* dec, int64_t dec_per_unit, int64_t& dec_pos, hipStream_t st) {
  thin_attn* h = kv.h;
  const int n = kv.n;
  const KvWs W = kv_ws(h, kv.units, n);
  int32_t* la = reinterpret_cast<int32_t*>(ws + W.off_la);
  int32_t* lb = reinterpret_cast<int32_t*>(ws + W.off_lb);
  int32_t* lc = reinterpret_cast<int32_t*>(ws + W.off_lc);
  double* G = reinterpret_cast<double*>(ws + W.off_g);
  unsigned char* dig = W.off_dig ? reinterpret_cast<unsigned char*>(ws + W.off_dig) : nullptr;
  const int64_t t0 = kv.tokens - n;   // first token of the finished block
  int rc;
  if (kv.m == 1) {
    THIN_HIP(thin::launch_kv_iota(la, kv.units, n, 6 * n, st));
    if ((rc = move_slots(kv, la, n, n, kv.nC, st))) return rc;
    kv.nC += n;
  } else {
    const int64_t r = kv.m / 2;
    const int log2r = log2_of(r);
    if (r <= n) {   // the block completes n / r groups: their representatives join the buffer
      const int per = static_cast<int>(n / r);
      THIN_HIP(thin::launch_kv_block_reps(kv.units, n, t0, log2r, kv.seed, la, st));
      if ((rc = move_slots(kv, la, per, per, 4 * n + kv.nBf, st))) return rc;
      kv.nBf += per;
    } else {        // the block lies inside one group of r tokens
      // its representative is held in slot 7n when it falls in this block (else the slot keeps itself) ...
      THIN_HIP(thin::launch_kv_group_rep(kv.units, t0 >> log2r, log2r, kv.seed, t0, t0 + n, 6 * n, 7 * n, la, st));
      if ((rc = move_slots(kv, la, 1, 1, 7 * n, st))) return rc;
      // ... and joins the buffer when this block completes the group
      if ((t0 + n) % r == 0) {
        THIN_HIP(thin::launch_kv_iota(la, kv.units, 1, 7 * n, st));
        if ((rc = move_slots(kv, la, 1, 1, 4 * n + kv.nBf, st))) return rc;
        kv.nBf += 1;
      }
    }
    if (kv.nBf == 2 * n) {
      THIN_HIP(thin::launch_kv_iota(la, kv.units, 2 * n, 4 * n, st));
      if ((rc = halve_slots(kv, la, 2 * n, lb, thin::kTagBatch, static_cast<uint64_t>(kv.nb), dec, dec_per_unit,
                            dec_pos, G, dig, st)))
        return rc;
      dec_pos += n;
      if ((rc = move_slots(kv, lb, n, n, kv.nC, st))) return rc;
      kv.nC += n;
      kv.nBf = 0;
      kv.nb += 1;
    }
  }
  if (kv.nC == 4 * n) {
    THIN_HIP(thin::launch_kv_iota(la, kv.units, 4 * n, 0, st));
    if ((rc = halve_slots(kv, la, 4 * n, lb, thin::kTagHalveFirst, static_cast<uint64_t>(kv.nh), dec, dec_per_unit,
                          dec_pos, G, dig, st)))
      return rc;
    dec_pos += 2 * n;
    if ((rc = halve_slots(kv, lb, 2 * n, lc, thin::kTagHalveSecond, static_cast<uint64_t>(kv.nh), dec, dec_per_unit,
                          dec_pos, G, dig, st)))
      return rc;
    dec_pos += n;
    // compact through the (empty) buffer region: kept slots -> [4n, 5n) -> [0, n)
    if ((rc = move_slots(kv, lc, n, n, 4 * n, st))) return rc;
    THIN_HIP(thin::launch_kv_iota(la, kv.units, n, 4 * n, st));
    if ((rc = move_slots(kv, la, n, n, 0, st))) return rc;
    kv.nC = n;
    kv.m *= 4;
    kv.nh += 1;
  }
  kv.nRaw = 0;
  return THIN_OK;
}

// Empty state, n_new >= n tokens: run the static schedule over the chunk
// (all batch halvings in parallel, then the HALVE chain) and copy the
// resulting cache, buffer and tail block into the state.
int bulk_ingest(thin_kv& kv, const void* k, const void* v, int64_t n_new, uint8_t* dec, char* ws, hipStream_t st) {
  thin_attn* h = kv.h;
  const int n = kv.n;
  const thin_attn_config& c = h->cfg;
  const CausalPlan p = plan_causal(h, kv.B, n_new, n);
  const thin::PointSource src{k, v, n_new, c.H_kv, c.E, c.D, c.dtype};
  thin::ExpressView ev{};
  int rc = express_thin(h, src, kv.units, p, kv.seed, dec, p.sc.decisions, ws, st, ev);
  if (rc) return rc;
  const int nblk = p.sc.nblk;
  if (nblk < 4) {
    if ((rc = put_tokens(kv, k, v, n_new, 0, nblk * n, 0, 0, nullptr, 0, st))) return rc;
    kv.nC = nblk * n;
    kv.m = 1;
  } else {
    int E = 1;
    while ((1LL << (2 * (E + 1))) <= nblk) ++E;
    const int64_t m = 1LL << (2 * E);
    const int since = static_cast<int>(nblk - m);
    const int nbc = static_cast<int>(since / m);
    const int rem = static_cast<int>(since % m);
    const int n_rep = static_cast<int>((static_cast<int64_t>(rem) * 2 * n) / m);
    if ((rc = put_tokens(kv, k, v, n_new, 0, n, 0, 0, ev.halve_out + static_cast<int64_t>(E - 1) * n,
                         static_cast<int64_t>(ev.n_halves) * n, st)))
      return rc;
    if (nbc > 0 &&
        (rc = put_tokens(kv, k, v, n_new, 0, nbc * n, n, 0, ev.batch_out + static_cast<int64_t>(3 * (E - 1)) * n,
                         static_cast<int64_t>(ev.n_batches_done) * n, st)))
      return rc;
    if (n_rep > 0 &&
        (rc = put_tokens(kv, k, v, n_new, 0, n_rep, 4 * n, 0,
                         ev.reps + static_cast<int64_t>(3 * (E - 1) + nbc) * 2 * n,
                         static_cast<int64_t>(ev.n_batches_alloc) * 2 * n, st)))
      return rc;
    kv.nC = n * (1 + nbc);
    kv.nBf = n_rep;
    kv.m = m;
    kv.nh = E;
    kv.nb = 3 * (E - 1) + nbc;
    // a group longer than a block still in progress: hold its representative
    // if the chunk already contains it (else the block that does captures it)
    const int64_t r = m / 2, done_tok = static_cast<int64_t>(nblk) * n;
    if (r > n && done_tok % r != 0) {
      int32_t* la = reinterpret_cast<int32_t*>(ws + p.off_hin);   // free again after the HALVE chain
      const int log2r = log2_of(r);
      THIN_HIP(thin::launch_kv_group_rep(kv.units, done_tok >> log2r, log2r, kv.seed, 0, done_tok, 0,
                                         static_cast<int32_t>(done_tok - 1), la, st));
      if ((rc = put_tokens(kv, k, v, n_new, 0, 1, 7 * n, 0, la, 1, st))) return rc;
    }
  }
  const int tail = static_cast<int>(n_new - static_cast<int64_t>(nblk) * n);
  if (tail > 0 && (rc = put_tokens(kv, k, v, n_new, static_cast<int64_t>(nblk) * n, tail, 6 * n, 0, nullptr, 0, st)))
    return rc;
  kv.nRaw = tail;
  kv.tokens = n_new;
  return THIN_OK;
}

// The counters every state holds after `tokens` tokens (the schedule is fixed
// by the token count): nblk full blocks; while fewer than 4 the cache holds
// them all (m = 1); after that, with m = 4^E the largest power of four <= nblk,
// the cache holds HALVE E's output and the batches completed since, and the
// buffer one representative per completed group of the batch in progress.
struct Counters {
  int64_t m;
  int nC, nBf, nRaw, nb, nh;
};

Counters counters_after(int64_t n, int64_t tokens) {
  Counters c{1, 0, 0, 0, 0, 0};
  const int64_t nblk = tokens / n;
  c.nRaw = static_cast<int>(tokens - nblk * n);
  if (nblk < 4) {
    c.nC = static_cast<int>(nblk * n);
    return c;
  }
  int E = 1;
  while ((1LL << (2 * (E + 1))) <= nblk) ++E;
  const int64_t m = 1LL << (2 * E);
  const int64_t since = nblk - m, nbc = since / m, rem = since % m;
  c.m = m;
  c.nC = static_cast<int>(n * (1 + nbc));
  c.nBf = static_cast<int>((rem * 2 * n) / m);
  c.nh = E;
  c.nb = static_cast<int>(3 * (E - 1) + nbc);
  return c;
}

int check_kv(thin_kv* kv) {
  if (!kv || !kv->h) return THIN_EINVAL;
  kv->h->err.clear();
  return THIN_OK;
}

}  // namespace

extern "C" {

size_t thin_attn_kv_state_size(const thin_attn_t* h, int64_t B, int64_t n_out) {
  if (!h || B <= 0 || n_out < 2 || !pow2(n_out)) return 0;
  return kv_layout(h, B * h->cfg.H_kv, n_out).bytes;
}

int thin_attn_kv_create(thin_attn_t* h, void* state, size_t state_bytes, int64_t B, int64_t n_out, uint64_t seed,
                        thin_kv_t** out) {
  if (!h || !out) return THIN_EINVAL;
  h->err.clear();
  if (B <= 0) return fail(h, THIN_EINVAL, "B must be positive");
  if (n_out == 0) n_out = h->cfg.n_out;
  if (n_out < 2 || !pow2(n_out)) return fail(h, THIN_EINVAL, "n_out must be a power of two >= 2");
  if (!walk_fits(4 * n_out))
    return fail(h, THIN_ENOTSUP, "n_out = %lld: the halving of a full cache (%lld points) exceeds the walk's LDS",
                (long long)n_out, (long long)(4 * n_out));
  const int G = h->cfg.H / h->cfg.H_kv;
  if (!thin::kv_decode_supported(h->cfg.dtype, h->cfg.E, h->cfg.D, G))
    return fail(h, THIN_ENOTSUP, "decode not built for E=%d D=%d and %d query heads per KV head", h->cfg.E, h->cfg.D, G);
  const size_t need = kv_layout(h, B * h->cfg.H_kv, n_out).bytes;
  if (!state || state_bytes < need) return fail(h, THIN_ENOMEM, "state of %zu bytes, need %zu", state_bytes, need);
  if (reinterpret_cast<uintptr_t>(state) & 255) return fail(h, THIN_EINVAL, "state must be 256-byte aligned");
  thin_kv* kv = new thin_kv();
  kv->h = h;
  kv->state = static_cast<char*>(state);
  kv->bytes = state_bytes;
  kv->B = static_cast<int>(B);
  kv->units = static_cast<int>(B * h->cfg.H_kv);
  kv->n = static_cast<int>(n_out);
  kv->seed = seed;
  kv->tokens = 0;
  kv->m = 1;
  kv->nC = kv->nBf = kv->nRaw = kv->nb = kv->nh = 0;
  kv->cnt_ready = false;
  *out = kv;
  return THIN_OK;
}

int thin_attn_kv_destroy(thin_kv_t* kv) {
  delete kv;
  return THIN_OK;
}

int64_t thin_attn_kv_tokens(const thin_kv_t* kv) { return kv ? kv->tokens : THIN_EINVAL; }

int64_t thin_attn_kv_decision_count(const thin_kv_t* kv, int64_t n_new) {
  if (!kv || n_new < 0) return THIN_EINVAL;
  if (!kv_range_ok(*kv, n_new)) return THIN_ENOTSUP;
  return decisions_for(*kv, n_new);
}

size_t thin_attn_kv_workspace_size(const thin_kv_t* kv, int64_t n_new) {
  if (!kv || n_new < 0) return 0;
  size_t need = kv_ws(kv->h, kv->units, kv->n).bytes;
  if (kv->tokens == 0 && n_new >= kv->n) need = std::max(need, plan_causal(kv->h, kv->B, n_new, kv->n).bytes);
  return need;
}

int thin_attn_kv_append(thin_kv_t* kv, const void* k, const void* v, int64_t n_new, uint8_t* decisions,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  thin_attn* h = kv->h;
  if (n_new < 0) return fail(h, THIN_EINVAL, "n_new < 0");
  if (n_new == 0) return THIN_OK;
  if (!k || !v) return fail(h, THIN_EINVAL, "null k or v");
  if (kv->tokens + n_new >= (1LL << 30)) return fail(h, THIN_ENOTSUP, "stream too long");
  if (!kv_range_ok(*kv, n_new)) return fail(h, THIN_ENOTSUP, "stream beyond 2^30 tokens");
  const size_t need = thin_attn_kv_workspace_size(kv, n_new);
  if (!workspace || workspace_bytes < need) return fail(h, THIN_ENOMEM, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(h, THIN_EINVAL, "workspace must be 256-byte aligned");
  const hipStream_t st = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  if (kv->tokens == 0 && n_new >= kv->n) return bulk_ingest(*kv, k, v, n_new, decisions, ws, st);
  const int64_t ndec = decisions_for(*kv, n_new);
  int64_t dec_pos = 0;
  int64_t done = 0;
  while (done < n_new) {
    const int take = static_cast<int>(std::min<int64_t>(n_new - done, kv->n - kv->nRaw));
    if ((rc = put_tokens(*kv, k, v, n_new, done, take, 6 * kv->n + kv->nRaw, kv->tokens - done, nullptr, 0, st)))
      return rc;
    kv->nRaw += take;
    kv->tokens += take;
    done += take;
    if (kv->nRaw == kv->n && (rc = ingest_block(*kv, ws, decisions, ndec, dec_pos, st))) return rc;
  }
  return THIN_OK;
}

int thin_attn_kv_decode(thin_kv_t* kv, const void* q, const void* k1, const void* v1, void* out, uint8_t* decisions,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  thin_attn* h = kv->h;
  if (!q || !k1 || !v1 || !out) return fail(h, THIN_EINVAL, "null q, k1, v1 or out");
  if (!kv_range_ok(*kv, 1)) return fail(h, THIN_ENOTSUP, "stream beyond 2^30 tokens");
  const KvWs W = kv_ws(h, kv->units, kv->n);
  if (!workspace || workspace_bytes < W.bytes) return fail(h, THIN_ENOMEM, "workspace of %zu bytes, need %zu", workspace_bytes, W.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(h, THIN_EINVAL, "workspace must be 256-byte aligned");
  const hipStream_t st = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  const thin_attn_config& c = h->cfg;
  const KvLayout L = kv_layout(h, kv->units, kv->n);
  // 1. attention of the new token's queries over the state and the token itself
  thin::KvDecodeLaunch a{};
  a.q = q;
  a.k1 = k1;
  a.v1 = v1;
  a.out = out;
  a.state_k = kv->state + L.off_k;
  a.state_v = kv->state + L.off_v;
  a.units = kv->units;
  a.slots = kv_slots(kv->n);
  a.n = kv->n;
  a.H = c.H;
  a.H_kv = c.H_kv;
  a.nC = kv->nC;
  a.nBf = kv->nBf;
  a.nRaw = kv->nRaw;
  a.lw_c = static_cast<float>(log2(static_cast<double>(kv->m)));
  a.lw_b = kv->m >= 2 ? static_cast<float>(log2(static_cast<double>(kv->m / 2))) : 0.f;
  a.scale_log2 = static_cast<float>(h->scale64 * 1.4426950408889634);
  a.partial = reinterpret_cast<float*>(ws + W.off_part);
  // the same launch appends the token to the raw block (slot 6n + nRaw)
  a.state_tok = reinterpret_cast<int32_t*>(kv->state + L.off_tok);
  a.new_slot = 6 * kv->n + kv->nRaw;
  a.new_tok = static_cast<int32_t>(kv->tokens);
  a.cnt = reinterpret_cast<int32_t*>(kv->state + L.off_cnt);
  if (!kv->cnt_ready) {   // first decode on this state: zero the split counters
    THIN_HIP(thin::launch_kv_fill(a.cnt, kv->units, 0, st));
    kv->cnt_ready = true;
  }
  THIN_HIP(timed(h, st, "kv_decode", [&] {
    return thin::launch_kv_decode(a, c.dtype, c.E, c.D, c.H / c.H_kv, st);
  }));
  // 2. the token has joined the raw block; a finished block is ingested
  const int64_t ndec = decisions_for(*kv, 1);
  int64_t dec_pos = 0;
  kv->nRaw += 1;
  kv->tokens += 1;
  if (kv->nRaw == kv->n && (rc = ingest_block(*kv, ws, decisions, ndec, dec_pos, st))) return rc;
  return THIN_OK;
}

int thin_attn_kv_coreset(thin_kv_t* kv, int32_t* idx, float* w, int32_t* len, void* stream) {
  int rc = check_kv(kv);
  if (rc) return rc;
  thin_attn* h = kv->h;
  const KvLayout L = kv_layout(h, kv->units, kv->n);
  THIN_HIP(thin::launch_kv_summary(reinterpret_cast<const int32_t*>(kv->state + L.off_tok), kv->units, kv_slots(kv->n), kv->n,
                                   kv->nC, kv->nBf, kv->nRaw, static_cast<float>(kv->m),
                                   static_cast<float>(kv->m >= 2 ? kv->m / 2 : 1), idx, w, len, 7 * kv->n,
                                   as_stream(stream)));
  return THIN_OK;
}

// Host-side counters of a state (the device rows are the caller's buffer).
struct thin_kv_meta {
  uint32_t magic, version;
  int32_t B, units, n, nC, nBf, nRaw, nb, nh;
  int64_t tokens, m;
  uint64_t seed;
};

int64_t thin_attn_kv_export(const thin_kv_t* kv, void* host, size_t bytes) {
  if (!kv) return THIN_EINVAL;
  if (!host) return static_cast<int64_t>(sizeof(thin_kv_meta));
  if (bytes < sizeof(thin_kv_meta)) return THIN_ENOMEM;
  thin_kv_meta m{0x544b5631u, 1, kv->B, kv->units, kv->n, kv->nC, kv->nBf, kv->nRaw, kv->nb, kv->nh,
                 kv->tokens, kv->m, kv->seed};
  memcpy(host, &m, sizeof(m));
  return static_cast<int64_t>(sizeof(m));
}

int thin_attn_kv_import(thin_kv_t* kv, const void* host, size_t bytes) {
  int rc = check_kv(kv);
  if (rc) return rc;
  if (!host || bytes < sizeof(thin_kv_meta)) return fail(kv->h, THIN_EINVAL, "metadata too short");
  thin_kv_meta m;
  memcpy(&m, host, sizeof(m));
  if (m.magic != 0x544b5631u || m.version != 1) return fail(kv->h, THIN_EINVAL, "not a state export");
  if (m.B != kv->B || m.units != kv->units || m.n != kv->n || m.seed != kv->seed)
    return fail(kv->h, THIN_EINVAL, "export of a different state (B, heads, n_out or seed)");
  // every counter is fixed by the token count: a record that disagrees is
  // corrupt, and restoring it would let later calls address slots outside the
  // state's rows
  if (m.tokens < 0 || m.tokens >= (1LL << 30)) return fail(kv->h, THIN_EINVAL, "token count out of range");
  {
    thin_kv probe = *kv;
    probe.tokens = 0;
    probe.m = 1;
    probe.nC = probe.nBf = probe.nRaw = probe.nb = probe.nh = 0;
    if (!kv_range_ok(probe, m.tokens)) return fail(kv->h, THIN_ENOTSUP, "token count beyond the supported schedule");
  }
  const Counters want = counters_after(kv->n, m.tokens);
  if (m.m != want.m || m.nC != want.nC || m.nBf != want.nBf || m.nRaw != want.nRaw || m.nb != want.nb ||
      m.nh != want.nh)
    return fail(kv->h, THIN_EINVAL, "state counters do not match the schedule of %lld tokens", (long long)m.tokens);
  kv->nC = m.nC;
  kv->nBf = m.nBf;
  kv->nRaw = m.nRaw;
  kv->nb = m.nb;
  kv->nh = m.nh;
  kv->tokens = m.tokens;
  kv->m = m.m;
  kv->cnt_ready = false;
  return THIN_OK;
}

}  // extern "C"
