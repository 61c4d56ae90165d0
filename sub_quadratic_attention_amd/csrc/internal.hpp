// Internal launch interfaces of the thin-attention library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thin {

// Random-stream tags (fourth counter word).
enum : uint32_t {
  kTagCompress = 0,
  kTagBatch = 1,
  kTagHalveFirst = 2,
  kTagHalveSecond = 3,
  kTagSubsample = 4,
  kTagBaseSample = 5,
};


// Where the points of one unit (batch entry b, KV head h) live:
// key [B, S, H_kv, E] and value [B, S, H_kv, D], row-major, of element type
// dtype (kF32, kBF16 or kFP8).
struct PointSource {
  const void* k;
  const void* v;
  int64_t S;
  int H_kv;
  int E;
  int D;
  int dtype;
};

// Pair Gram of many bins at once.  Bin z holds N points whose token indices
// are idx[z * idx_stride + 0 .. N); its pairs are (2i, 2i+1).  The launch
// writes G[z][i][j] = <h_i, h_j> for the upper triangle j >= i (row-major P x P,
// P = N / 2), h_i = kappa(x_2i, .) - kappa(x_2i+1, .).
struct GramLaunch {
  PointSource src;
  // Thresholds of the walk that follows (bins of P > 64 pairs): pair i's
  // a_i (1 - 2 u_i) goes to the unused lower triangle, G[i][i-1] for i >= 1
  // and G[P-1][0] for pair 0, from the Philox stream (pair, bin_base + bin,
  // unit, tag) under seed and delta.
  uint64_t seed, tag, bin_base;
  double delta;
  int greedy;               // 1: greedy signs (threshold 0: keep the first point iff alpha_i < 0)
  const int32_t* idx;       // bin (u, j) list at idx + u * idx_unit_stride + j * idx_stride
  int64_t idx_stride;
  int64_t idx_unit_stride;
  int N;
  int nbins;
  int bins_per_unit;
  double scale;
  double* G;
  // Point indices outside [0, S) are clamped (and reported through err, when set).
  int* err;
  // Scratch of the exact integer Gram (gram8_scratch_bytes for nbins * N points),
  // or nullptr: the fp64 tiles run instead.
  unsigned char* dig;
  // Rows of the digit scratch (digits, scales, fit flags per point row):
  // dig_npts rows (0: nbins * N).  Point pt = bin * N + q of this launch is
  // row dig_row0 + pt, which its digit pass writes; or, with dig_map, row
  // dig_map[pt], written by earlier launches, and no digit pass runs.
  const int32_t* dig_map;
  int64_t dig_npts;
  int64_t dig_row0;
};

// Kernel-halving decisions of many bins at once (one workgroup per bin).
struct SweepLaunch {
  const double* G;          // from GramLaunch, P x P per bin
  int N;
  int nbins;
  int bins_per_unit;
  const int32_t* idx_in;    // the bins' point lists (as in GramLaunch)
  int64_t in_stride;
  int64_t in_unit_stride;
  int32_t* idx_out;         // kept token indices, P per bin
  int64_t out_stride;
  // optional: the kept points' digit-scratch rows, laid out as idx_out; point
  // pt = bin * N + q is row row_map[pt], or row0 + pt without a map
  int32_t* row_out;
  const int32_t* row_map;
  int64_t row0;
  uint8_t* dec;             // optional decision log (1 = first point kept)
  int64_t dec_per_unit;
  int64_t dec_base;         // offset of this launch's first bin inside a unit's log
  int dec_mode;             // 0: dec_base + bin * P;  1: Express batch order
  uint64_t seed;
  uint32_t tag;
  uint64_t bin_base;        // Philox bin id = bin_base + bin-in-unit
  double delta;
  int greedy;               // 1: greedy signs (threshold 0: keep the first point iff alpha_i < 0)
};

// Express schedule view used by the causal attention kernel and helpers.
struct ExpressView {
  int n;                 // cache size n_out = block size
  int nblk;              // full blocks in the sequence
  int n_batches_done;    // batch halvings that complete inside the sequence
  int n_batches_alloc;   // batches with at least one representative
  int n_halves;          // HALVEs inside the sequence
  const int32_t* halve_out;  // [units][n_halves][n]
  const int32_t* batch_out;  // [units][n_batches_done][n]
  const int32_t* reps;       // [units][n_batches_alloc][2n]
};

struct AttnLaunch {
  const void* q;        // [B, T, H, E]
  const void* k;        // [B, S, H_kv, E]
  const void* v;        // [B, S, H_kv, D]
  void* out;            // [B, T, H, D]
  int B, T, S, H, H_kv;
  float scale;          // softmax scale s
  int causal;           // 0: one index segment per unit; 1: Express view
  // unmasked coreset (per unit: cs_n entries at unit * cs_stride)
  const int32_t* cs_idx;   // nullptr => all S keys in order
  const float* cs_w;       // nullptr => common log-weight cs_lnw
  int cs_n;
  int64_t cs_stride;
  float cs_lnw;
  ExpressView ev;
  // Gathered token indices outside [0, S) are clamped into range (no read
  // leaves the unit's rows) and, when err is set, reported by storing 1 there.
  int* err;
  // Query rows [t0, t1) of every (b, h) are computed (t1 = 0: all T rows).
  int t0, t1;
};

// Row moves into / inside the streaming Express state (see kv.hip).
struct KvRowsLaunch {
  void* state_k;               // [units][slots][E]
  void* state_v;               // [units][slots][D]
  const int32_t* state_tok;    // token of every slot (read side of state moves)
  int32_t* state_tok_out;      // token of every slot (write side)
  int units, slots, E, D, elt;
  int cnt;                     // rows per unit
  int dst_first;               // first destination slot
  const int32_t* src_list;     // state-to-state: source slots [units][list_stride]
  int64_t list_stride;
  const void* src_k;           // token source [B, S_src, H_kv, E] (when src_list == nullptr)
  const void* src_v;
  int64_t S_src;
  int H_kv;
  int64_t src_first;           // first token of the source range (tok_list == nullptr)
  const int32_t* tok_list;     // or explicit token list [units][list_stride]
  int64_t tok_base;            // stream position of source token 0
};

struct KvDecodeLaunch {
  const void* q;        // [B, H, E] (one token)
  const void* k1;       // [B, H_kv, E]
  const void* v1;       // [B, H_kv, D]
  void* out;            // [B, H, D]
  const void* state_k;
  const void* state_v;
  int units, slots, n, H, H_kv;
  int nC, nBf, nRaw;    // visible cache, buffer and raw rows (before the new token)
  float lw_c, lw_b;     // log2 weights of cache and buffer rows
  float scale_log2;     // softmax scale * log2(e)
  float* partial;       // [units][splits][G][D + 4] (rows padded to 16 bytes)
  int splits;
  int32_t* state_tok;   // token index of every state slot
  int new_slot;         // raw-block slot the new token takes
  int32_t new_tok;      // its stream position
  int32_t* cnt;         // [units] splits done (zero before and after each launch)
};

// Launchers (return hipError_t of the launch).
// The pair Gram: the exact integer kernels when a.dig is set and
// gram8_supported() holds, else the fp64 tiles.
hipError_t launch_pair_gram(const GramLaunch& a, hipStream_t s);
// Exact integer pair Gram (bf16 and fp8 rows, E and D multiples of 64 up to
// 256, bins of at least 256 points) and its scratch for npts points.
bool gram8_supported(int dtype, int E, int D, int N);
bool gram8_fits(int dtype, int64_t npts, int E, int D);
size_t gram8_scratch_bytes(int dtype, int E, int D, int64_t npts);
hipError_t launch_pair_gram8(const GramLaunch& a, hipStream_t s);
// Its two launches (the digit pass, then thresholds, fix-ups and tiles), and
// whether launch_pair_gram takes that path for a.
hipError_t launch_gram8_digits(const GramLaunch& a, hipStream_t s);
// done (optional): an event the launch's own dispatch signals when it completes
// (no marker of its own in the stream's queue)
hipError_t launch_gram8_tiles(const GramLaunch& a, hipStream_t s, hipEvent_t done = nullptr);
bool gram8_runs(const GramLaunch& a);
hipError_t launch_halving_sweep(const SweepLaunch& a, hipStream_t s, hipEvent_t done = nullptr);
// Bins of at most 16 points: the pair Gram, thresholds and walk of a
// GramLaunch / SweepLaunch pair in one kernel (same outputs as the two).
bool small_halving_supported(int N, int E, int D);
hipError_t launch_small_halving(const GramLaunch& g, const SweepLaunch& a, hipStream_t s);
// Bins of 20 to 32 points: the same in one workgroup per bin.
bool medium_halving_supported(int N, int E, int D, int dtype);
hipError_t launch_medium_halving(const GramLaunch& g, const SweepLaunch& a, hipStream_t s);
hipError_t launch_iota(int32_t* out, int64_t units, int64_t n, int64_t stride, hipStream_t s);
// Base subsampling: out[u][t] = list[u][t r + min(floor(u_t r), r - 1)], t < L / r,
// u_t the Philox uniform of (t, 0, u, kTagBaseSample); list == nullptr means
// position = token.  list is [units][L], out [units][L / r].
hipError_t launch_base_sample(const int32_t* list, int64_t L, int units, int64_t r, uint64_t seed, int32_t* out,
                              hipStream_t s);
hipError_t launch_express_reps(const ExpressView& ev, int units, uint64_t seed, int32_t* reps, hipStream_t s);
// Digit-scratch rows of the HALVE outputs ([units][n_halves][n]) and batch
// outputs ([units][n_batches_done][n]), and the rows of a HALVE's input (out,
// [units][4n]; nullptr: not formed).
struct HalveRows {
  const int32_t* halve;
  const int32_t* batch;
  int32_t* out;
};
hipError_t launch_halve_input(const ExpressView& ev, int units, int e, int32_t* halve_in, hipStream_t s,
                              const HalveRows& rows = HalveRows{nullptr, nullptr, nullptr});
hipError_t launch_express_final(const ExpressView& ev, int units, int S, int32_t* idx, float* w,
                                int32_t* len, int64_t cap, hipStream_t s);
hipError_t launch_fill_coreset(const int32_t* src, int64_t src_stride, int units, int n, float w,
                               int32_t* idx, float* wout, int32_t* len, hipStream_t s);
hipError_t launch_attention(const AttnLaunch& a, int dtype, int E, int D, hipStream_t s);
// Copy of a caller's index list with every entry clamped into [0, S);
// stores 1 to *err (when err is set) if any entry was outside.
hipError_t launch_sanitize_indices(const int32_t* in, int64_t n, int32_t S, int32_t* out, int* err, hipStream_t s);
// LDS bytes of the walk of one bin of N points (bins of more than 128 points).
size_t sweep_lds_bytes(int N);
hipError_t launch_philox_words(const uint64_t* ctr, int64_t n, uint64_t seed, uint64_t* out, hipStream_t s);

// Host mirror of the Express schedule (r <= n_out range only).
struct ExpressSchedule {
  int n, nblk, n_batches_done, n_batches_alloc, n_halves;
  int64_t decisions;     // per unit
};
ExpressSchedule express_schedule(int64_t S, int n);
hipError_t launch_kv_rows(const KvRowsLaunch& a, hipStream_t s);
hipError_t launch_kv_block_reps(int units, int n, int64_t t0, int log2r, uint64_t seed, int32_t* list, hipStream_t s);
hipError_t launch_kv_iota(int32_t* out, int units, int cnt, int first, hipStream_t s);
// Representative of subsampling group g (2^log2r tokens) per unit: list[u] = base + (token - lo)
// if the token lies in [lo, hi), else fallback.
hipError_t launch_kv_group_rep(int units, int64_t g, int log2r, uint64_t seed, int64_t lo, int64_t hi, int64_t base,
                               int32_t fallback, int32_t* list, hipStream_t s);
hipError_t launch_kv_fill(int32_t* out, int64_t n, int32_t value, hipStream_t s);
hipError_t launch_kv_decode(const KvDecodeLaunch& a, int dtype, int E, int D, int G, hipStream_t s);
bool kv_decode_supported(int dtype, int E, int D, int G);
hipError_t launch_kv_summary(const int32_t* tok, int units, int slots, int n, int nC, int nBf, int nRaw, float wc,
                             float wb, int32_t* idx, float* w, int32_t* len, int cap, hipStream_t s);
int kv_decode_splits(int n);
bool attention_supported(int dtype, int E, int D);

}  // namespace thin
