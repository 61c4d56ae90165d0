/*
 * thin_attn.h - C ABI of the MI355X (gfx950) Thinformer / Thinformer Express
 * attention library.
 *
 * What is computed.  For every batch entry b and KV head h (a "unit") the S
 * key-value pairs x_j = (k_j, v_j) are thinned to a small weighted coreset
 * by kernel halving under the key-value attention kernel
 *     kappa((k, v), (k', v')) = exp(s <k, k'>) (<v, v'> + 1),
 * and every query attends to that coreset:
 *     out(q) = sum_j w_j exp(s <q, k_j>) v_j / sum_j w_j exp(s <q, k_j>).
 * Sources: the "Thinformer" README (introduction and "Getting Started":
 * Thinformer for unmasked attention, Thinformer Express for causal attention,
 * the (query, key, value, causal) call and its shapes) and "Express Language
 * Modeling" (sections "The EXPRESS Meta-Procedure" and "Thinformer Express":
 * the exact / thin / HALVE weighted cache, kernel halving, kappa_att).
 *
 * Conventions shared by every call.
 *  - Tensors are dense, row-major, on the device: query [B, T, H, E],
 *    key [B, S, H_kv, E], value [B, S, H_kv, D], output [B, T, H, D], all of
 *    the configured dtype (float32, or bfloat16 as raw 16-bit patterns).
 *    Query head h reads KV head h / (H / H_kv).
 *  - The caller owns every device buffer (inputs, outputs, workspace); the
 *    library owns only the host-side handle.  No call allocates device
 *    memory.  Work is enqueued asynchronously on `stream` (a hipStream_t,
 *    NULL = the default stream); device faults surface at the caller's next
 *    synchronisation.
 *  - Return value 0 (THIN_OK) on success, a negative THIN_E* code otherwise.
 *    Argument errors are detected before anything is enqueued; the message
 *    is kept in the handle (thin_attn_last_error).  Token indices a caller
 *    passes in device memory (key_idx, idx, points) can only be checked on
 *    the device: an entry outside [0, S) is clamped into range, so that no
 *    read leaves the unit's rows, and flagged; the flag is reported (and
 *    cleared) as THIN_EINVAL by the next call on the handle that finds it set,
 *    or by thin_attn_status, which waits for the stream first.
 *  - Same inputs, seed and configuration give bit-identical results.
 *  - One handle must not be used from two host threads at once.
 */
#ifndef THIN_ATTN_H
#define THIN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of query, key and value.  THIN_FP8_E4M3: OCP FP8 E4M3
 * (E4M3FN: sign, 4 exponent bits of bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 NaN) as raw bytes; the output is then bfloat16, and per-tensor
 * scale factors are the caller's to fold into `scale` (query and key) and
 * into the output (value). */
enum thin_dtype { THIN_F32 = 0, THIN_BF16 = 1, THIN_FP8_E4M3 = 2 };

/* Configuration flags (thin_attn_config.flags).
 * THIN_GREEDY_SIGNS: every kernel-halving walk takes its signs greedily
 *   instead of at random: pair i keeps its first point exactly when the
 *   running signed sum alpha_i = sum_{j<i} eta_j <h_j, h_i> is negative, and
 *   its second point otherwise (alpha_i = 0 included, so the first pair of
 *   every bin keeps its second point).  The sigma recursion and the draws u_i
 *   play no part.  This is the deterministic accuracy/cost variant of the
 *   self-balancing walk the Thinformer pages build on ("Kernel halving",
 *   Compress); the pages' sub-Gaussian guarantee is stated for the randomised
 *   walk only.  Representative draws of the Express batches stay random.
 *   Off by default. */
/* THIN_SUBSAMPLE_BASE: unmasked thinning (thin_attn_forward with causal = 0
 *   and thin_attn_forward_subset) first keeps one random point of every
 *   stratum of r consecutive points of the list, r the largest divisor of the
 *   Compress base block s0 (L = 4^j s0, j >= 1) with r * r <= s0 and
 *   s0 / r >= 4^g; the Compress then runs on those L / r points and every
 *   coreset point carries weight r 2^j'.  For s0 = r^2 the coreset has
 *   sqrt(L) points (56 for the 56 x 56 ViT grid instead of 392), the size the
 *   Thinformer pages quote for their unmasked experiments.  Stratum t keeps
 *   point t r + min(floor(u r), r - 1), u the Philox4x64-10 uniform of counter
 *   (t, 0, unit, 5) under the call's seed.  r = 1 (no Compress level, or s0
 *   without such a divisor) changes nothing.  thin_attn_coreset_size,
 *   thin_attn_decision_count and thin_attn_workspace_size follow the flag. */
/* THIN_ONE_STREAM: every launch of a call goes on the caller's stream.  By
 *   default the causal path (thin_attn_forward with causal = 1 and the bulk
 *   thin_attn_kv_append) also uses a second stream the handle creates on the
 *   device current at creation: the batch halvings and the attention of each
 *   finished epoch run there beside the HALVE chain, and the caller's stream
 *   waits for all of it before the call's last launch.  Results are the same
 *   either way; the flag gives serial launches (per-kernel timing). */
/* THIN_FP64_GRAM: every pair Gram of the kernel-halving walks runs on the
 *   fp64 matrix cores.  By default the Grams of bf16 and fp8 inputs (E and D
 *   multiples of 64, bins of at least 256 points) take their dot products on
 *   the int8 matrix cores instead: each row is scaled by a power of two into
 *   integers, split into balanced base-256 digits, and the digit products are
 *   summed exactly, so every dot product is the exact one rounded once to
 *   fp64; rows whose features span more than the digits hold (bf16 features
 *   more than 22 binades below the row's largest) have their pairs'
 *   Gram entries recomputed in fp64.  Decisions agree with the fp64 Gram up
 *   to the rounding of its dot products (near ties).  The workspace sizes
 *   include the integer Gram's scratch unless the flag is set. */
enum thin_flags { THIN_GREEDY_SIGNS = 1u, THIN_SUBSAMPLE_BASE = 2u, THIN_ONE_STREAM = 4u, THIN_FP64_GRAM = 8u };

enum thin_status {
  THIN_OK = 0,
  THIN_EINVAL = -1,   /* bad argument: null pointer, shape, dtype, layout */
  THIN_ENOTSUP = -2,  /* valid but not built: head dims, schedule range    */
  THIN_ENOMEM = -3,   /* workspace smaller than thin_attn_workspace_size   */
  THIN_EHIP = -4      /* a HIP launch reported an error                    */
};

typedef struct thin_attn_config {
  int32_t dtype;   /* THIN_F32 or THIN_BF16 (query, key, value, output)              */
  int32_t E;       /* query / key head dim: 64 or 128                                  */
  int32_t D;       /* value head dim: 64, 128 or 256 (see thin_attn_create)            */
  int32_t H;       /* query heads                                                      */
  int32_t H_kv;    /* key / value heads, H % H_kv == 0                                 */
  int32_t g;       /* unmasked oversampling: base blocks of size >= 4^g; 4^g >= S
                      disables thinning (exact attention)                              */
  int32_t n_out;   /* causal cache size and block length, a power of two >= 2;
                      0 = smallest power of two p with p*p >= S; n_out >= S disables
                      thinning (exact causal attention)                                */
  double delta;    /* kernel-halving failure parameter; <= 0 means 0.5                */
  float scale;     /* softmax scale s; 0 means 1/sqrt(E)                              */
  uint32_t flags;  /* THIN_GREEDY_SIGNS | THIN_SUBSAMPLE_BASE | THIN_ONE_STREAM | THIN_FP64_GRAM;
                      others rejected */
} thin_attn_config;

typedef struct thin_attn thin_attn_t;

/* Create a handle.  Supported head dims: float32 E=64 with D=64 or 128, E=128
 * with D=128; bfloat16 E=64 with D=64, 128 or 256, E=128 with D=64 or 128.
 * Returns THIN_EINVAL for inconsistent values, THIN_ENOTSUP for other dims.
 * *out is set only on success. */
int thin_attn_create(const thin_attn_config* cfg, thin_attn_t** out);

/* Destroy a handle (NULL is accepted).  Work already enqueued is unaffected. */
int thin_attn_destroy(thin_attn_t* h);

/* Last error message of the handle ("" if none); NULL gives the message of
 * the last failed thin_attn_create.  Valid until the next call on h. */
const char* thin_attn_last_error(const thin_attn_t* h);

/* Wait for `stream`, then report index errors the device found in calls
 * enqueued on the handle so far: THIN_EINVAL (and the flag cleared) if a
 * caller's token index lay outside [0, S), THIN_EHIP if the wait failed,
 * THIN_OK otherwise. */
int thin_attn_status(thin_attn_t* h, void* stream);

/* Coreset size of one unit.  Unmasked: n_out = S / 2^j with
 * j = max{ j : 4^j | S and S / 4^j >= 4^g } (each point of weight 2^j).
 * Causal: the cache size n_out (the configured value or the default rule).
 * Returns a negative status on invalid arguments. */
int64_t thin_attn_coreset_size(const thin_attn_t* h, int64_t S, int causal);

/* Entries per unit of the optional coreset arrays of thin_attn_forward:
 * unmasked n_out; causal 6 * n_out (the cache bound of EXPRESS). */
int64_t thin_attn_coreset_capacity(const thin_attn_t* h, int64_t S, int causal);

/* Number of kernel-halving decisions per unit (bytes per unit of the
 * optional decision log). */
int64_t thin_attn_decision_count(const thin_attn_t* h, int64_t S, int causal);

/* Workspace bytes thin_attn_forward needs for these sizes (0 if invalid). */
size_t thin_attn_workspace_size(const thin_attn_t* h, int64_t B, int64_t T, int64_t S, int causal);

/*
 * Thinned attention forward: the Thinformer / Thinformer Express attention
 * layer of the "Thinformer" README ("Getting Started": a drop-in attention
 * call on (query, key, value) with a causal switch, returning the output and
 * the coreset as its second result), with the thinning of "Express Language
 * Modeling" ("Thinformer Express": kernel halving under kappa_att as the base
 * halving; "The EXPRESS Meta-Procedure": the causal exact / thin / HALVE
 * cache).
 *
 * causal = 0 (Thinformer): each unit's S pairs are thinned by a recursive
 * four-way Compress: base blocks of s0 = S / 4^j consecutive tokens; every
 * merge concatenates four compressed quarters and applies one kernel halving
 * (Philox stream: pair, (level << 20) | block, unit, tag 0).  Every query
 * attends to the unit's n_out points (weight 2^j each).
 *
 * causal = 1 (Thinformer Express, requires T == S): tokens are ingested in
 * blocks of n_out.  While m = 1 blocks enter the cache unchanged (exact
 * phase).  While m >= 4 every aligned group of r = m / 2 tokens contributes
 * one Philox-chosen representative of weight r (uniform subsampling); each
 * 2 n_out representatives are halved to n_out points of weight m that join
 * the cache (thin phase).  When the cache holds 4 n_out points it is halved
 * twice back to n_out and m becomes 4 m (HALVE).  A query at token t in block
 * beta attends to the cache and buffer left by blocks 0 .. beta-1 plus the raw
 * tokens beta n_out .. t (weight 1).  Once m / 2 > n_out (past about
 * 2 n_out^2 tokens) a group spans several blocks: its representative joins
 * the buffer when the block completing the group is ingested, and until then
 * the group's earlier tokens carry no weight.  n_out >= 2048 with S >= 4 n_out
 * is THIN_ENOTSUP (the walk of a full cache exceeds one workgroup's LDS).
 *
 * causal = 0 needs the last Compress bin, s0 2^(j+1) points, within the
 * walk's LDS (at most 8106 points), else THIN_ENOTSUP before any launch.
 *
 * Sizes: S, T < 2^30, and one batch entry's keys or values must fit 2 GiB
 * (S * H_kv * max(E, D) * element size < 2^31, H_kv * max(E, D) * element
 * size < 2^24), else THIN_ENOTSUP.
 *
 * Arguments: q, k, v, out as described above (out must not alias inputs);
 * seed keys the Philox4x64-10 stream; optional outputs (NULL to skip):
 *   coreset_idx [B * H_kv, capacity] int32 token indices, ascending, padded -1;
 *   coreset_w   [B * H_kv, capacity] float32 weights, padded 0;
 *   coreset_len [B * H_kv] int32 entries used (causal: final cache, buffer and
 *               trailing partial block; weights sum to S);
 *   decisions   [B * H_kv, decision_count] uint8, 1 = first point of the pair
 *               kept, in the order: unmasked by level, block, pair; causal by
 *               the chronological order of the halvings.
 * workspace must hold thin_attn_workspace_size bytes (256-byte aligned).
 */
int thin_attn_forward(thin_attn_t* h, const void* q, const void* k, const void* v,
                      int64_t B, int64_t T, int64_t S, int causal, uint64_t seed,
                      void* out, int32_t* coreset_idx, float* coreset_w,
                      int32_t* coreset_len, uint8_t* decisions,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * thin_attn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * thin_attn_forward; its scratch is instead a device array of
 * THIN_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  Sizes whose thin_attn_workspace_size exceeds it return
 * THIN_ENOMEM before anything is enqueued.  The call allocates nothing (its
 * device address is looked up once per device, at thin_attn_create for the
 * current device or at the first call on another) and records no launch
 * timing.  Every call on one GPU shares that GPU's array and nothing in it
 * needs clearing between calls; calls whose work overlaps on one GPU (other
 * streams, other host threads, other handles) race on it: serialise them.
 */
#define THIN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int thin_attn_forward_static(thin_attn_t* h, const void* q, const void* k, const void* v,
                             int64_t B, int64_t T, int64_t S, int causal, uint64_t seed,
                             void* out, int32_t* coreset_idx, float* coreset_w,
                             int32_t* coreset_len, uint8_t* decisions, void* stream);

/*
 * Unmasked Thinformer attention over a caller-chosen subset of the keys
 * (thinning after a KV selector: the "Express Language Modeling" explainer
 * on gist.science, "Experimental Results", accelerated KV cache compression,
 * where the thinning step is decoupled from how the initial keys were
 * chosen).  Unit (b, h_kv) thins the L keys key_idx[unit * L + i] (token
 * indices into k / v, each in [0, S), in the order given; any order and
 * repeats allowed) exactly as thin_attn_forward thins S keys in token order:
 * the Compress recursion over list positions, with the coreset size rule,
 * decision layout and Philox streams of an unmasked forward with S = L.
 * Every query then attends to that coreset.  key_idx is read on the device
 * into a copy in the workspace: entries outside [0, S) are clamped into range
 * and reported (see the conventions above), never read out of bounds.
 *
 * Sizes: as thin_attn_forward (unmasked) for S, and L >= 1.  The workspace
 * is thin_attn_workspace_size(h, B, T, L, 0) bytes; the optional outputs
 * have the shapes of an unmasked forward with S = L (capacity
 * thin_attn_coreset_capacity(h, L, 0), decision_count(h, L, 0)) and hold
 * token indices into k / v.
 */
int thin_attn_forward_subset(thin_attn_t* h, const void* q, const void* k, const void* v,
                             const int32_t* key_idx, int64_t B, int64_t T, int64_t S, int64_t L,
                             uint64_t seed, void* out, int32_t* coreset_idx, float* coreset_w,
                             int32_t* coreset_len, uint8_t* decisions,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Weighted-coreset attention alone (no thinning): every query of unit
 * (b, h_kv) attends to the n keys idx[unit * n + j] (token indices into k / v,
 * each in [0, S)) with weights w[unit * n + j] > 0 (w may be NULL: weight 1).
 * idx may be NULL with n == S: exact attention over all keys.  idx entries
 * outside [0, S) are clamped into range and reported (conventions above).
 */
int thin_attn_coreset_attention(thin_attn_t* h, const void* q, const void* k, const void* v,
                                int64_t B, int64_t T, int64_t S, const int32_t* idx,
                                const float* w, int64_t n, void* out, void* stream);

/*
 * One kernel halving per unit, on a given point list (the base halving of
 * both paths, exposed on its own).  points [B * H_kv, N] int32 token indices
 * in [0, S) (N even, 2 <= N <= 2048) name each unit's list x_0 .. x_{N-1};
 * pairs are (x_2i, x_2i+1).  The Philox stream is (pair, bin, unit, tag).
 * Outputs: kept [B * H_kv, N/2] the kept token of every pair; decisions
 * (optional) [B * H_kv, N/2], 1 = first point kept; gram [B * H_kv, N/2, N/2]
 * float64 receives the pair Gram G_ij = <h_i, h_j>, h_i = kappa(x_2i, .) -
 * kappa(x_2i+1, .) (upper triangle G[i][j], j >= i; the rest is left
 * unspecified) and is also the kernel's scratch.  points outside [0, S) are
 * clamped into range and reported (conventions above).  workspace (device,
 * 256-byte aligned, thin_attn_halving_workspace_size bytes, or NULL) is the
 * scratch of the exact integer Gram (THIN_FP64_GRAM); with NULL, or a size
 * of 0, the fp64 Gram runs.  A non-NULL workspace of fewer bytes is
 * THIN_ENOMEM.
 */
int thin_attn_halving(thin_attn_t* h, const void* k, const void* v, int64_t B, int64_t S,
                      const int32_t* points, int64_t N, uint64_t seed, uint32_t tag, uint64_t bin,
                      int32_t* kept, uint8_t* decisions, double* gram, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes of thin_attn_halving over B batch entries with lists of N
 * points (0: its Gram runs in fp64 and needs none). */
size_t thin_attn_halving_workspace_size(const thin_attn_t* h, int64_t B, int64_t N);

/* Philox4x64-10 block for n counters (device arrays, 4 words each) under key
 * (seed, 0); out receives 4 words per counter.  Exposes the generator the
 * halving and subsampling steps draw from. */
int thin_attn_philox(const uint64_t* counters, int64_t n, uint64_t seed, uint64_t* out, void* stream);

/*
 * Streaming Express state for decoding (KV-cache thinning).
 *
 * A state summarises the tokens streamed into it for every unit with the
 * causal schedule of thin_attn_forward (same blocks of n_out tokens, same
 * representatives, halvings and Philox streams, keyed by `seed`), and keeps
 * compact copies of the rows it needs: cache (<= 4 n_out rows), buffer
 * (< 2 n_out) and the block being streamed (< n_out).  Its size does not
 * depend on the stream length ("Express Language Modeling", "The EXPRESS
 * Meta-Procedure": the cache stays within 6 n_out).  Decode queries see
 * exactly what a causal forward query at the same position sees.
 *
 * The caller allocates the device state buffer (thin_attn_kv_state_size
 * bytes, 256-byte aligned) and the per-call workspace; the returned host
 * handle holds the counters and must be destroyed with thin_attn_kv_destroy
 * before the thin_attn handle it was created from.  Streams of any length
 * below 2^30 tokens; n_out <= 1024.  A subsampling group longer than a block
 * keeps its representative's row in the state from the block that contains
 * it until the block that completes the group.
 */
typedef struct thin_kv thin_kv_t;

/* Device bytes of the state of B batch entries (all H_kv heads). 0 if invalid. */
size_t thin_attn_kv_state_size(const thin_attn_t* h, int64_t B, int64_t n_out);

/* Create an empty state over `state` (n_out 0 = the handle's n_out). */
int thin_attn_kv_create(thin_attn_t* h, void* state, size_t state_bytes, int64_t B, int64_t n_out,
                        uint64_t seed, thin_kv_t** out);
int thin_attn_kv_destroy(thin_kv_t* kv);

/* Tokens streamed so far. */
int64_t thin_attn_kv_tokens(const thin_kv_t* kv);

/* Halving decisions per unit that appending n_new tokens will make (decode = 1). */
int64_t thin_attn_kv_decision_count(const thin_kv_t* kv, int64_t n_new);

/* Workspace bytes of an append of n_new tokens or of a decode step (n_new = 1). */
size_t thin_attn_kv_workspace_size(const thin_kv_t* kv, int64_t n_new);

/* Append n_new tokens: k [B, n_new, H_kv, E], v [B, n_new, H_kv, D].  From an
 * empty state with n_new >= n_out the whole chunk is thinned at once (batch
 * halvings in parallel, then the HALVE chain); otherwise block by block.
 * decisions (optional) [B * H_kv, thin_attn_kv_decision_count] receives the
 * decisions of this call in chronological order. */
int thin_attn_kv_append(thin_kv_t* kv, const void* k, const void* v, int64_t n_new, uint8_t* decisions,
                        void* workspace, size_t workspace_bytes, void* stream);

/* One decode step: the new token (k1 [B, H_kv, E], v1 [B, H_kv, D]) is
 * appended and its queries q [B, H, E] attend to the state plus the token
 * itself; out [B, H, D].  decisions as for append (n_new = 1). */
int thin_attn_kv_decode(thin_kv_t* kv, const void* q, const void* k1, const void* v1, void* out,
                        uint8_t* decisions, void* workspace, size_t workspace_bytes, void* stream);

/* What the next query would see: token indices [B * H_kv, 7 n_out] (padded
 * -1), weights (padded 0) and lengths [B * H_kv]; weights sum to the tokens
 * streamed. */
int thin_attn_kv_coreset(thin_kv_t* kv, int32_t* idx, float* w, int32_t* len, void* stream);

/* Checkpoint of the host counters (the device state is the caller's buffer:
 * copy it alongside).  export with host == NULL returns the bytes needed;
 * import restores the counters into a state created with the same B, heads,
 * n_out and seed.  Every counter is fixed by the token count, so import
 * rejects (THIN_EINVAL) a record whose counters differ from the schedule of
 * its token count. */
int64_t thin_attn_kv_export(const thin_kv_t* kv, void* host, size_t bytes);
int thin_attn_kv_import(thin_kv_t* kv, const void* host, size_t bytes);

/* Launch timing.  thin_attn_set_timing(h, 1) starts a fresh list of records:
 * from then on every kernel launch of thin_attn_forward is bracketed by two
 * HIP events on the caller's stream.  thin_attn_timing_count gives the number
 * of records; thin_attn_timing_read(i) waits for record i, copies its kernel
 * label (NUL-terminated, at most label_len bytes) and its duration in
 * milliseconds.  set_timing(h, 0) stops recording and frees the events. */
int thin_attn_set_timing(thin_attn_t* h, int enable);
int64_t thin_attn_timing_count(const thin_attn_t* h);
int thin_attn_timing_read(thin_attn_t* h, int64_t i, char* label, size_t label_len, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* THIN_ATTN_H */
