// Streaming Express state for decoding (gfx950).
//
// The state of a unit holds compact copies of the rows it summarises, so its
// size does not grow with the sequence ("Express Language Modeling",
// "The EXPRESS Meta-Procedure": the cache stays within 6 n_out whatever n):
//
//   slots [0, 4n)    cache C   (weight m)
//   slots [4n, 6n)   buffer Bf (weight m / 2, representatives of the batch)
//   slots [6n, 7n)   raw block (weight 1, tokens of the block being streamed)
//   slot  7n         the representative of a subsampling group longer than a
//                    block (m / 2 > n), held from the block that contains it
//                    until the block that completes the group (not visible)
//
// K rows [units][7n + 1][E], V rows [units][7n + 1][D] (input dtype) and the
// token index of every slot [units][7n + 1] live in the caller's state buffer.  Block
// ingest, batch halving and HALVE move rows between these regions; the
// halvings themselves run the pair-Gram and walk kernels on slot lists.

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace thin {

namespace {

inline unsigned grid1d(int64_t n, int block) { return static_cast<unsigned>((n + block - 1) / block); }

// Copy rows of `cnt` entries per unit.  Source row of entry j of unit u:
//   src_list == nullptr: token src_first + j of a [B, S_src, H_kv, *] tensor (unit = b * H_kv + h)
//   src_list != nullptr: slot src_list[u * list_stride + j] of the state (state-to-state move)
// Destination: state slot dst_first + j.  One 16-byte piece per thread.
__global__ void kv_rows_kernel(KvRowsLaunch a) {
  const int ke = a.E * a.elt / 16, ve = a.D * a.elt / 16;   // 16-byte pieces per row
  const int per_row = ke + ve + 1;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.units) * a.cnt * per_row;
  if (i >= total) return;
  const int piece = static_cast<int>(i % per_row);
  const int64_t e = i / per_row;
  const int j = static_cast<int>(e % a.cnt);
  const int u = static_cast<int>(e / a.cnt);
  const int64_t dslot = static_cast<int64_t>(u) * a.slots + a.dst_first + j;
  const char* sk;
  const char* sv;
  int32_t tok;
  if (a.src_list) {
    const int32_t slot = a.src_list[static_cast<int64_t>(u) * a.list_stride + j];
    const int64_t s = static_cast<int64_t>(u) * a.slots + slot;
    sk = static_cast<const char*>(a.state_k) + s * a.E * a.elt;
    sv = static_cast<const char*>(a.state_v) + s * a.D * a.elt;
    tok = a.state_tok[s];
  } else {
    const int b = u / a.H_kv, h = u % a.H_kv;
    const int64_t tk = a.tok_list ? a.tok_list[static_cast<int64_t>(u) * a.list_stride + j] : a.src_first + j;
    const int64_t row = (static_cast<int64_t>(b) * a.S_src + tk) * a.H_kv + h;
    sk = static_cast<const char*>(a.src_k) + row * a.E * a.elt;
    sv = static_cast<const char*>(a.src_v) + row * a.D * a.elt;
    tok = static_cast<int32_t>(a.tok_base + tk);
  }
  if (piece < ke) {
    reinterpret_cast<uint4*>(static_cast<char*>(a.state_k) + dslot * a.E * a.elt)[piece] =
        reinterpret_cast<const uint4*>(sk)[piece];
  } else if (piece < ke + ve) {
    reinterpret_cast<uint4*>(static_cast<char*>(a.state_v) + dslot * a.D * a.elt)[piece - ke] =
        reinterpret_cast<const uint4*>(sv)[piece - ke];
  } else {
    a.state_tok_out[dslot] = tok;
  }
}

// Slots of the representatives of the block starting at token t0 (groups of
// r <= n tokens; each contributes the token at offset floor(u r) of its group,
// u from counter (group, log2 r, unit, subsample tag)).
__global__ void kv_block_reps_kernel(int units, int n, int64_t t0, int log2r, uint64_t seed, int32_t* list) {
  const int per = n >> log2r;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(units) * per) return;
  const int u = static_cast<int>(i / per);
  const int k = static_cast<int>(i % per);
  const int64_t g = (t0 >> log2r) + k;
  const uint64_t word = philox_word0(static_cast<uint64_t>(g), static_cast<uint64_t>(log2r), static_cast<uint64_t>(u),
                                     kTagSubsample, seed);
  const int64_t off = log2r ? static_cast<int64_t>(word >> (64 - log2r)) : 0;
  list[i] = static_cast<int32_t>(6 * n + ((g << log2r) + off - t0));
}

// The representative of group g (r = 2^log2r tokens): token g r + floor(u r),
// u from counter (g, log2 r, unit, subsample tag).  list[u] = base + (token -
// lo) when the token lies in [lo, hi), else fallback.
__global__ void kv_group_rep_kernel(int units, int64_t g, int log2r, uint64_t seed, int64_t lo, int64_t hi, int64_t base,
                                    int32_t fallback, int32_t* list) {
  const int u = static_cast<int>(static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
  if (u >= units) return;
  const uint64_t word = philox_word0(static_cast<uint64_t>(g), static_cast<uint64_t>(log2r), static_cast<uint64_t>(u),
                                     kTagSubsample, seed);
  const int64_t tok = (g << log2r) + (log2r ? static_cast<int64_t>(word >> (64 - log2r)) : 0);
  list[u] = (tok >= lo && tok < hi) ? static_cast<int32_t>(base + (tok - lo)) : fallback;
}

__global__ void kv_fill_kernel(int32_t* out, int64_t n, int32_t value) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = value;
}

__global__ void kv_iota_kernel(int32_t* out, int units, int cnt, int first) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(units) * cnt) return;
  out[i] = first + static_cast<int>(i % cnt);
}

// Token indices and weights of what the next query would see (cache, buffer,
// raw block), padded with -1 / 0 up to cap.
__global__ void kv_summary_kernel(const int32_t* tok, int slots, int n, int nC, int nBf, int nRaw, float wc, float wb,
                                  int32_t* idx, float* w, int32_t* len, int cap) {
  const int u = blockIdx.x;
  const int total = nC + nBf + nRaw;
  for (int j = threadIdx.x; j < cap; j += blockDim.x) {
    int32_t id = -1;
    float wt = 0.f;
    if (j < nC) {
      id = tok[static_cast<int64_t>(u) * slots + j];
      wt = wc;
    } else if (j < nC + nBf) {
      id = tok[static_cast<int64_t>(u) * slots + 4 * n + (j - nC)];
      wt = wb;
    } else if (j < total) {
      id = tok[static_cast<int64_t>(u) * slots + 6 * n + (j - nC - nBf)];
      wt = 1.f;
    }
    if (idx) idx[static_cast<int64_t>(u) * cap + j] = id;
    if (w) w[static_cast<int64_t>(u) * cap + j] = wt;
  }
  if (len && threadIdx.x == 0) len[u] = total;
}

// ---------------------------------------------------------------------------
// Decode attention: one query token, G = H / H_kv query heads per unit.
// Visible keys = cache slots [0, nC) (log2 weight lw_c), buffer slots
// [4n, 4n + nBf) (lw_b), raw slots [6n, 6n + nRaw) (weight 1) and the new
// token itself (read from the caller's k1 / v1).  The key range is split
// across workgroups of KPW keys (32, 64 or 128, the smallest whose partials
// the merge can hold in LDS, so short states still spread over many
// workgroups); each writes a partial (max, sum,
// unnormalised output) per query head, and the last workgroup of a unit to
// finish (a per-unit counter, zero before and after the launch) merges them.
// Workgroup 0 of a unit also appends the new token to the raw block.
//
// Every memory read of a workgroup is issued up front: the queries, the key
// rows (256 / KPW threads per key, each holding every (256 / KPW)-th 16-byte
// piece, so a wave reads whole rows coalesced) and the split's value rows
// into LDS.  The threads of a key form partial dots for all G heads and sum
// them with lane shuffles; P V then runs from LDS with one thread per (head,
// pair of dimensions).
// ---------------------------------------------------------------------------
constexpr int kMinSplitKeys = 32;   // smallest keys per workgroup

// Row of visible key kk: its state row u * slots + slot, or -1 for the new token (kk = total - 1).
__device__ __forceinline__ int64_t key_state_row(const KvDecodeLaunch& a, int u, int kk, int total) {
  const int slot = kk < a.nC ? kk : (kk < a.nC + a.nBf ? 4 * a.n + kk - a.nC : 6 * a.n + kk - a.nC - a.nBf);
  return kk < total - 1 ? static_cast<int64_t>(u) * a.slots + slot : -1;
}

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other) through device-scope atomic stores and loads, which go to the
// coherence point, so no cache-wide fence is needed.
__device__ __forceinline__ void put_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_partial(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the partials of unit u (run by its last workgroup): out = sum_s
// 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s.  When the unit's partials fit
// kMergeBytes, they are copied into LDS in one round (LDS-DMA loads with the
// device-coherent cache policy, 16 bytes a lane, all in flight at once); the
// per-split weights are then formed by one thread per head and every output
// sums its splits from LDS.  Otherwise each output reads its splits itself.
constexpr int kMergeBytes = 64 * 1024;
constexpr int kMergeSplits = 64;
constexpr int kDmaSc1 = 16;   // cache policy of a device-scope coherent load (sc1)

template <int ET, int D, int G>
__device__ __forceinline__ void combine_unit(const float* partial, int u, int splits, int H, int H_kv, void* out,
                                             unsigned char* lds) {
  constexpr int PS = D + 4;   // floats per partial row
  __shared__ float s_w[kMergeSplits][G];
  const int b = u / H_kv, hk = u % H_kv;
  const float* unit_p = partial + static_cast<int64_t>(u) * splits * G * PS;
  const int pieces = splits * G * PS / 4;
  const bool fast = splits <= kMergeSplits && (pieces + 63) / 64 * 1024 <= kMergeBytes;
  const float* sp = reinterpret_cast<const float*>(lds);
  if (fast) {
    typedef __attribute__((address_space(1))) const void* gptr;
    typedef __attribute__((address_space(3))) void* lptr;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int i = w; i < (pieces + 63) / 64; i += 4) {
      const int piece = min(64 * i + lane, pieces - 1);   // lanes past the end reload the last piece into padding
      __builtin_amdgcn_global_load_lds((gptr)(unit_p + 4 * piece), (lptr)(lds + 1024 * i), 16, 0, kDmaSc1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // weights of head gh: one wave, a lane per split
    for (int gh = w; gh < G; gh += 4) {
      const bool in = lane < splits;
      const float ms = in ? sp[(lane * G + gh) * PS + D] : -INFINITY;
      const float ls = in ? sp[(lane * G + gh) * PS + D + 1] : 0.f;
      float m = ms;
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      const float e = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m);
      float den = e * ls;
      for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, 64);
      if (in) s_w[lane][gh] = e / den;
    }
    __syncthreads();
  }
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
    const int gh = x / D, d = x % D;
    float o;
    if (fast) {
      o = 0.f;
      for (int s = 0; s < splits; ++s) o = fmaf(s_w[s][gh], sp[(s * G + gh) * PS + d], o);
    } else {
      const float* base = unit_p + static_cast<int64_t>(gh) * PS;
      float m = -INFINITY;
#pragma unroll 8
      for (int s = 0; s < splits; ++s) m = fmaxf(m, get_partial(base + static_cast<int64_t>(s) * G * PS + D));
      float num = 0.f, den = 0.f;
#pragma unroll 8
      for (int s = 0; s < splits; ++s) {
        const float* p = base + static_cast<int64_t>(s) * G * PS;
        const float ms = get_partial(p + D);
        const float sc = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m);
        num = fmaf(sc, get_partial(p + d), num);
        den = fmaf(sc, get_partial(p + D + 1), den);
      }
      o = num / den;
    }
    const int64_t off = (static_cast<int64_t>(b) * H + hk * G + gh) * D + d;
    if constexpr (ET != kF32)   // bfloat16 output (fp8 inputs too)
      static_cast<uint16_t*>(out)[off] = float_to_bf16_bits(o);
    else
      static_cast<float*>(out)[off] = o;
  }
}

template <int ET, int E, int D, int G, int KPW>
__global__ __launch_bounds__(256) void kv_decode_kernel(KvDecodeLaunch a) {
  constexpr int ELT = elt_size<ET>();
  constexpr int FP = 16 / ELT;                          // features per 16-byte piece
  constexpr int VP = D * ELT / 16;                      // 16-byte pieces per value row
  constexpr int VLOADS = KPW * VP / 256;                // value pieces per thread
  constexpr int KP = E * ELT / 16;                      // 16-byte pieces per key row
  constexpr int TPK = 256 / KPW;                        // threads per key
  constexpr int KPT = KP / TPK;                         // key pieces per thread
  static_assert(KPT * TPK == KP && VLOADS * 256 == KPW * VP, "key or value rows do not tile the workgroup");
  const int u = blockIdx.y;
  const int split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = u / a.H_kv, hk = u % a.H_kv;
  const int total = a.nC + a.nBf + a.nRaw + 1;
  const int k0 = split * KPW;
  const int nk = min(total, k0 + KPW) - k0;

  constexpr int PS = D + 4;                              // floats per partial row (16-byte multiple)
  // value rows of the split; later the unit's partials when this workgroup merges
  constexpr int kBuf = KPW * D * ELT > kMergeBytes ? KPW * D * ELT : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char sv[kBuf];
  __shared__ __attribute__((aligned(16))) float sq[G][E];
  __shared__ float sp[G][KPW];
  __shared__ float red[4][G];
  __shared__ float smax[G], ssum[G];

  // value rows of the split (rows past the range are not read)
  uint4 vr[VLOADS];
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) {
    const int piece = tid + 256 * i, j = piece / VP;
    const int64_t r = key_state_row(a, u, k0 + j, total);
    const uint4* src = r >= 0 ? reinterpret_cast<const uint4*>(static_cast<const char*>(a.state_v) + r * (D * ELT))
                              : reinterpret_cast<const uint4*>(static_cast<const char*>(a.v1) +
                                                               (static_cast<int64_t>(b) * a.H_kv + hk) * (D * ELT));
    vr[i] = j < nk ? src[piece % VP] : uint4{0u, 0u, 0u, 0u};
  }
  // this thread's share of key kk: pieces slice, slice + TPK, ...
  const int jk = tid / TPK, slice = tid % TPK;
  const int kk = k0 + jk;
  const bool live = jk < nk;
  uint4 kr[KPT];
  if (live) {
    const int64_t r = key_state_row(a, u, kk, total);
    const uint4* krow = r >= 0 ? reinterpret_cast<const uint4*>(static_cast<const char*>(a.state_k) + r * (E * ELT))
                               : reinterpret_cast<const uint4*>(static_cast<const char*>(a.k1) +
                                                                (static_cast<int64_t>(b) * a.H_kv + hk) * (E * ELT));
#pragma unroll
    for (int i = 0; i < KPT; ++i) kr[i] = krow[slice + TPK * i];
  }
  // queries of the group
  for (int x = tid; x < G * E; x += 256) {
    const int gh = x / E, e = x % E;
    const int64_t off = (static_cast<int64_t>(b) * a.H + hk * G + gh) * E + e;
    if constexpr (ET == kFP8)
      sq[gh][e] = fp8_low_to_float(static_cast<const uint8_t*>(a.q)[off]);
    else if constexpr (ET == kBF16)
      sq[gh][e] = bf16_bits_to_float(static_cast<const uint16_t*>(a.q)[off]);
    else
      sq[gh][e] = static_cast<const float*>(a.q)[off];
  }
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) reinterpret_cast<uint4*>(sv)[tid + 256 * i] = vr[i];
  __syncthreads();

  // logits: the TPK threads of a key sum their partial dots
  float acc[G];
#pragma unroll
  for (int gh = 0; gh < G; ++gh) acc[gh] = 0.f;
  if (live) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int piece = slice + TPK * i;
      const uint32_t wv[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
      float kv[FP];
      if constexpr (ET == kFP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) kv[4 * j + bb] = fp8_byte_to_float(wv[j], bb);
      } else if constexpr (ET == kBF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv[2 * j] = __uint_as_float(wv[j] << 16);
          kv[2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[j] = __uint_as_float(wv[j]);
      }
#pragma unroll
      for (int gh = 0; gh < G; ++gh)
#pragma unroll
        for (int j4 = 0; j4 < FP; j4 += 4) {   // the group's queries, 16 bytes per LDS read
          const float4 qv = *reinterpret_cast<const float4*>(&sq[gh][piece * FP + j4]);
          acc[gh] = fmaf(qv.x, kv[j4], acc[gh]);
          acc[gh] = fmaf(qv.y, kv[j4 + 1], acc[gh]);
          acc[gh] = fmaf(qv.z, kv[j4 + 2], acc[gh]);
          acc[gh] = fmaf(qv.w, kv[j4 + 3], acc[gh]);
        }
    }
  }
  float logit[G];
  const float lw = kk < a.nC ? a.lw_c : (kk < a.nC + a.nBf ? a.lw_b : 0.f);
#pragma unroll
  for (int gh = 0; gh < G; ++gh) {
    float d = acc[gh];
#pragma unroll
    for (int off = 1; off < TPK; off <<= 1) d += __shfl_xor(d, off, 64);
    logit[gh] = live ? fmaf(d, a.scale_log2, lw) : -INFINITY;
  }
  // max and sum over the split (the threads of a key hold the same logit, so
  // the wave reductions run over lanes TPK apart: one lane per key)
#pragma unroll
  for (int gh = 0; gh < G; ++gh) {
    float m = logit[gh];
#pragma unroll
    for (int off = 32; off >= TPK; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (lane == 0) red[w][gh] = m;
  }
  __syncthreads();
  if (tid < G) smax[tid] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
  __syncthreads();
#pragma unroll
  for (int gh = 0; gh < G; ++gh) {
    const float p = live ? __builtin_amdgcn_exp2f(logit[gh] - smax[gh]) : 0.f;
    if (slice == 0) sp[gh][jk] = p;
    float s = p;
#pragma unroll
    for (int off = 32; off >= TPK; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) red[w][gh] = s;
  }
  __syncthreads();
  if (tid < G) ssum[tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
  // P V from LDS: thread = (head, two dimensions)
  float* part = a.partial + ((static_cast<int64_t>(u) * gridDim.x + split) * G) * PS;
  for (int x = tid; x < G * D / 2; x += 256) {
    const int gh = x / (D / 2), d2 = x % (D / 2);
    float o0 = 0.f, o1 = 0.f;
    for (int j = 0; j < nk; ++j) {
      const float p = sp[gh][j];
      float v0, v1;
      if constexpr (ET == kFP8) {
        const uint32_t vv = reinterpret_cast<const uint16_t*>(sv + j * D * ELT)[d2];
        v0 = fp8_byte_to_float(vv, 0);
        v1 = fp8_byte_to_float(vv, 1);
      } else if constexpr (ET == kBF16) {
        const uint32_t vv = reinterpret_cast<const uint32_t*>(sv + j * D * ELT)[d2];
        v0 = __uint_as_float(vv << 16);
        v1 = __uint_as_float(vv & 0xffff0000u);
      } else {
        const float2 vv = reinterpret_cast<const float2*>(sv + j * D * ELT)[d2];
        v0 = vv.x;
        v1 = vv.y;
      }
      o0 = fmaf(p, v0, o0);
      o1 = fmaf(p, v1, o1);
    }
    put_partial(part + gh * PS + 2 * d2, o0);
    put_partial(part + gh * PS + 2 * d2 + 1, o1);
  }
  if (tid < G) {
    put_partial(part + tid * PS + D, smax[tid]);
    put_partial(part + tid * PS + D + 1, ssum[tid]);
  }
  // workgroup 0: the new token joins the raw block (slot new_slot, which no
  // workgroup of this launch reads)
  if (split == 0) {
    const int64_t dst = static_cast<int64_t>(u) * a.slots + a.new_slot;
    const int64_t src = static_cast<int64_t>(b) * a.H_kv + hk;
    if (tid < KP)
      reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.state_k)) + dst * (E * ELT))[tid] =
          reinterpret_cast<const uint4*>(static_cast<const char*>(a.k1) + src * (E * ELT))[tid];
    else if (tid < KP + VP)
      reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.state_v)) + dst * (D * ELT))[tid - KP] =
          reinterpret_cast<const uint4*>(static_cast<const char*>(a.v1) + src * (D * ELT))[tid - KP];
    else if (tid == KP + VP)
      a.state_tok[dst] = a.new_tok;
  }
  // the last workgroup of the unit merges the partials.  The workgroup's
  // partial stores happen before its count (barrier, then a release at device
  // scope by the counting thread); the workgroup that takes the last count
  // acquires at device scope before any of its threads reads a partial.
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int prior = __hip_atomic_fetch_add(&a.cnt[u], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prior == static_cast<int>(gridDim.x) - 1;
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_last) return;   // the whole workgroup
  combine_unit<ET, D, G>(a.partial, u, gridDim.x, a.H, a.H_kv, a.out, sv);
  if (tid == 0) __hip_atomic_store(&a.cnt[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Keys per workgroup: the smallest of 32, 64, 128 whose partials the merge
// holds in LDS (else 128, merged from global memory).
template <int D, int G>
int decode_keys_per_wg(int total) {
  for (int kpw = kMinSplitKeys; kpw < 128; kpw *= 2) {
    const int splits = (total + kpw - 1) / kpw;
    const int pieces = splits * G * (D + 4) / 4;
    if (splits <= kMergeSplits && (pieces + 63) / 64 * 1024 <= kMergeBytes) return kpw;
  }
  return 128;
}

template <int ET, int E, int D, int G>
hipError_t decode_one(const KvDecodeLaunch& a, hipStream_t s) {
  const int total = a.nC + a.nBf + a.nRaw + 1;
  const int kpw = decode_keys_per_wg<D, G>(total);
  KvDecodeLaunch b = a;
  b.splits = (total + kpw - 1) / kpw;
  const dim3 grid(b.splits, a.units);
  if (kpw == 32)
    hipLaunchKernelGGL((kv_decode_kernel<ET, E, D, G, 32>), grid, dim3(256), 0, s, b);
  else if (kpw == 64)
    hipLaunchKernelGGL((kv_decode_kernel<ET, E, D, G, 64>), grid, dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL((kv_decode_kernel<ET, E, D, G, 128>), grid, dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace

int kv_decode_splits(int n) { return (7 * n + kMinSplitKeys) / kMinSplitKeys; }   // 7n + 1 keys at most

hipError_t launch_kv_rows(const KvRowsLaunch& a, hipStream_t s) {
  const int per_row = (a.E + a.D) * a.elt / 16 + 1;
  const int64_t total = static_cast<int64_t>(a.units) * a.cnt * per_row;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_rows_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_block_reps(int units, int n, int64_t t0, int log2r, uint64_t seed, int32_t* list, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(units) * (n >> log2r);
  hipLaunchKernelGGL(kv_block_reps_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, units, n, t0, log2r, seed, list);
  return hipGetLastError();
}

hipError_t launch_kv_group_rep(int units, int64_t g, int log2r, uint64_t seed, int64_t lo, int64_t hi, int64_t base,
                               int32_t fallback, int32_t* list, hipStream_t s) {
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_group_rep_kernel, dim3(grid1d(units, 256)), dim3(256), 0, s, units, g, log2r, seed, lo, hi,
                     base, fallback, list);
  return hipGetLastError();
}

hipError_t launch_kv_fill(int32_t* out, int64_t n, int32_t value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_fill_kernel, dim3(grid1d(n, 256)), dim3(256), 0, s, out, n, value);
  return hipGetLastError();
}

hipError_t launch_kv_iota(int32_t* out, int units, int cnt, int first, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(units) * cnt;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_iota_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, out, units, cnt, first);
  return hipGetLastError();
}

hipError_t launch_kv_summary(const int32_t* tok, int units, int slots, int n, int nC, int nBf, int nRaw, float wc,
                             float wb, int32_t* idx, float* w, int32_t* len, int cap, hipStream_t s) {
  if (units == 0 || (!idx && !w && !len)) return hipSuccess;
  hipLaunchKernelGGL(kv_summary_kernel, dim3(units), dim3(256), 0, s, tok, slots, n, nC, nBf, nRaw, wc, wb, idx, w, len,
                     cap);
  return hipGetLastError();
}

bool kv_decode_supported(int dtype, int E, int D, int G) {
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  if (dtype == kFP8) return g_ok && E == 128 && D == 128;
  return g_ok && ((E == 128 && D == 128) || (E == 64 && D == 64));
}

hipError_t launch_kv_decode(const KvDecodeLaunch& a, int dtype, int E, int D, int G, hipStream_t s) {
#define THIN_KV_CASE(BF, EE, DD, GG) \
  if (dtype == BF && E == EE && D == DD && G == GG) return decode_one<BF, EE, DD, GG>(a, s);
  THIN_KV_CASE(1, 128, 128, 1)
  THIN_KV_CASE(1, 128, 128, 2)
  THIN_KV_CASE(1, 128, 128, 4)
  THIN_KV_CASE(1, 128, 128, 8)
  THIN_KV_CASE(1, 64, 64, 1)
  THIN_KV_CASE(1, 64, 64, 2)
  THIN_KV_CASE(1, 64, 64, 4)
  THIN_KV_CASE(1, 64, 64, 8)
  THIN_KV_CASE(0, 128, 128, 1)
  THIN_KV_CASE(0, 128, 128, 2)
  THIN_KV_CASE(0, 128, 128, 4)
  THIN_KV_CASE(0, 128, 128, 8)
  THIN_KV_CASE(0, 64, 64, 1)
  THIN_KV_CASE(0, 64, 64, 2)
  THIN_KV_CASE(0, 64, 64, 4)
  THIN_KV_CASE(0, 64, 64, 8)
  THIN_KV_CASE(2, 128, 128, 1)
  THIN_KV_CASE(2, 128, 128, 2)
  THIN_KV_CASE(2, 128, 128, 4)
  THIN_KV_CASE(2, 128, 128, 8)
#undef THIN_KV_CASE
  return hipErrorInvalidValue;
}

}  // namespace thin
