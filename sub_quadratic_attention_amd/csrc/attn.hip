// Weighted-coreset / Express softmax attention on gfx950, fp32, bf16 and fp8.
//
// out(q) = sum_j w_j e^{s <q, k_j>} v_j / sum_j w_j e^{s <q, k_j>} over the keys
// a query sees ("Express Language Modeling": attention against a small
// weighted summary of the keys and values).  ln w_j is folded into the logit,
// the softmax is taken online (running maximum and sum), accumulation is fp32,
// and both products run on MFMA: v_mfma_f32_16x16x32_bf16 for bf16 inputs,
// v_mfma_f32_16x16x4f32 for fp32 inputs.  FP8 (E4M3) inputs take Q K^T on the
// gfx950 FP8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, unit scales, one
// instruction per 128 features) and P V on the bf16 MFMA: V rows are widened
// to bf16 (exactly) as they are staged, and P is rounded to bf16 as for bf16
// inputs, so the arithmetic after Q K^T is the bf16 path's.
//
// The keys a query sees are a gathered part (a coreset, or the cache and
// buffer index lists of the Express state, each list with its log-weight)
// followed by a raw token range (weight 1; causal inside the block being
// streamed).
//
// Layout:
//  * one workgroup = 4 waves x 16 NQG queries of one (b, h); two workgroups
//    fit one CU, so one workgroup's MFMA phase overlaps the other's softmax;
//  * the keys visible to the workgroup form one stream: its token indices
//    (gathered lists, then the raw tail) are staged in LDS in windows of up to
//    kIdxCap keys (a stream of only a raw range needs none), then 64-key chunks
//    of K and V go through two LDS buffers with one barrier per chunk: chunk
//    c + 1 is copied from memory straight into LDS (global_load_lds_dwordx4,
//    16 bytes per lane, no registers) while chunk c is consumed;
//  * K and V rows sit unpadded in LDS; the 16-byte pieces of row R are stored
//    permuted (piece q at q ^ f(R)), which the copy does for free by choosing
//    the global piece each lane fetches, and which puts the operand reads on
//    distinct banks;
//  * S^T = K Q^T keeps one query per lane column, so softmax statistics and
//    the O^T = V^T P^T accumulator of a query share lanes; each K (and V)
//    fragment read from LDS feeds the NQG query groups of the wave;
//  * bf16: the V operand of P V is read with the gfx950 transposing LDS read
//    (ds_read_tr16_b64): within each 16-lane group, lane j receives element
//    j % 4 of the 8-byte pieces addressed by lanes j/4 + 4k (k = 0..3), so
//    lanes addressing V[k0 + i/4][d0 + 4 (i % 4)] deliver V[k0..k0+3][d0 + j]
//    to lane j: four keys of one dimension, as the MFMA operand wants;
//  * fp32: the order of the reduction inside an MFMA only has to agree between
//    its operands, so lane group g of k-step t of feature block kq takes
//    feature 16 kq + 4 g + t (one 16-byte K read per four MFMAs); for P V, a
//    lane reads four consecutive dimensions of a key row with one 16-byte read
//    and feeds them to four output blocks whose rows interleave the
//    dimensions (block 4 j + d4, row r = dimension 64 j + 4 r + d4).

#include <limits.h>
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace thin {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kC = 64;          // keys per chunk
constexpr int kIdxCap = 1536;   // gathered indices staged per window
constexpr int kIdxPT = kIdxCap / kThreads;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0), other counters unconstrained

template <int ET, int E, int D>
constexpr int nqg() { return (ET != kF32 ? (E <= 128 && D <= 128) : D <= 64) ? 2 : 1; }   // 16-query groups per wave

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) unsigned char lds_byte;   // LDS views of the buffers

// Maximum / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// holding one query's keys) with the gfx950 lane swaps, which stay in the
// VALU (a shuffle through ds_bpermute waits on an LDS round trip).  Each swap
// returns both halves, so max / sum of the pair is the value of lane l ^ 32
// (then l ^ 16) combined with lane l's, identically in both lanes.
__device__ __forceinline__ float group_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Piece permutations.  K is read 16 bytes per lane, 16 consecutive rows at one
// logical piece: 128-byte rows (two per 256 bytes of banks) take
// q ^ (R / 2 % 8), longer rows q ^ (R % 16).  bf16 V is read 8 bytes per lane
// by the transposing read, 8 rows x 32 bytes (pieces 2d, 2d + 1) at a time:
// the permutation keeps the pair together, 2 (R / 2 % 4) for 128-byte rows,
// 2 (R % 8) for longer ones.  fp32 V is read a whole row per 16 lanes and
// needs no permutation.
template <int RB>
__device__ __forceinline__ int kswz(int R) { return RB == 128 ? (R >> 1) & 7 : R & 15; }
template <bool BF16, int RB>
__device__ __forceinline__ int vswz(int R) {   // BF16: V staged as bf16 rows (bf16 and fp8 inputs)
  if constexpr (!BF16) return 0;
  else return RB == 128 ? 2 * ((R >> 1) & 3) : 2 * (R & 7);
}

// Gathered part of a stream: up to three index lists, one after the other.
// Lists 0 and 1 carry log2-weight lnw2, list 2 half that weight (lnw2 - 1);
// a single list may instead carry per-entry weights w.
struct Gather {
  const int32_t* p[3];
  int cnt[3];
  float lnw2;
  const float* w;
};

// Raw part: tokens start .. start + count - 1, log2-weight lnw2, causal mask.
struct Raw {
  int start, count;
  float lnw2;
  int causal;
};

// NB chunk buffers: two let the copy of the next chunk overlap the current
// one; a stream of at most one chunk (a coreset of <= kC keys) needs one,
// which leaves LDS for more workgroups per CU.
template <int ET, int E, int D, int NB>
struct Smem {
  // row bytes: K as given, V as staged (bf16 for fp8 inputs)
  static constexpr int KB = E * elt_size<ET>(), VB = D * (ET == kF32 ? 4 : 2);
  alignas(16) unsigned char k[NB][kC * KB];   // 16-byte pieces permuted by kswz(row)
  alignas(16) unsigned char v[NB][kC * VB];   // 16-byte pieces permuted by vswz(row)
  float lnw2[NB][kC];
  int idx[kIdxCap];
};

// RAW: the stream is one raw token range (exact attention), tokens computed;
// otherwise every token of the stream is staged in sm.idx.  NB = 1: every
// window is a single chunk (the launcher picks it only then).
template <int ET, int E, int D, bool RAW, int NB>
struct Attn {
  static constexpr bool BF16 = ET != kF32;            // bf16 P V (bf16 and fp8 inputs)
  static constexpr bool FP8 = ET == kFP8;
  static constexpr int ELT = elt_size<ET>();
  static constexpr int KB = E * ELT;                  // K row bytes (memory and LDS)
  static constexpr int VB = D * (BF16 ? 2 : 4);       // V row bytes in LDS
  static constexpr int VGB = D * ELT;                 // V row bytes in memory
  static constexpr int NQG = nqg<ET, E, D>();
  static constexpr int NQF = FP8 ? E / 128 : (BF16 ? E / 32 : E / 4);   // Q operand registers per query group
  static constexpr int ND = D / 16;                   // 16-dimension output blocks
  static constexpr int KP = KB / 16, VP = VB / 16;    // 16-byte pieces per row (LDS)
  static constexpr int VGP = VGB / 16;                // 16-byte pieces per V row in memory
  static constexpr int KPT = kC * KP / kThreads;      // copies per thread per chunk
  static constexpr int VPT = kC * VP / kThreads;
  static constexpr int VGPT = kC * VGP / kThreads;    // fp8: V pieces loaded per thread per chunk
  using QF = typename std::conditional<FP8, i32x8_t, typename std::conditional<BF16, bf16x8_t, float>::type>::type;

  const AttnLaunch& a;
  Smem<ET, E, D, NB>& sm;
  int b, h, hk, unit, lane, g;
  // K / V rows of this unit: token t starts at kbase + t * kstride bytes;
  // offsets stay below 2^31 (checked by the host), so they are 32-bit
  const unsigned char* kbase;
  const unsigned char* vbase;
  uint32_t kstride, vstride;
  int qr[NQG];
  bool live[NQG];
  QF qf[NQG][NQF];
  QF qn[NQG][NQF];   // NB = 1: the next tile's operands, fetched ahead
  f32x4_t o[NQG][ND];
  f32x4_t osum[NQG];   // bf16: row sums of P (all four elements equal)
  float m_run[NQG], l_run[NQG];

  uint4 vreg[VGPT > 0 ? VGPT : 1];   // fp8: V pieces of the next chunk, in flight

  // the stream: G gathered keys, then raw.count raw ones; current window [w0, w0 + wl)
  Gather gs;
  Raw raw;
  int G, w0, wl;
  // the key at stream position pos is visible to query group qg's query iff
  // pos <= vlim[qg]: every gathered key and the raw keys up to the query's
  // token (INT_MAX without the causal mask, -1 when the query is not in the
  // stream's block); padding keys carry log-weight -inf instead.  rows_ok:
  // every query of the wave is in the block (then only raw causal keys need
  // the test)
  int vlim[NQG];
  bool rows_ok;

  __device__ __forceinline__ Attn(const AttnLaunch& la, Smem<ET, E, D, NB>& s, int q0, int bh) : a(la), sm(s) {
    b = bh / a.H;
    h = bh % a.H;
    hk = h / (a.H / a.H_kv);
    unit = b * a.H_kv + hk;
    kstride = static_cast<uint32_t>(a.H_kv * KB);
    vstride = static_cast<uint32_t>(a.H_kv * VGB);
    kbase = static_cast<const unsigned char*>(a.k) + (static_cast<int64_t>(b) * a.S * a.H_kv + hk) * KB;
    vbase = static_cast<const unsigned char*>(a.v) + (static_cast<int64_t>(b) * a.S * a.H_kv + hk) * VGB;
    lane = threadIdx.x & 63;
    g = lane >> 4;
    load_q(q0);
  }

  // Row of query group qg in the tile starting at q0 (rows >= T are not live).
  __device__ __forceinline__ int q_row(int q0, int qg) const {
    return q0 + 16 * NQG * (threadIdx.x >> 6) + 16 * qg + (lane & 15);
  }

  // The query operands of the tile starting at q0 into dst (zeros past T).
  __device__ __forceinline__ void fetch_q(int q0, QF (&dst)[NQG][NQF]) const {
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      const int r = q_row(q0, qg);
      const bool ok = r < a.t1;
      const int64_t qrow = ((static_cast<int64_t>(b) * a.T + (ok ? r : 0)) * a.H + h) * E;
      if constexpr (FP8) {
        // lane group g: features 32 g .. 32 g + 31 of each 128 (the K operand uses the same slices)
#pragma unroll
        for (int kk = 0; kk < NQF; ++kk) {
          const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) + qrow + kk * 128 + 32 * g);
          const uint4 lo = ok ? src[0] : uint4{0u, 0u, 0u, 0u}, hi = ok ? src[1] : uint4{0u, 0u, 0u, 0u};
          dst[qg][kk] = i32x8_t{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                                static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                                static_cast<int>(hi.z), static_cast<int>(hi.w)};
        }
      } else if constexpr (BF16) {
#pragma unroll
        for (int kk = 0; kk < NQF; ++kk) {
          const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(static_cast<const uint16_t*>(a.q) + qrow + kk * 32 + 8 * g);
          dst[qg][kk] = ok ? *src : bf16x8_t{};
        }
      } else {
#pragma unroll
        for (int kq = 0; kq < E / 16; ++kq) {
          const float4 x = ok ? *reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qrow + 16 * kq + 4 * g)
                              : float4{0.f, 0.f, 0.f, 0.f};
          dst[qg][4 * kq] = x.x, dst[qg][4 * kq + 1] = x.y, dst[qg][4 * kq + 2] = x.z, dst[qg][4 * kq + 3] = x.w;
        }
      }
    }
  }

  // Rows of the tile starting at q0; accumulators cleared.
  __device__ __forceinline__ void start_tile(int q0) {
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      qr[qg] = q_row(q0, qg);
      live[qg] = qr[qg] < a.t1;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[qg][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      osum[qg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_run[qg] = -INFINITY;
      l_run[qg] = 0.f;
    }
  }

  // The query tile starting at q0 into registers; accumulators cleared.
  __device__ __forceinline__ void load_q(int q0) {
    fetch_q(q0, qf);
    start_tile(q0);
  }

  // One-chunk streams (NB = 1): another query tile of the same unit against the
  // chunk that run_stream left in buffer 0 (nothing writes the buffers after
  // it is staged, so no barrier is needed).  Unmasked only: every row is in the
  // stream.  Its operands were fetched into qn one tile earlier; the tile at
  // q0_next (>= T: none) is fetched now, to land while this one computes.
  __device__ __forceinline__ void rerun_single(int q0, int q0_next) {
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk) qf[qg][kk] = qn[qg][kk];
    start_tile(q0);
    fetch_q(q0_next, qn);
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) vlim[qg] = INT_MAX;
    consume(0, 0, (const lds_byte*)&sm.k[0][0], (const lds_byte*)&sm.v[0][0]);
  }

  // token of window position r (r < wl)
  __device__ __forceinline__ int token(int r) const {
    if constexpr (RAW) return raw.start + w0 + r;
    else return sm.idx[min(r, kIdxCap - 1)];
  }

  // Copy chunk c of the window into buffers kdst / vdst, memory -> LDS.  Wave
  // w fills 16-byte slots [w KPT 64, (w + 1) KPT 64) of K (and likewise of V):
  // slot s is row s / KP, stored piece s % KP, which holds logical piece
  // (s % KP) ^ kswz(row).  Rows beyond the window copy the unit's first row;
  // zero_tail() clears them.  The tokens of a lane's rows are read from LDS
  // first, all at once: read between copies, each would wait for its own LDS
  // round trip (a copy into LDS may, for the compiler, overwrite sm.idx).
  __device__ __forceinline__ int chunk_token(int r) const {
    const int t = token(r);   // in bounds for any r; the value is discarded past the window
    return r < wl ? t : 0;
  }
  __device__ __forceinline__ void copy(int c, lds_byte* kdst, lds_byte* vdst) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    typedef __attribute__((address_space(1))) const void* gptr;
    typedef __attribute__((address_space(3))) void* lptr;
    constexpr bool kSameRows = !FP8 && VP == KP && VPT == KPT;   // V slot s is on K slot s's row
    constexpr int VT = FP8 ? VGPT : VPT;
    constexpr int VRP = FP8 ? VGP : VP;                          // V pieces per row, as copied
    int ktok[KPT], vtok[kSameRows ? 1 : VT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) ktok[i] = chunk_token(kC * c + ((w * KPT + i) * 64 + lane) / KP);
    if constexpr (!kSameRows) {
#pragma unroll
      for (int i = 0; i < VT; ++i) vtok[i] = chunk_token(kC * c + ((w * VT + i) * 64 + lane) / VRP);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int s = (w * KPT + i) * 64 + lane;
      const int R = s / KP, P = s % KP;
      const uint32_t off = __umul24(static_cast<uint32_t>(ktok[i]), kstride) + static_cast<uint32_t>(16 * (P ^ kswz<KB>(R)));
      __builtin_amdgcn_global_load_lds((gptr)(kbase + off), (lptr)(kdst + (w * KPT + i) * 1024), 16, 0, 0);
    }
    if constexpr (FP8) {   // V through registers: widened to bf16 by store_v once they land
#pragma unroll
      for (int i = 0; i < VGPT; ++i) {
        const int s = (w * VGPT + i) * 64 + lane;
        const int P = s % VGP;
        const uint32_t off = __umul24(static_cast<uint32_t>(vtok[i]), vstride) + static_cast<uint32_t>(16 * P);
        vreg[i] = *reinterpret_cast<const uint4*>(vbase + off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int s = (w * VPT + i) * 64 + lane;
        const int R = s / VP, P = s % VP;
        const int t = kSameRows ? ktok[i] : vtok[kSameRows ? 0 : i];
        const uint32_t off = __umul24(static_cast<uint32_t>(t), vstride) +
                             static_cast<uint32_t>(16 * (P ^ vswz<BF16, VB>(R)));
        __builtin_amdgcn_global_load_lds((gptr)(vbase + off), (lptr)(vdst + (w * VPT + i) * 1024), 16, 0, 0);
      }
    }
  }

  // fp8: the V pieces copy() loaded (16 values each, landed) as bf16 into buffer vdst:
  // piece P of row R holds dimensions 16 P .. 16 P + 15, the staged row's pieces 2 P
  // and 2 P + 1, stored at (2 P) ^ vswz(R) (even, so the two stay adjacent)
  __device__ __forceinline__ void store_v(lds_byte* vdst) {
    if constexpr (FP8) {
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      typedef __attribute__((address_space(3))) u32x4v_t lds_u4;
#pragma unroll
      for (int i = 0; i < VGPT; ++i) {
        const int s = (w * VGPT + i) * 64 + lane;
        const int R = s / VGP, P = s % VGP;
        const uint32_t wv[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wv[j]), false);
          const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wv[j]), true);
          o[2 * j] = (__float_as_uint(f01[1]) & 0xffff0000u) | (__float_as_uint(f01[0]) >> 16);
          o[2 * j + 1] = (__float_as_uint(f23[1]) & 0xffff0000u) | (__float_as_uint(f23[0]) >> 16);
        }
        lds_byte* row = vdst + R * VB + 16 * ((2 * P) ^ vswz<true, VB>(R));
        *reinterpret_cast<lds_u4*>(row) = u32x4v_t{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<lds_u4*>(row + 16) = u32x4v_t{o[4], o[5], o[6], o[7]};
      }
    }
  }

  // Weighted coreset: entry weight of the key thread tid describes in chunk c.
  __device__ __forceinline__ float entry_weight(int c) const {
    return gs.w[min(w0 + kC * c + static_cast<int>(threadIdx.x), G - 1)];
  }

  // Per-key visibility and log2-weight of chunk c into buffer buf (threads < kC).
  // A weighted coreset's entry weight is loaded and used here; callers take
  // meta before the chunk's copy, so that waiting for that load never waits
  // for the copy (memory loads complete in order for the wait counter).
  // Nothing of it is carried from chunk to chunk: a value loaded one chunk
  // ahead and kept in a register made the compiler wait for every load in
  // flight, the next chunk's copy included, before the chunk's reads.
  __device__ __forceinline__ void meta(int c, int nch, int buf) {
    (void)nch;
    const int tid = threadIdx.x;
    if (tid < kC) {
      const int r = kC * c + tid;
      const int pos = w0 + r;   // position in the stream
      float lg = gs.lnw2 - (pos < gs.cnt[0] + gs.cnt[1] ? 0.f : 1.f);
      if constexpr (!RAW) {
        if (gs.w != nullptr) lg = log2f(entry_weight(c));
      }
      float lw = pos < G ? lg : raw.lnw2;
      lw = r < wl ? lw : -INFINITY;
      sm.lnw2[buf][tid] = lw;
    }
  }

  // Rows of chunk c beyond the window are zeroed (after its copy has landed).
  __device__ __forceinline__ void zero_tail(int c, int buf) {
    const int first = wl - kC * c;   // rows [first, kC) are padding
    for (int e = threadIdx.x; e < (kC - first) * KP; e += kThreads)
      reinterpret_cast<uint4*>(&sm.k[buf][first * KB])[e] = uint4{0, 0, 0, 0};
    for (int e = threadIdx.x; e < (kC - first) * VP; e += kThreads)
      reinterpret_cast<uint4*>(&sm.v[buf][first * VB])[e] = uint4{0, 0, 0, 0};
  }

  // S^T (keys x queries) of the chunk in buffer kbuf: st[qg][kb] holds keys
  // 16 kb + 4 g + i (i = 0..3) for query lane % 16.  bf16 and fp8: the K
  // fragments of key block kb + 1 are read before the MFMAs of block kb (two
  // register sets), and scheduling barriers keep the compiler from sinking
  // the reads next to their use, so an LDS round trip overlaps a block of
  // MFMAs instead of stalling between them.
  template <int NF>
  struct KFrag {
    typename std::conditional<FP8, i32x8_t, bf16x8_t>::type f[NF];
  };
  __device__ __forceinline__ void kread(const lds_byte* kbuf, int kb, KFrag<NQF>& kf) const {
    const int R = 16 * kb + (lane & 15);
    if constexpr (FP8) {
      // lane group g: features 32 g .. 32 g + 31 of each 128, logical pieces 2 g and 2 g + 1
      typedef __attribute__((address_space(3))) const u32x4v_t lds_u4;
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk) {
        const u32x4v_t lo = *reinterpret_cast<lds_u4*>(kbuf + R * KB + 16 * ((8 * kk + 2 * g) ^ kswz<KB>(R)));
        const u32x4v_t hi = *reinterpret_cast<lds_u4*>(kbuf + R * KB + 16 * ((8 * kk + 2 * g + 1) ^ kswz<KB>(R)));
        kf.f[kk] = i32x8_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                           static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                           static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      }
    } else {
      typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
#pragma unroll
      for (int kk = 0; kk < NQF; ++kk)
        kf.f[kk] = *reinterpret_cast<lds_bf16x8*>(kbuf + R * KB + 16 * ((4 * kk + g) ^ kswz<KB>(R)));
    }
  }
  __device__ __forceinline__ void kmfma(const KFrag<NQF>& kf, f32x4_t (&acc)[NQG]) const {
#pragma unroll
    for (int kk = 0; kk < NQF; ++kk)
#pragma unroll
      for (int qg = 0; qg < NQG; ++qg) {
        if constexpr (FP8)   // E4M3 operands (format 0), unit block scales (E8M0 127)
          acc[qg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf.f[kk], qf[qg][kk], acc[qg], 0, 0, 0, 127, 0,
                                                                    127);
        else
          acc[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.f[kk], qf[qg][kk], acc[qg], 0, 0, 0);
      }
  }

  __device__ __forceinline__ void scores(const lds_byte* kbuf, f32x4_t st[NQG][4]) const {
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) st[qg][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
      KFrag<NQF> kf[2];
      kread(kbuf, 0, kf[0]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb + 1 < 4) kread(kbuf, kb + 1, kf[(kb + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t acc[NQG];
#pragma unroll
        for (int qg = 0; qg < NQG; ++qg) acc[qg] = st[qg][kb];
        kmfma(kf[kb & 1], acc);
#pragma unroll
        for (int qg = 0; qg < NQG; ++qg) st[qg][kb] = acc[qg];
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const int R0 = lane & 15;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int R = 16 * kb + R0;
        typedef __attribute__((address_space(3))) const f32x4_t lds_f4;
#pragma unroll
        for (int kq = 0; kq < E / 16; ++kq) {
          const f32x4_t kf = *reinterpret_cast<lds_f4*>(kbuf + R * KB + 16 * ((4 * kq + g) ^ kswz<KB>(R)));
          const float kv[4] = {kf[0], kf[1], kf[2], kf[3]};
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int qg = 0; qg < NQG; ++qg)
              st[qg][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[t], qf[qg][4 * kq + t], st[qg][kb], 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void consume(int c, int buf, const lds_byte* kbuf, const lds_byte* vbuf) {
    f32x4_t st[NQG][4];
    scores(kbuf, st);
    // padding keys carry log-weight -inf; only causal keys and queries outside
    // the stream's block need the visibility test
    const bool masked = !rows_ok || (raw.causal && w0 + kC * (c + 1) > G);
    const float sc = a.scale * kLog2e;
    float lw[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 lv = *reinterpret_cast<const float4*>(&sm.lnw2[buf][kb * 16 + 4 * g]);
      lw[kb][0] = lv.x, lw[kb][1] = lv.y, lw[kb][2] = lv.z, lw[kb][3] = lv.w;
    }
    // online softmax; p[qg][kb][i] is the weight of key 16 kb + 4 g + i
    float p[NQG][4][4];
    if (masked) {   // two copies of the logit loop, so the common one carries no test
#pragma unroll
      for (int qg = 0; qg < NQG; ++qg) {
        const int t = vlim[qg] - (w0 + kC * c) - 4 * g;   // key 16 kb + 4 g + i visible iff 16 kb + i <= t
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[qg][kb][i] = 16 * kb + i <= t ? fmaf(st[qg][kb][i], sc, lw[kb][i]) : -INFINITY;
      }
    } else {
#pragma unroll
      for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[qg][kb][i] = fmaf(st[qg][kb][i], sc, lw[kb][i]);
    }
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, p[qg][kb][i]);
      mx = group_max(mx);
      const float m_new = fmaxf(m_run[qg], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qg] - m_use);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[qg][kb][i] = __builtin_amdgcn_exp2f(p[qg][kb][i] - m_use);
      if constexpr (!BF16) {   // bf16: the row sum comes out of the P V MFMAs (a block of ones)
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) rs += p[qg][kb][i];
        rs = group_sum(rs);
        l_run[qg] = l_run[qg] * alpha + rs;
      }
      m_run[qg] = m_new;
      if (__ballot(alpha != 1.0f)) {   // most chunks leave every maximum where it was
#pragma unroll
        for (int d = 0; d < ND; ++d) o[qg][d] *= alpha;
        if constexpr (BF16) osum[qg] *= alpha;
      }
    }
    if constexpr (BF16) {
      bf16x8_t pb[NQG][2];
#pragma unroll
      for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pb[qg][hh][i] = static_cast<__bf16>(p[qg][2 * hh][i]);
            pb[qg][hh][4 + i] = static_cast<__bf16>(p[qg][2 * hh + 1][i]);
          }
      // O^T += V^T P^T: lane group g's operand slots 0-3 / 4-7 are keys
      // 32hh + 4g + (0..3) and 32hh + 16 + 4g + (0..3) (the S^T layout).  The
      // fragments of dimension block d + 1 are read before the MFMAs of block
      // d (two register sets, scheduling barriers as in scores()).
      const int i16 = lane & 15;
      typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
      auto vread = [&](int d, bf16x8_t (&vf)[2]) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // logical elements 16 d + 4 (i16 % 4) .. + 3: piece 2 d + (i16 % 4) / 2, half i16 % 2
          const int q = 2 * d + ((i16 & 3) >> 1);
          const int R0 = 32 * hh + 4 * g + (i16 >> 2), R1 = R0 + 16;
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(vbuf + R0 * VB + 16 * (q ^ vswz<BF16, VB>(R0)) + 8 * (i16 & 1)));
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(vbuf + R1 * VB + 16 * (q ^ vswz<BF16, VB>(R1)) + 8 * (i16 & 1)));
          vf[hh] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      bf16x8_t vf[2][2];
      vread(0, vf[0]);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        if (d + 1 < ND) vread(d + 1, vf[(d + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int qg = 0; qg < NQG; ++qg)
            o[qg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d & 1][hh], pb[qg][hh], o[qg][d], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // a 16-row block of ones: every row of its output is the query's sum of P
      const bf16x8_t ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                             (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int qg = 0; qg < NQG; ++qg)
          osum[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qg][hh], osum[qg], 0, 0, 0);
    } else {
      // O^T += V^T P^T, four keys per MFMA: key 16 kb + 4 g + i is lane group
      // g's k-index in step (kb, i); one 16-byte read gives dimensions
      // 64 j + 4 (lane % 16) .. + 3 of that key for output blocks 4 j .. 4 j + 3
      typedef __attribute__((address_space(3))) const f32x4_t lds_f4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * kb + 4 * g + i;
#pragma unroll
          for (int j = 0; j < D / 64; ++j) {
            const f32x4_t vv = *reinterpret_cast<lds_f4*>(vbuf + key * VB + 16 * (16 * j + (lane & 15)));
            const float vx[4] = {vv[0], vv[1], vv[2], vv[3]};
#pragma unroll
            for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
              for (int qg = 0; qg < NQG; ++qg)
                o[qg][4 * j + d4] = __builtin_amdgcn_mfma_f32_16x16x4f32(vx[d4], p[qg][kb][i], o[qg][4 * j + d4], 0, 0, 0);
          }
        }
    }
  }

  // One window: its tokens are staged (all loads in flight at once), then
  // its chunks stream through the two buffers.
  __device__ __forceinline__ void run_window() {
    __syncthreads();   // earlier users of sm.idx and of the buffers are done
    if constexpr (!RAW) {
      const int c0 = gs.cnt[0], c01 = gs.cnt[0] + gs.cnt[1];
      int v[kIdxPT];
#pragma unroll
      for (int i = 0; i < kIdxPT; ++i) {
        const int pos = w0 + min(static_cast<int>(threadIdx.x) + kThreads * i, wl - 1);
        const int gp = min(pos, G - 1);   // in bounds of the gathered lists whenever it is read
        const int32_t* src = gp < c0 ? gs.p[0] + gp : (gp < c01 ? gs.p[1] + (gp - c0) : gs.p[2] + (gp - c01));
        v[i] = pos < G ? *src : raw.start + (pos - G);
      }
      // a gathered index outside the unit's rows is clamped (and reported): no
      // read may leave [0, S)
      bool bad = false;
#pragma unroll
      for (int i = 0; i < kIdxPT; ++i) {
        const int e = threadIdx.x + kThreads * i;
        bad = bad || (e < wl && static_cast<unsigned>(v[i]) >= static_cast<unsigned>(a.S));
        v[i] = min(max(v[i], 0), a.S - 1);
        if (e < wl) sm.idx[e] = v[i];
      }
      if (bad && a.err) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __syncthreads();
    }
    const int nch = (wl + kC - 1) / kC;
    meta(0, nch, 0);
    copy(0, (lds_byte*)&sm.k[0][0], (lds_byte*)&sm.v[0][0]);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    store_v((lds_byte*)&sm.v[0][0]);
    if (kC > wl) {
      __syncthreads();
      zero_tail(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {   // unrolled by two: the buffer of each step is a constant
      step<0>(c, nch);
      if constexpr (NB == 2) {
        if (c + 1 < nch) step<1>(c + 1, nch);
      }
    }
  }

  // chunk c sits in buffer B; chunk c + 1 is copied into the other buffer meanwhile
  template <int B>
  __device__ __forceinline__ void step(int c, int nch) {
    constexpr int NX = NB == 2 ? 1 - B : B;   // (NB = 1: there is no next chunk)
    overlap(c, nch, (const lds_byte*)&sm.k[B][0], (const lds_byte*)&sm.v[B][0], (lds_byte*)&sm.k[NX][0],
            (lds_byte*)&sm.v[NX][0]);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);   // this thread's copies have landed
    if (c + 1 < nch) store_v((lds_byte*)&sm.v[NX][0]);
    if (c + 1 < nch && kC * (c + 2) > wl) {
      __syncthreads();
      zero_tail(c + 1, NX);
    }
    __syncthreads();
  }

  // The copy into one buffer overlaps the MFMA reads of the other.  The
  // restrict-qualified views tell the compiler so: without them it would wait
  // for the copy before the first LDS read of the current buffer.
  __device__ __forceinline__ void overlap(int c, int nch, const lds_byte* __restrict__ kc,
                                          const lds_byte* __restrict__ vc, lds_byte* __restrict__ kn,
                                          lds_byte* __restrict__ vn) {
    if (c + 1 < nch) {
      meta(c + 1, nch, (c + 1) & 1);
      copy(c + 1, kn, vn);
    }
    consume(c, c & 1, kc, vc);
  }

  // The whole stream, in windows of at most kIdxCap staged tokens.
  __device__ __forceinline__ void run_stream(const Gather& gather, const Raw& r, const bool row_ok[NQG]) {
    gs = gather;
    raw = r;
    G = gs.cnt[0] + gs.cnt[1] + gs.cnt[2];
    bool all = true;
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      vlim[qg] = row_ok[qg] ? (raw.causal ? qr[qg] - raw.start + G : INT_MAX) : -1;
      all = all && row_ok[qg];
    }
    rows_ok = __ballot(!all) == 0;
    const int L = G + raw.count;
    const int cap = RAW ? L : kIdxCap;
    for (w0 = 0; w0 < L; w0 += cap) {
      wl = min(cap, L - w0);
      run_window();
    }
  }

  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      if (!live[qg]) continue;
      const float l = BF16 ? osum[qg][0] : l_run[qg];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int64_t orow = ((static_cast<int64_t>(b) * a.T + qr[qg]) * a.H + h) * D;
      if constexpr (BF16) {
        // block d, accumulator element i: dimension 16 d + 4 g + i
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          uint16_t* dst = static_cast<uint16_t*>(a.out) + orow + 16 * d + 4 * g;
          const uint32_t lo = float_to_bf16_bits(o[qg][d][0] * inv) |
                              (static_cast<uint32_t>(float_to_bf16_bits(o[qg][d][1] * inv)) << 16);
          const uint32_t hi = float_to_bf16_bits(o[qg][d][2] * inv) |
                              (static_cast<uint32_t>(float_to_bf16_bits(o[qg][d][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
        }
      } else {
        // block 4 j + d4, accumulator element i (row 4 g + i): dimension 64 j + 4 (4 g + i) + d4
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dst = static_cast<float*>(a.out) + orow + 64 * j + 16 * g + 4 * i;
            *reinterpret_cast<float4*>(dst) = float4{o[qg][4 * j][i] * inv, o[qg][4 * j + 1][i] * inv,
                                                     o[qg][4 * j + 2][i] * inv, o[qg][4 * j + 3][i] * inv};
          }
      }
    }
  }
};

// Stream of the queries of block beta (tokens [beta n, (beta + 1) n)) among
// the workgroup's: the Express state after blocks 0 .. beta-1, then the block
// itself up to key_end with the causal mask:
//   beta < 4: everything before is still exact (raw, weight 1);
//   else, with E = floor(log4 beta), m = 4^E, since = beta - m:
//     cache   = HALVE output E-1 and batches 3(E-1) .. 3(E-1) + since/m - 1 (weight m),
//     buffer  = the first (since % m) 2n / m representatives of batch 3(E-1) + since/m
//               (weight m/2),
//   each weight as log2 added to the logit.
__device__ __forceinline__ void express_pass(const ExpressView& ev, int unit, int beta, int S, int key_end,
                                             Gather& gs, Raw& raw) {
  gs = Gather{{nullptr, nullptr, nullptr}, {0, 0, 0}, 0.f, nullptr};
  if (beta < 4) {
    raw = Raw{0, min(key_end, S), 0.f, 1};
    return;
  }
  int Ep = 1;
  while ((1LL << (2 * (Ep + 1))) <= beta) ++Ep;
  const int m = 1 << (2 * Ep);
  const int since = beta - m;
  const int nbc = since / m;
  const int rem = since % m;
  gs.lnw2 = static_cast<float>(2 * Ep);
  gs.p[0] = ev.halve_out + (static_cast<int64_t>(unit) * ev.n_halves + (Ep - 1)) * ev.n;
  gs.cnt[0] = ev.n;
  gs.p[1] = ev.batch_out + (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (Ep - 1)) * ev.n;
  gs.cnt[1] = nbc * ev.n;
  gs.p[2] = ev.reps + (static_cast<int64_t>(unit) * ev.n_batches_alloc + 3 * (Ep - 1) + nbc) * 2 * ev.n;
  gs.cnt[2] = static_cast<int>((static_cast<int64_t>(rem) * 2 * ev.n) / m);
  const int bn = beta * ev.n;
  raw = Raw{bn, min(key_end, S) - bn, 0.f, 1};
}

// Unmasked: one pass (the coreset, or all S keys).  Causal: one pass per
// block beta met by the workgroup's queries.
// Waves per SIMD the register budget is set for: three for the one-buffer
// bf16 build with E = D = 64 (168 registers, 5 spilled); two elsewhere (the
// one-buffer D = 256 build spills 41 registers at three and runs faster at two
// with none).
// Query tiles per workgroup: a one-chunk coreset is staged once and serves
// kTilesOne consecutive tiles of its unit.
constexpr int kTilesOne = 4;

template <int ET, int E, int D, int NB>
constexpr int attn_waves() { return (NB == 1 && ET == kBF16 && E == 64 && D == 64) ? 3 : 2; }

template <int ET, int E, int D, bool RAW, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(attn_waves<ET, E, D, NB>()))) void attn_kernel(
    AttnLaunch a) {
  constexpr int kQ = 16 * nqg<ET, E, D>() * kWaves;
  constexpr int NQG = Attn<ET, E, D, RAW, NB>::NQG;
  __shared__ Smem<ET, E, D, NB> sm;
  const int64_t tile = xcd_remap(blockIdx.y * static_cast<int64_t>(gridDim.x) + blockIdx.x,
                                 static_cast<int64_t>(gridDim.x) * gridDim.y);
  // causal: a head's query tiles in reverse, so that the later blocks, whose
  // states hold more keys, start first and the last workgroups are short
  const int qt = static_cast<int>(tile % gridDim.x);
  const int q0 = a.t0 + (a.causal ? static_cast<int>(gridDim.x) - 1 - qt : qt) * kQ * (NB == 1 ? kTilesOne : 1);
  Attn<ET, E, D, RAW, NB> at(a, sm, q0, static_cast<int>(tile / gridDim.x));
  if constexpr (NB == 1) at.fetch_q(q0 + kQ, at.qn);
  const int q_last = min(q0 + kQ - 1, a.t1 - 1);
  const int n = a.causal ? a.ev.n : 1;
  const int beta_lo = a.causal ? q0 / n : 0, beta_hi = a.causal ? q_last / n : 0;
  for (int beta = beta_lo; beta <= beta_hi; ++beta) {
    Gather gs;
    Raw raw;
    bool row_ok[NQG];
    if (!a.causal) {
      gs = Gather{{nullptr, nullptr, nullptr}, {0, 0, 0}, a.cs_lnw * kLog2e, nullptr};
      raw = Raw{0, 0, 0.f, 0};
      if (a.cs_idx) {
        gs.p[0] = a.cs_idx + at.unit * a.cs_stride;
        gs.cnt[0] = a.cs_n;
        gs.w = a.cs_w ? a.cs_w + at.unit * a.cs_stride : nullptr;
      } else {
        raw = Raw{0, a.S, a.cs_lnw * kLog2e, 0};
      }
      for (int qg = 0; qg < NQG; ++qg) row_ok[qg] = true;
    } else {
      express_pass(a.ev, at.unit, beta, a.S, min(q_last + 1, (beta + 1) * n), gs, raw);
      for (int qg = 0; qg < NQG; ++qg) row_ok[qg] = (at.qr[qg] / n) == beta;
    }
    at.run_stream(gs, raw, row_ok);
  }
  at.finish();
  if constexpr (NB == 1) {   // unmasked, one chunk: the next tiles reuse the staged keys
    for (int t = 1; t < kTilesOne && q0 + t * kQ < a.t1; ++t) {
      at.rerun_single(q0 + t * kQ, t + 1 < kTilesOne ? q0 + (t + 1) * kQ : a.t1);
      at.finish();
    }
  }
}

template <int ET, int E, int D>
hipError_t launch(const AttnLaunch& a, hipStream_t s) {
  constexpr int kQ = 16 * nqg<ET, E, D>() * kWaves;
  const int rows = a.t1 - a.t0;
  dim3 grid((rows + kQ - 1) / kQ, a.B * a.H);
  if (!a.causal && a.cs_idx == nullptr)   // exact attention: one raw range, nothing staged
    hipLaunchKernelGGL((attn_kernel<ET, E, D, true, 2>), grid, dim3(kThreads), 0, s, a);
  else if (!a.causal && a.cs_n <= kC)     // a coreset of one chunk: one buffer, kTilesOne tiles per workgroup
    hipLaunchKernelGGL((attn_kernel<ET, E, D, false, 1>), dim3((rows + kQ * kTilesOne - 1) / (kQ * kTilesOne), a.B * a.H),
                       dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<ET, E, D, false, 2>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int dtype, int E, int D) {
  if (dtype == kFP8) return E == 128 && D == 128;
  if (dtype == kBF16) return (E == 64 && (D == 64 || D == 128 || D == 256)) || (E == 128 && (D == 128 || D == 64));
  return (E == 64 && (D == 64 || D == 128)) || (E == 128 && D == 128);
}

hipError_t launch_attention(const AttnLaunch& la, int dtype, int E, int D, hipStream_t s) {
  AttnLaunch a = la;
  if (a.t1 <= 0) a.t1 = a.T;
  a.t0 = a.t0 < 0 ? 0 : a.t0;
  a.t1 = a.t1 > a.T ? a.T : a.t1;
  if (a.t1 <= a.t0 || a.B * a.H == 0) return hipSuccess;
  if (dtype == kFP8) {
    if (E == 128 && D == 128) return launch<kFP8, 128, 128>(a, s);
  } else if (dtype == kBF16) {
    if (E == 64 && D == 64) return launch<kBF16, 64, 64>(a, s);
    if (E == 64 && D == 128) return launch<kBF16, 64, 128>(a, s);
    if (E == 64 && D == 256) return launch<kBF16, 64, 256>(a, s);
    if (E == 128 && D == 128) return launch<kBF16, 128, 128>(a, s);
    if (E == 128 && D == 64) return launch<kBF16, 128, 64>(a, s);
  } else {
    if (E == 64 && D == 64) return launch<kF32, 64, 64>(a, s);
    if (E == 64 && D == 128) return launch<kF32, 64, 128>(a, s);
    if (E == 128 && D == 128) return launch<kF32, 128, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace thin
