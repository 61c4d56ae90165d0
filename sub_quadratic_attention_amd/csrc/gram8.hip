// Exact integer pair Gram on the gfx950 int8 MFMA, for bf16 and fp8 rows.
//
// The walk of kernel halving (kernel-thinning papers; "Express Language
// Modeling", "Thinformer Express") must decide like a float64 reference, so
// the dot products behind kappa((k, v), (k', v')) = exp(s <k, k'>) (<v, v'> + 1)
// need fp64 accuracy.  They get it here from integer arithmetic:
//
//  * every bf16 or fp8 feature is x = sig 2^p with an integer significand
//    (sig < 2^8 for bf16, < 2^4 for fp8).  A row scaled by 2^s with
//    s = C - p_max (p_max the largest p among its nonzero features; C = 22 for
//    bf16, 18 for fp8) holds integers X = x 2^s, |X| < 2^30 (bf16) or 2^22
//    (fp8), exactly so when every feature has p + s + ctz(sig) >= 0.  A bf16
//    row "fits" when its features span at most 22 binades below its largest
//    (about 1e-4 of the rows of the synthetic workloads miss); fp8 rows always
//    fit (E4M3 spans 14 binades);
//  * X is written as ND balanced base-256 digits, X = sum_a 256^a d_a with
//    d_a in [-128, 127] (ND = 4 for bf16, 3 for fp8), so that
//      <x, y> 2^(s_x + s_y) = sum_{a,b} 256^(a+b) sum_f d_a(x_f) d_b(y_f);
//    each inner sum is exact on v_mfma_i32_16x16x64_i8 (|d_a d_b| <= 2^14, at
//    most 2^22 over 256 features), and the products of equal a + b share an
//    accumulator (at most 2^24);
//  * the 2 ND - 1 accumulators are joined in fp64 as two integers below 2^53
//    (exact) and one final fma: the exact dot product rounded once, which is
//    at least as accurate as fp64 accumulation;
//  * the pairs of a row that does not fit are left to fp64: their Gram rows
//    (and columns) are recomputed by fp64 FMAs from the raw features.
//
// Everything after the dot products (fp64 exp, the pair combination, the
// thresholds in the lower triangle, the output layout) is the fp64 tiles'.
//
// Two launches: a digit pass (one lane group per point row of the launch:
// scales, digits, fit flags) and the Gram launch (threshold workgroups, kFixGroups
// workgroups for the pairs that do not fit, then the tiles).

#include <limits.h>
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "khdev.hpp"

namespace thin {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

template <int ET>
constexpr int nd() { return ET == kFP8 ? 3 : 4; }        // digits per feature
template <int ET>
constexpr int top_shift() { return ET == kFP8 ? 18 : 22; }   // C: |X| < 2^C sig

constexpr int kSlots = 128;      // row and column points of a tile
constexpr int kSlotBytes = 256;  // one point's digits of one 64-feature step (ND 64 bytes, padded)
constexpr int kFixGroups = 16;   // workgroups recomputing the pairs whose rows do not fit

// Scratch of a launch with npts points:
//   digits [npts][ND (E + D)]: a point's K digits, then its V digits; inside a
//          part, step m (features 64 m .. 64 m + 63) holds ND runs of 64 bytes,
//          digit d of feature 64 m + f at byte 64 (ND m + d) + f;
//   scales [npts][2] int32 (s_K, s_V);
//   flags  [npts][2] uint8: 1 when the point's K (V) row does not fit.
struct Scratch8 {
  unsigned char* dig;
  int32_t* scale;
  uint8_t* flag;
  int64_t pbytes;   // digit bytes per point
};

__host__ __device__ inline int64_t digit_bytes(int nd_, int E, int D) { return static_cast<int64_t>(nd_) * (E + D); }

__host__ __device__ inline Scratch8 scratch8(unsigned char* base, int nd_, int E, int D, int64_t npts) {
  Scratch8 s;
  s.pbytes = digit_bytes(nd_, E, D);
  s.dig = base;
  const int64_t off_scale = (npts * s.pbytes + 255) / 256 * 256;
  s.scale = reinterpret_cast<int32_t*>(base + off_scale);
  s.flag = reinterpret_cast<uint8_t*>(base + off_scale + npts * 8);
  return s;
}

// Points of the digit scratch, and the scratch row of point pt of the launch
// (another launch's point when its digit pass serves this one).
__host__ __device__ inline int64_t dig_points(const GramLaunch& a) {
  return a.dig_npts ? a.dig_npts : static_cast<int64_t>(a.nbins) * a.N;
}
__device__ __forceinline__ int64_t drow(const GramLaunch& a, int64_t pt) {
  return a.dig_map ? a.dig_map[pt] : a.dig_row0 + pt;
}

// Fit flags of pair c of the launch (points 2c, 2c + 1; K and V): nonzero when
// any of the four rows does not fit.
__device__ __forceinline__ uint32_t pair_flags(const GramLaunch& a, const uint8_t* flag, int64_t c) {
  const uint16_t* f2 = reinterpret_cast<const uint16_t*>(flag);
  return static_cast<uint32_t>(f2[drow(a, 2 * c)]) | static_cast<uint32_t>(f2[drow(a, 2 * c + 1)]);
}

// Token of point q of bin z, clamped into [0, S) (an index outside is reported).
__device__ __forceinline__ int64_t point_row(const GramLaunch& a, int z, int q) {
  const int unit = z / a.bins_per_unit, lb = z % a.bins_per_unit;
  const int b = unit / a.src.H_kv, h = unit % a.src.H_kv;
  int tok = a.idx[static_cast<int64_t>(unit) * a.idx_unit_stride + static_cast<int64_t>(lb) * a.idx_stride + q];
  if (static_cast<uint32_t>(tok) >= static_cast<uint32_t>(a.src.S)) {
    if (a.err) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    tok = tok < 0 ? 0 : static_cast<int>(a.src.S - 1);
  }
  return (static_cast<int64_t>(b) * a.src.S + tok) * a.src.H_kv + h;
}

// ---------------------------------------------------------------------------
// Digit pass.  Items are point rows of one part (all K rows, then all V
// rows); a row of F features takes F / 16 consecutive lanes (an aligned group
// of a wave), each with 16 consecutive features: one or two 16-byte loads, a
// group maximum of the exponents, and one 16-byte store per digit.
// ---------------------------------------------------------------------------
template <int ET>
__global__ __launch_bounds__(256) void gram8_digits_kernel(GramLaunch a, int blocks_k) {
  constexpr int ND = nd<ET>();
  const int64_t npts = static_cast<int64_t>(a.nbins) * a.N;
  const int part = static_cast<int>(blockIdx.x) >= blocks_k ? 1 : 0;
  const int F = part ? a.src.D : a.src.E;
  const int gl = F / 16;   // lanes per row (16 features each): 4, 8 or 16, a power of two dividing 256
  const int64_t t = (static_cast<int64_t>(blockIdx.x) - (part ? blocks_k : 0)) * 256 + threadIdx.x;
  const int64_t pt = t / gl;
  const int j = static_cast<int>(t % gl);
  if (pt >= npts) return;   // whole groups (gl divides 256)
  const Scratch8 sc = scratch8(a.dig, ND, a.src.E, a.src.D, dig_points(a));
  const int64_t row = point_row(a, static_cast<int>(pt / a.N), static_cast<int>(pt % a.N));
  const unsigned char* src = static_cast<const unsigned char*>(part ? a.src.v : a.src.k) +
                             (row * F + 16 * j) * elt_size<ET>();
  uint32_t w[8];
  {
    const uint4 x = *reinterpret_cast<const uint4*>(src);
    w[0] = x.x, w[1] = x.y, w[2] = x.z, w[3] = x.w;
  }
  if constexpr (ET != kFP8) {
    const uint4 x = *reinterpret_cast<const uint4*>(src + 16);
    w[4] = x.x, w[5] = x.y, w[6] = x.z, w[7] = x.w;
  }
  int sgn[16], sig[16], p[16];
  int pmax = INT_MIN;
  bool ok = true;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    if constexpr (ET == kFP8) {
      const uint32_t b = (w[u >> 2] >> (8 * (u & 3))) & 255u;
      const uint32_t e4 = (b >> 3) & 15u, m3 = b & 7u;
      sgn[u] = static_cast<int>(b >> 7);
      sig[u] = e4 ? static_cast<int>(8u + m3) : static_cast<int>(m3);
      p[u] = e4 ? static_cast<int>(e4) - 10 : -9;
      if ((b & 0x7fu) == 0x7fu) ok = false, sig[u] = 0;   // NaN
    } else {
      const uint32_t h = (w[u >> 1] >> (16 * (u & 1))) & 0xffffu;
      const uint32_t e8 = (h >> 7) & 255u, m7 = h & 127u;
      sgn[u] = static_cast<int>(h >> 15);
      sig[u] = e8 ? static_cast<int>(128u + m7) : static_cast<int>(m7);
      p[u] = e8 ? static_cast<int>(e8) - 134 : -133;
      if (e8 == 255u) ok = false, sig[u] = 0;   // infinity or NaN
    }
    if (sig[u]) pmax = max(pmax, p[u]);
  }
  for (int off = gl / 2; off >= 1; off >>= 1) pmax = max(pmax, __shfl_xor(pmax, off, 64));
  const int s = pmax == INT_MIN ? 0 : top_shift<ET>() - pmax;
  uint32_t dg[ND][4] = {};
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = p[u] + s;
    if (sig[u] && e + __builtin_ctz(static_cast<unsigned>(sig[u])) < 0) ok = false;
    int X = e >= 0 ? (sig[u] << e) : (e > -31 ? (sig[u] >> -e) : 0);
    X = sgn[u] ? -X : X;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int lo = d < ND - 1 ? static_cast<int>(static_cast<signed char>(X & 255)) : X;
      dg[d][u >> 2] |= (static_cast<uint32_t>(lo) & 255u) << (8 * (u & 3));
      X = (X - lo) >> 8;
    }
  }
  const int f0 = 16 * j;
  const int64_t dr = a.dig_row0 + pt;   // this point's scratch row
  unsigned char* o = sc.dig + dr * sc.pbytes + (part ? ND * a.src.E : 0) + 64 * ND * (f0 / 64) + (f0 % 64);
#pragma unroll
  for (int d = 0; d < ND; ++d) *reinterpret_cast<uint4*>(o + 64 * d) = uint4{dg[d][0], dg[d][1], dg[d][2], dg[d][3]};
  // the row fits when every lane of its group fits
  int bad = ok ? 0 : 1;
  for (int off = gl / 2; off >= 1; off >>= 1) bad |= __shfl_xor(bad, off, 64);
  if (j == 0) {
    sc.scale[2 * dr + part] = s;
    sc.flag[2 * dr + part] = static_cast<uint8_t>(bad);
  }
}

// ---------------------------------------------------------------------------
// Tiles.  The fp64 tiles' decomposition: a workgroup takes a 32 x 32 tile of
// pairs (64 row points, 64 column points) of the bin's upper triangle; wave
// (wr, wc) owns pair rows 16 wr .. and pair columns 16 wc .. of the tile.  Its
// MFMA blocks: row block rb (points 32 wr + 16 rb + i) against column block
// cb (the points of parity cb of its 16 column pairs), so the accumulator
// element t of lane l is row point 4 (l / 16) + t against column pair l % 16:
// the four point products of a pair pair are in one lane.  Both operands read
// 16 bytes of a slot: lane group g takes bytes 16 g .. 16 g + 15 of a digit's
// 64 (the MFMA reduces over whatever k-order its A and B operands share).
//
// LDS: two buffers of 128 slots x 256 bytes (one 64-feature step of every
// point, copied straight from memory with global_load_lds); the 16-byte piece
// j of slot s is stored at j ^ dswz(s), which puts the 16 slots an operand
// read touches (consecutive, or every other one) on distinct banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dswz(int s) { return (s ^ (s >> 4)) & 15; }

template <int ET>
struct Tile8 {
  static constexpr int ND = nd<ET>();
  static constexpr int NG = 2 * ND - 1;   // accumulator groups (a + b)
  const GramLaunch& a;
  Scratch8 sc;
  int P, z, tr, tc, lane, w, wr, wc, cbase, nslots;
  bool diag, active;
  int64_t pt0;          // first point of the bin in the launch
  i32x4_t acc[2][2][NG];
  double kx[2][2][4];   // e^(s <k, k'>), then kappa, of the lane's point pairs

  __device__ __forceinline__ Tile8(const GramLaunch& la, const Scratch8& s) : a(la), sc(s) {}

  // bin position of the point in slot s (past the bin: the bin's first point)
  __device__ __forceinline__ int slot_pos(int s) const {
    const int q = s < 64 ? 64 * tr + s : 64 * tc + (s - 64);
    return q < a.N ? q : 0;
  }

  // This lane's source pieces (bytes from sc.dig, without the step's offset):
  // wave w fills slots [w nslots / 4, (w + 1) nslots / 4) of a buffer, four
  // per instruction; past a point's ND pieces of a step (fp8) it loads piece 0
  // into the unused slot bytes.
  uint32_t goff[8];
  __device__ __forceinline__ void init_copy() {
    const int per = nslots / 16;   // instructions per wave
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = ((w * per + i) * 64 + lane) * 16;   // this lane's LDS byte
      const int s = o >> 8;
      const int lp = ((o >> 4) & 15) ^ dswz(s);          // logical piece
      goff[i] = i < per ? static_cast<uint32_t>(drow(a, pt0 + slot_pos(s)) * sc.pbytes + 16 * (lp < 4 * ND ? lp : 0)) : 0u;
    }
  }

  // Step st (K steps first, then V) into buf.
  __device__ __forceinline__ void copy(int st, lds_byte* buf) const {
    typedef __attribute__((address_space(1))) const void* gptr;
    typedef __attribute__((address_space(3))) void* lptr;
    const int KS = a.src.E / 64;
    const uint32_t off = static_cast<uint32_t>(st < KS ? 64 * ND * st : ND * a.src.E + 64 * ND * (st - KS));
    const int per = nslots / 16;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < per)
        __builtin_amdgcn_global_load_lds((gptr)(sc.dig + (goff[i] + off)), (lptr)(buf + (w * per + i) * 1024), 16, 0, 0);
  }

  __device__ __forceinline__ i32x4_t piece(const lds_byte* buf, int s, int lp) const {
    typedef __attribute__((address_space(3))) const i32x4_t lds_i4;
    return *reinterpret_cast<lds_i4*>(buf + s * kSlotBytes + 16 * (lp ^ dswz(s)));
  }

  // One step: the copy of step st + 1 into nxt is issued, then the products
  // of step st are taken from cur.  The restrict-qualified views tell the
  // compiler the two do not overlap, so the reads of cur need not wait for
  // the copy.
  __device__ __forceinline__ void overlap(int st, int nst, const lds_byte* __restrict__ cur,
                                          lds_byte* __restrict__ nxt) {
    if (st + 1 < nst) copy(st + 1, nxt);
    if (active) consume(cur);
  }

  // The first V step: its products, then the exponentials of the K part,
  // which depend only on kx and so can issue while the products run.
  __device__ __forceinline__ void overlap_exp(int st, int nst, const lds_byte* __restrict__ cur,
                                              lds_byte* __restrict__ nxt, const double* T) {
    if (st + 1 < nst) copy(st + 1, nxt);
    if (active) consume<true>(cur, T);
  }

  // all digit products of one step; EXP: after the products of each digit d
  // of the row points, the exponentials of a quarter of kx (K part)
  template <bool EXP = false>
  __device__ __forceinline__ void consume(const lds_byte* buf, const double* T = nullptr) {
    const int g = lane >> 4, i16 = lane & 15;
    i32x4_t bo[2][ND];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < ND; ++e) bo[cb][e] = piece(buf, cbase + 32 * wc + 2 * i16 + cb, 4 * e + g);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      i32x4_t ao[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) ao[rb] = piece(buf, 32 * wr + 16 * rb + i16, 4 * d + g);
#pragma unroll
      for (int e = 0; e < ND; ++e)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            acc[rb][cb][d + e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao[rb], bo[cb][e], acc[rb][cb][d + e], 0, 0, 0);
      if constexpr (EXP) {
#pragma unroll
        for (int x = (16 * d) / ND; x < (16 * (d + 1)) / ND; ++x)
          kx[x >> 3][(x >> 2) & 1][x & 3] = exp_tab(kx[x >> 3][(x >> 2) & 1][x & 3], T);
      }
    }
  }

  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int q = 0; q < NG; ++q) acc[rb][cb][q] = i32x4_t{0, 0, 0, 0};
  }

  // The exact dot products of one part, rounded once: the digit groups as two
  // integers below 2^53 (lo: groups 0 .. 3, hi: the rest), then one fma.
  // part 0: kx = s <k, k'> (its exponential is taken during the next step);
  // part 1: kx *= <v, v'> + 1.
  template <int PART>
  __device__ __forceinline__ void finish_part(const int* s_scale, const double* T, double scale) {
    constexpr int part = PART;
    const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int cs = cbase + 32 * wc + 2 * i16 + cb;
        const int csh = s_scale[2 * cs + part];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          double lo = static_cast<double>(acc[rb][cb][3][t]);
          lo = fma(lo, 256.0, static_cast<double>(acc[rb][cb][2][t]));
          lo = fma(lo, 256.0, static_cast<double>(acc[rb][cb][1][t]));
          lo = fma(lo, 256.0, static_cast<double>(acc[rb][cb][0][t]));
          double hi = static_cast<double>(acc[rb][cb][NG - 1][t]);
#pragma unroll
          for (int q = NG - 2; q >= 4; --q) hi = fma(hi, 256.0, static_cast<double>(acc[rb][cb][q][t]));
          const double tot = NG > 4 ? fma(hi, 4294967296.0, lo) : lo;   // 2^32: hi starts at group 4
          const int rs = 32 * wr + 16 * rb + 4 * g + t;
          const double dot = __builtin_amdgcn_ldexp(tot, -(s_scale[2 * rs + part] + csh));
          if constexpr (PART == 0)
            kx[rb][cb][t] = scale * dot;
          else
            kx[rb][cb][t] *= dot + 1.0;
        }
      }
  }

  // G entries of the lane's four pair pairs; pairs whose rows do not fit are
  // left to the fix-up workgroups
  __device__ __forceinline__ void store(const int* s_flag) const {
    const int g = lane >> 4, i16 = lane & 15;
    const int cl = 16 * wc + i16;   // column pair within the tile
    const int col = 32 * tc + cl;
    const bool cbad = s_flag[cbase + 2 * cl] | s_flag[cbase + 2 * cl + 1];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int rl = 16 * wr + 8 * rb + 2 * g + pr;   // row pair within the tile
        const int row = 32 * tr + rl;
        const double gv = (kx[rb][0][2 * pr] - kx[rb][1][2 * pr]) - (kx[rb][0][2 * pr + 1] - kx[rb][1][2 * pr + 1]);
        const bool rbad = s_flag[2 * rl] | s_flag[2 * rl + 1];
        if (row < P && col < P && col >= row && !rbad && !cbad)
          a.G[static_cast<int64_t>(z) * P * P + static_cast<int64_t>(row) * P + col] = gv;
      }
  }
};

template <int ET>
__device__ void gram8_tile(const GramLaunch& a, int tile, int ntiles, lds_byte* smem, double* T, int* s_scale,
                           int* s_flag) {
  constexpr int ND = nd<ET>();
  Tile8<ET> t(a, scratch8(a.dig, ND, a.src.E, a.src.D, dig_points(a)));
  t.P = a.N / 2;
  const int nt = (t.P + 31) / 32;
  const int tiles = nt * (nt + 1) / 2;
  const int bid = static_cast<int>(xcd_remap(tile, ntiles));
  t.z = bid / tiles;
  const int q = bid % tiles;
  int tc = static_cast<int>((sqrtf(8.0f * q + 1.0f) - 1.0f) * 0.5f);   // q -> (tr, tc), tr <= tc
  while (tc * (tc + 1) / 2 > q) --tc;
  while ((tc + 1) * (tc + 2) / 2 <= q) ++tc;
  t.tc = tc;
  t.tr = q - tc * (tc + 1) / 2;
  t.diag = t.tr == t.tc;
  t.cbase = t.diag ? 0 : 64;
  t.nslots = t.diag ? 64 : 128;
  t.lane = threadIdx.x & 63;
  t.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.wr = t.w >> 1;
  t.wc = t.w & 1;
  t.pt0 = static_cast<int64_t>(t.z) * a.N;
  const int r0 = 32 * t.tr + 16 * t.wr, c0 = 32 * t.tc + 16 * t.wc;
  t.active = c0 + 15 >= r0 && r0 < t.P && c0 < t.P;

  if (static_cast<int>(threadIdx.x) < t.nslots) {
    const int64_t pt = drow(a, t.pt0 + t.slot_pos(threadIdx.x));
    s_scale[2 * threadIdx.x] = t.sc.scale[2 * pt];
    s_scale[2 * threadIdx.x + 1] = t.sc.scale[2 * pt + 1];
    s_flag[threadIdx.x] = t.sc.flag[2 * pt] | t.sc.flag[2 * pt + 1];
  }
  T[threadIdx.x] = exp_f64(threadIdx.x * 0.0027076061740622863);   // 2^(j/256), ln 2 / 256
  const int KS = a.src.E / 64, nst = (a.src.E + a.src.D) / 64;
  const double scale = a.scale;
  constexpr int kBuf = kSlots * kSlotBytes;
  t.init_copy();
  t.copy(0, smem);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  t.clear();
  // K steps; the K part's dot products are joined after the last of them
  for (int st = 0; st < KS; ++st) {
    t.overlap(st, nst, smem + (st & 1) * kBuf, smem + ((st + 1) & 1) * kBuf);
    if (t.active && st == KS - 1) {
      t.template finish_part<0>(s_scale, T, scale);
      t.clear();
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this thread's copies have landed
    __syncthreads();
  }
  // the first V step takes the K part's exponentials beside its products
  t.overlap_exp(KS, nst, smem + (KS & 1) * kBuf, smem + ((KS + 1) & 1) * kBuf, T);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int st = KS + 1; st < nst; ++st) {
    t.overlap(st, nst, smem + (st & 1) * kBuf, smem + ((st + 1) & 1) * kBuf);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (t.active) t.template finish_part<1>(s_scale, T, scale);
  if (t.active) t.store(s_flag);
}

// ---------------------------------------------------------------------------
// Pairs whose rows do not fit.  Workgroup f of kFixGroups scans the pairs
// f 256 + [0, 256), (f + kFixGroups) 256 + ..., and for each pair i of bin z
// it finds forms G[z][i][j] for every pair j in fp64 (raw features, FMAs), writing
// row i (j >= i) and, where pair j fits, column i (j < i).
// ---------------------------------------------------------------------------
template <int ET>
__device__ void fix_pair(const GramLaunch& a, const uint8_t* flag, int z, int i, double* xs) {
  const int P = a.N / 2;
  const int E = a.src.E, D = a.src.D, F = E + D;
  // the pair's two rows, widened: xs[c * F + f] (K features, then V)
  for (int e = threadIdx.x; e < 2 * F; e += 256) {
    const int c = e / F, f = e % F;
    const int64_t row = point_row(a, z, 2 * i + c);
    double x;
    if (f < E) {
      Raw8 r;
      load8<ET>(a.src.k, row * E + (f & ~7), r);
      x = raw8_at<ET>(r, f & 7);
    } else {
      Raw8 r;
      load8<ET>(a.src.v, row * D + ((f - E) & ~7), r);
      x = raw8_at<ET>(r, (f - E) & 7);
    }
    xs[e] = x;
  }
  __syncthreads();
  const int64_t pt0 = static_cast<int64_t>(z) * a.N;
  for (int j = threadIdx.x; j < P; j += 256) {
    double kap[2][2];   // [point of pair i][point of pair j]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t row = point_row(a, z, 2 * j + c);
      double dk[2] = {0.0, 0.0}, dv[2] = {0.0, 0.0};
      for (int f = 0; f < E; f += 8) {
        Raw8 r;
        load8<ET>(a.src.k, row * E + f, r);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double y = raw8_at<ET>(r, u);
          dk[0] = fma(xs[f + u], y, dk[0]);
          dk[1] = fma(xs[F + f + u], y, dk[1]);
        }
      }
      for (int f = 0; f < D; f += 8) {
        Raw8 r;
        load8<ET>(a.src.v, row * D + f, r);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double y = raw8_at<ET>(r, u);
          dv[0] = fma(xs[E + f + u], y, dv[0]);
          dv[1] = fma(xs[F + E + f + u], y, dv[1]);
        }
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) kap[r][c] = exp_f64(a.scale * dk[r]) * (dv[r] + 1.0);
    }
    const double gv = (kap[0][0] - kap[0][1]) - (kap[1][0] - kap[1][1]);
    double* G = a.G + static_cast<int64_t>(z) * P * P;
    if (j >= i) {
      G[static_cast<int64_t>(i) * P + j] = gv;
    } else if (pair_flags(a, flag, pt0 / 2 + j) == 0) {   // K and V flags of both points
      G[static_cast<int64_t>(j) * P + i] = gv;
    }
  }
  __syncthreads();
}

template <int ET>
__device__ void gram8_fixup(const GramLaunch& a, int f, double* smem) {
  const int64_t npts = static_cast<int64_t>(a.nbins) * a.N;
  const Scratch8 sc = scratch8(a.dig, nd<ET>(), a.src.E, a.src.D, dig_points(a));
  const int P = a.N / 2;
  const int64_t total = npts / 2;   // pairs of the launch: pair c holds points 2c, 2c + 1
  int* list = reinterpret_cast<int*>(smem + 2 * (a.src.E + a.src.D));
  int* cnt = list + 256;
  for (int64_t c0 = static_cast<int64_t>(f) * 256; c0 < total; c0 += static_cast<int64_t>(kFixGroups) * 256) {
    if (threadIdx.x == 0) *cnt = 0;
    __syncthreads();
    const int64_t c = c0 + threadIdx.x;
    if (c < total && pair_flags(a, sc.flag, c) != 0) list[atomicAdd(cnt, 1)] = threadIdx.x;
    __syncthreads();
    const int n = *cnt;
    for (int k = 0; k < n; ++k) {
      const int64_t pc = c0 + list[k];
      fix_pair<ET>(a, sc.flag, static_cast<int>(pc / P), static_cast<int>(pc % P), smem);
    }
    __syncthreads();
  }
}

template <int ET>
__global__ __launch_bounds__(256, 2) void gram8_kernel(GramLaunch a, int nthr, int per_wave, int ntiles) {
  // 64 KB of digit buffers, then 2^(j/256), then the tile's scales and flags
  __shared__ __attribute__((aligned(16))) double smem[2 * kSlots * kSlotBytes / 8 + 256 + kSlots + kSlots / 2];
  const int bid = blockIdx.x;
  if (bid < nthr) {
    threshold_workgroup<ET>(a, bid, nthr, per_wave, smem);
    return;
  }
  if (bid < nthr + kFixGroups) {
    gram8_fixup<ET>(a, bid - nthr, smem);
    return;
  }
  double* T = smem + 2 * kSlots * kSlotBytes / 8;
  int* s_scale = reinterpret_cast<int*>(T + 256);
  int* s_flag = s_scale + 2 * kSlots;
  gram8_tile<ET>(a, bid - nthr - kFixGroups, ntiles, (lds_byte*)smem, T, s_scale, s_flag);
}

}  // namespace

bool gram8_supported(int dtype, int E, int D, int N) {   // E, D in {64, 128, 256}: the digit pass's lane groups
  const auto dim_ok = [](int F) { return F == 64 || F == 128 || F == 256; };
  return (dtype == kBF16 || dtype == kFP8) && dim_ok(E) && dim_ok(D) && N >= 256 && N % 2 == 0;
}

bool gram8_fits(int dtype, int64_t npts, int E, int D) {   // the tiles address the digits with 32-bit offsets
  return npts * digit_bytes(dtype == kFP8 ? 3 : 4, E, D) < (static_cast<int64_t>(1) << 31);
}

size_t gram8_scratch_bytes(int dtype, int E, int D, int64_t npts) {
  const int nd_ = dtype == kFP8 ? 3 : 4;
  const int64_t dig = (npts * digit_bytes(nd_, E, D) + 255) / 256 * 256;
  return static_cast<size_t>(dig + npts * 10);
}

// Launch geometry of the integer Gram over a.
static bool gram8_launch_ok(const GramLaunch& a) {
  return a.dig && gram8_supported(a.src.dtype, a.src.E, a.src.D, a.N) &&
         gram8_fits(a.src.dtype, dig_points(a), a.src.E, a.src.D) &&
         (a.dig_map || a.dig_row0 + static_cast<int64_t>(a.nbins) * a.N <= dig_points(a));
}

hipError_t launch_gram8_digits(const GramLaunch& a, hipStream_t s) {
  if (!gram8_launch_ok(a) || a.dig_map) return hipErrorInvalidValue;
  const int64_t npts = static_cast<int64_t>(a.nbins) * a.N;
  if (npts == 0) return hipSuccess;
  const int64_t blocks_k = (npts * (a.src.E / 16) + 255) / 256, blocks_v = (npts * (a.src.D / 16) + 255) / 256;
  const dim3 g1(static_cast<unsigned>(blocks_k + blocks_v));
  if (a.src.dtype == kFP8)
    hipLaunchKernelGGL(gram8_digits_kernel<kFP8>, g1, dim3(256), 0, s, a, static_cast<int>(blocks_k));
  else
    hipLaunchKernelGGL(gram8_digits_kernel<kBF16>, g1, dim3(256), 0, s, a, static_cast<int>(blocks_k));
  return hipGetLastError();
}

hipError_t launch_gram8_tiles(const GramLaunch& a, hipStream_t s, hipEvent_t done) {
  if (!gram8_launch_ok(a)) return hipErrorInvalidValue;
  const int64_t npts = static_cast<int64_t>(a.nbins) * a.N;
  if (npts == 0) return hipSuccess;
  const int P = a.N / 2;
  const int nt = (P + 31) / 32;
  const int64_t tiles = static_cast<int64_t>(nt) * (nt + 1) / 2 * a.nbins;
  int nthr, per_wave;
  threshold_groups(a, nthr, per_wave);
  const dim3 g2(static_cast<unsigned>(nthr + kFixGroups + tiles));
  if (a.src.dtype == kFP8)
    launch_signal(gram8_kernel<kFP8>, g2, dim3(256), 0, s, done, a, nthr, per_wave, static_cast<int>(tiles));
  else
    launch_signal(gram8_kernel<kBF16>, g2, dim3(256), 0, s, done, a, nthr, per_wave, static_cast<int>(tiles));
  return hipGetLastError();
}

hipError_t launch_pair_gram8(const GramLaunch& a, hipStream_t s) {
  const hipError_t e = a.dig_map ? hipSuccess : launch_gram8_digits(a, s);
  return e != hipSuccess ? e : launch_gram8_tiles(a, s);
}

bool gram8_runs(const GramLaunch& a) { return gram8_launch_ok(a); }

}  // namespace thin
