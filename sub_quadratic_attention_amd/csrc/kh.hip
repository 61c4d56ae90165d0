// Kernel halving on gfx950: fp64 pair Gram under kappa_att and the sequential
// self-balancing walk, plus the index bookkeeping of Compress and EXPRESS.
//
// kappa((k, v), (k', v')) = exp(s <k, k'>) (<v, v'> + 1): the exponential
// dot-product kernel on keys times the linear kernel on (v, 1), whose inner
// products are exactly the two sums softmax attention needs ("Express
// Language Modeling", section "Thinformer Express", names this key-value
// attention kernel).  The walk is kernel halving as published in the
// kernel-thinning papers (Dwivedi and Mackey, "Kernel Thinning"; Shetty,
// Dwivedi and Mackey, "Distribution Compression in Near-linear Time").
//
// Precision: every dot product is accumulated in fp64 (products of fp32,
// bf16 or fp8 inputs are exact in fp64) and exp is evaluated in fp64, so that the
// randomised sign decisions agree with a float64 reference except at true
// near-ties.

#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "khdev.hpp"

namespace thin {

namespace {

// ---------------------------------------------------------------------------
// Pair Gram.  One workgroup (4 waves) computes a 32 x 32 tile of pairs
// (64 x 64 points); wave (wr, wc) owns the 16 x 16 pair block (16 wr..,
// 16 wc..).  The products run on the fp64 MFMA 4x4x4 with four blocks: block
// beta of an instruction multiplies A[m][k] (lane 16 k + 4 beta + m) by
// B[k][n] (lane 16 k + 4 beta + n) into D[m][n] (lane 16 m + 4 beta + n).
// A carries the same four row points in every block and B sixteen column
// points, four per block, so one instruction is a 4 x 16 strip of point
// products over four features.  A wave keeps 8 row quads (the even and the
// odd points of its 16 row pairs, four pairs each) against 2 column sets
// (even and odd points of its 16 column pairs): the four point products of a
// pair pair land in one lane, and G = k_ee - k_eo - k_oe + k_oo needs no lane
// exchange.  Pass 0 accumulates <k, k'>, pass 1 <v, v'>.
//
// On gfx950 this form of the fp64 MFMA sustains about 1.5x the rate of the
// 16x16x4 form, and vector instructions issued between fp64 MFMAs delay them,
// so the inner loop holds nothing but LDS reads and MFMAs: points are widened
// to fp64 once, when a step of 16 features is staged (loaded into registers
// one step ahead, then written to LDS, double buffered).  The tile's 64 row
// points take slots 0..63 and its column points 64..127 (a diagonal tile
// reads its columns from the row slots); within a set, slot s holds the point
// of parity (s >> 2) & 1 of pair 4 (s >> 3) + (s & 3), so every row quad is
// four consecutive slots.  A slot's eight 16-byte pieces (two features each)
// are stored XOR-swizzled by gswz(slot), which puts the sixteen column points
// a B read touches into distinct LDS banks.
// ---------------------------------------------------------------------------
constexpr int kStageF = 16;            // features staged per step
constexpr int kStage = kStageF * 8;    // bytes of one staged point
constexpr int kSlots = 128;            // row and column points of a tile
constexpr int kRing = 4;               // staging register sets
constexpr int kAhead = 2;              // steps a load is issued ahead of its use (keeps 4 workgroups per CU)
typedef __attribute__((address_space(3))) unsigned char lds_byte;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int gswz(int slot) { return ((slot >> 1) & 1) | ((slot >> 2) & 6); }

// tile point (0..63) held by slot s of a set
__device__ __forceinline__ int slot_point(int s) { return 8 * (s >> 3) + 2 * (s & 3) + ((s >> 2) & 1); }


// Tiles.  Bins get the upper-triangular 32 x 32 pair tiles of their own
// P x P Gram (G is symmetric; the walk reads G[j][i] for j <= i, so the
// contribution of pairs j to every later pair i is a contiguous row segment),
// except bins with P dividing 32 (P < 32), which are packed: a unit's bins
// are consecutive in its point list, so one diagonal tile of 32 pairs covers
// 32 / P whole bins and only entries of equal bin are kept.  Blocks lying
// entirely below the diagonal are skipped.  Points beyond the bin (or the
// unit's last bin) are loaded from a valid point; the entries they touch are
// never stored.
template <int ET>
struct GramTile {
  int lane, wr, wc, nK, nst;
  bool active, loader;
  int cbase;                       // first slot of the column set (0 on the diagonal)
  int wofs;                        // this thread's staging slot and half, as an LDS byte offset base
  const unsigned char* kp;         // staging: this thread's point row in K and V, plus its half
  const unsigned char* vp;
  u32x4_t raw[kRing][2];           // staging registers, a ring over steps: 8 features (bf16: [0]; fp8: [0].xy)
  double acc[2][2][4][2];          // [pass][row parity][row quad][column parity]

  // Staging role: thread t loads features 8 (t & 1) .. + 7 of step st for the
  // point of slot t >> 1 (threads of slots >= 64 idle on a diagonal tile).
  // Loads are issued unconditionally (steps past the end repeat the last one,
  // idle threads read a valid row) so that no branch hides them from the
  // wait counting: a write waits for its own step only.
  template <int R>
  __device__ __forceinline__ void load(int st) {
    st = st < nst ? st : nst - 1;
    const bool vpass = st >= nK;
    const unsigned char* src = (vpass ? vp : kp) + (vpass ? st - nK : st) * (kStageF * elt_size<ET>());
    if constexpr (ET == kFP8) {
      const uint2 x = *reinterpret_cast<const uint2*>(src);
      raw[R][0][0] = x.x;
      raw[R][0][1] = x.y;
    } else {
      raw[R][0] = *reinterpret_cast<const u32x4_t*>(src);
    }
    if constexpr (ET == kF32) raw[R][1] = *reinterpret_cast<const u32x4_t*>(src + 16);
  }

  template <int R>
  __device__ __forceinline__ double feature(int j) const {
    if constexpr (ET == kFP8) {
      return static_cast<double>(fp8_byte_to_float(raw[R][0][j >> 2], j & 3));
    } else if constexpr (ET == kBF16) {
      const uint32_t word = raw[R][0][j >> 1];
      return static_cast<double>(__uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16)));
    } else {
      return static_cast<double>(__uint_as_float(raw[R][j >> 2][j & 3]));
    }
  }

  // The staged features, widened, into buffer dst: pieces 4 (t & 1) + i of
  // the slot, two features each.
  template <int R>
  __device__ __forceinline__ void write(lds_byte* dst) const {
    typedef __attribute__((address_space(3))) f64x2_t lds_f64x2;
    if (!loader) return;
    const int slot = wofs >> 1, half = wofs & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = (4 * half + i) ^ gswz(slot);
      *reinterpret_cast<lds_f64x2*>(dst + slot * kStage + 16 * piece) = f64x2_t{feature<R>(2 * i), feature<R>(2 * i + 1)};
    }
  }

  // All products of one staged step into acc[PASS]: lane group k reads piece
  // k + 4 jj of its row quads and column points; element e of those pieces
  // (feature 8 jj + 2 k + e) is one MFMA k-step.
  template <int PASS>
  __device__ __forceinline__ void consume(const lds_byte* cur) {
    typedef __attribute__((address_space(3))) const f64x2_t lds_f64x2;
    const int k = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      f64x2_t ra[2][4], rb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = 32 * wr + 8 * r + 4 * e + (lane & 3);
          ra[e][r] = *reinterpret_cast<lds_f64x2*>(cur + slot * kStage + 16 * ((k + 4 * jj) ^ gswz(slot)));
        }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int slot = cbase + 32 * wc + 8 * ((lane >> 2) & 3) + 4 * c + (lane & 3);
        rb[c] = *reinterpret_cast<lds_f64x2*>(cur + slot * kStage + 16 * ((k + 4 * jj) ^ gswz(slot)));
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[PASS][e][r][0] = __builtin_amdgcn_mfma_f64_4x4x4f64(ra[e][r][x], rb[0][x], acc[PASS][e][r][0], 0, 0, 0);
            acc[PASS][e][r][1] = __builtin_amdgcn_mfma_f64_4x4x4f64(ra[e][r][x], rb[1][x], acc[PASS][e][r][1], 0, 0, 0);
          }
    }
  }

  // Step st (st % kRing == R) is in buffer R & 1.  Step st + 1, loaded
  // kAhead - 1 steps ago, is written to the other buffer, the load of step
  // st + kAhead issued, then the products of step st taken.
  template <int PASS, int R>
  __device__ __forceinline__ void step(int st, lds_byte* smem) {
    if (st + 1 < nst) write<(R + 1) % kRing>(smem + ((R + 1) & 1) * kSlots * kStage);
    load<(R + kAhead) % kRing>(st + kAhead);
    if (active) consume<PASS>(smem + (R & 1) * kSlots * kStage);
    __syncthreads();
  }

  template <int PASS>
  __device__ __forceinline__ void steps(int st, lds_byte* smem) {   // st % kRing == 0
    step<PASS, 0>(st, smem);
    step<PASS, 1>(st + 1, smem);
    step<PASS, 2>(st + 2, smem);
    step<PASS, 3>(st + 3, smem);
  }
};


template <int ET>
__device__ void gram_tile(const GramLaunch& a, int nthr, lds_byte* smem, double* T) {
  const int P = a.N / 2;
  const bool packed = P < 32 && (32 % P) == 0;   // whole bins per tile
  const int bid = static_cast<int>(xcd_remap(blockIdx.x - nthr, gridDim.x - nthr));
  int unit, tr, tc, z;
  if (packed) {
    const int tiles = (a.bins_per_unit * P + 31) / 32;
    unit = bid / tiles;
    tr = tc = bid % tiles;
    z = -1;
  } else {
    const int nt = (P + 31) / 32;
    const int tiles = nt * (nt + 1) / 2;
    z = bid / tiles;
    const int t = bid % tiles;
    // t -> (tc, tr) with tr <= tc: tile row tr, tile column tc of the upper triangle
    tc = static_cast<int>((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while (tc * (tc + 1) / 2 > t) --tc;
    while ((tc + 1) * (tc + 2) / 2 <= t) ++tc;
    tr = t - tc * (tc + 1) / 2;
    unit = z / a.bins_per_unit;
  }
  const int b = unit / a.src.H_kv;
  const int h = unit % a.src.H_kv;
  const bool diag = tr == tc;          // rows and columns are the same points

  GramTile<ET> t;
  t.lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.wr = w >> 1;
  t.wc = w & 1;
  t.cbase = diag ? 0 : 64;
  t.nK = a.src.E / kStageF;
  t.nst = t.nK + a.src.D / kStageF;

  const int64_t ubase = static_cast<int64_t>(unit) * a.idx_unit_stride;
  auto token = [&](int q) -> int {   // q-th point of the tile's range; the range's first if none
    if (packed) {
      const int bin = q / a.N;
      const bool in = bin < a.bins_per_unit;
      return a.idx[ubase + static_cast<int64_t>(in ? bin : 0) * a.idx_stride + (in ? q % a.N : 0)];
    }
    return a.idx[ubase + static_cast<int64_t>(z % a.bins_per_unit) * a.idx_stride + (q < a.N ? q : 0)];
  };
  {
    const int slot = threadIdx.x >> 1, half = threadIdx.x & 1;
    t.wofs = threadIdx.x;
    t.loader = slot < (diag ? 64 : 128);
    const int tp = slot_point(slot & 63);
    int tok = t.loader ? token((slot < 64 ? 64 * tr : 64 * tc) + tp) : 0;
    if (static_cast<uint32_t>(tok) >= static_cast<uint32_t>(a.src.S)) {   // clamped, and reported
      if (a.err) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      tok = tok < 0 ? 0 : static_cast<int>(a.src.S - 1);
    }
    const int elt = elt_size<ET>();
    const int64_t row = (static_cast<int64_t>(b) * a.src.S + tok) * a.src.H_kv + h;
    t.kp = static_cast<const unsigned char*>(a.src.k) + (row * a.src.E + 8 * half) * elt;
    t.vp = static_cast<const unsigned char*>(a.src.v) + (row * a.src.D + 8 * half) * elt;
  }

  // does this wave's 16 x 16 pair block hold anything the walk reads?
  const int r0 = 32 * tr + 16 * t.wr;    // first pair row of the block
  const int c0 = 32 * tc + 16 * t.wc;    // first pair column
  bool active = c0 + 15 >= r0;            // not entirely below the diagonal
  if (packed && active && t.wr != t.wc) active = (r0 % P) != 0;   // a bin straddles the two halves
  if (!packed && (r0 >= P || c0 >= P)) active = false;
  t.active = active;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) t.acc[p][e][r][0] = t.acc[p][e][r][1] = 0.0;

  // 2^(j/256), j = 0..255, for exp_tab (published by the barrier below)
  T[threadIdx.x] = exp_f64(threadIdx.x * 0.0027076061740622863);   // ln 2 / 256
  t.template load<0>(0);
  t.template load<1>(1);
  t.template write<0>(smem);
  __syncthreads();
  for (int st = 0; st < t.nK; st += kRing) t.template steps<0>(st, smem);   // E and D are multiples of kRing steps
  for (int st = t.nK; st < t.nst; st += kRing) t.template steps<1>(st, smem);
  if (!active) return;

  // accumulator of lane l: row point (l >> 4) of its quad, column (l & 15) of its set
  const int col = c0 + (t.lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = r0 + 4 * r + (t.lane >> 4);
    double kx[2][2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int c = 0; c < 2; ++c) kx[e][c] = exp_tab(a.scale * t.acc[0][e][r][c], T) * (t.acc[1][e][r][c] + 1.0);
    const double gv = (kx[0][0] - kx[0][1]) - (kx[1][0] - kx[1][1]);
    if (packed) {
      const int bin = row / P;
      if (bin == col / P && bin < a.bins_per_unit && col >= row)
        a.G[(static_cast<int64_t>(unit) * a.bins_per_unit + bin) * P * P + (row % P) * P + (col % P)] = gv;
    } else if (row < P && col < P && col >= row) {   // below the diagonal: thresholds
      a.G[static_cast<int64_t>(z) * P * P + static_cast<int64_t>(row) * P + col] = gv;
    }
  }
}

// The first nthr workgroups form the thresholds, the others the tiles.
template <int ET>
__global__ __launch_bounds__(256, 4) void pair_gram_kernel(GramLaunch a, int nthr, int thr_per_wave) {
  __shared__ __attribute__((aligned(16))) double smem[2 * kSlots * kStage / sizeof(double) + 256];
  if (static_cast<int>(blockIdx.x) < nthr) {
    threshold_workgroup<ET>(a, blockIdx.x, nthr, thr_per_wave, smem);
    return;
  }
  gram_tile<ET>(a, nthr, (lds_byte*)smem, smem + 2 * kSlots * kStage / sizeof(double));
}

// ---------------------------------------------------------------------------
// Kernel-halving walk of one bin per workgroup, on thresholds formed by the
// pair-Gram launch.
//
// The walk runs in panels of 64 pairs.  alpha_i = sum_{j<i} eta_j G_ji is
// kept for every pair in LDS.  For panel p:
//   wave 0   takes the 64 decisions: lane l holds alpha of pair p0+l and its
//            column of the panel's diagonal block; one ballot per decision;
//   wave 1-2 stage the next panel's diagonal block (double buffered);
// then all waves add the panel's contribution sum_j eta_j G[j][i] to the
// alpha of every later pair (coalesced row segments, many in flight).
// ---------------------------------------------------------------------------
// Digit-scratch row of point q of bin z (the integer Gram's rows).
__device__ __forceinline__ int32_t kept_row(const SweepLaunch& a, int z, int q) {
  const int64_t pt = static_cast<int64_t>(z) * a.N + q;
  return static_cast<int32_t>(a.row_map ? a.row_map[pt] : a.row0 + pt);
}

__device__ __forceinline__ int64_t dec_offset(const SweepLaunch& a, int lb, int P) {
  if (a.dec_mode == 1) {   // Express batch k = lb: HALVE 0, then (3 batches, HALVE) per epoch
    const int64_t n = P;
    return 3 * n + 6 * n * (lb / 3) + n * (lb % 3);
  }
  return a.dec_base + static_cast<int64_t>(lb) * P;
}

// Rows q0..q0+63, columns q0..q0+63 of a bin's G into LDS (row stride 65),
// `PER` consecutive doubles per thread, all loads issued before any store.
// Entries below the diagonal are copied too: the chain only reads G[j][i]
// for j < i (the upper triangle), so they never influence a decision.  Rows
// and columns beyond P read as 0.
template <int PER>
__device__ __forceinline__ void stage_block(const double* G, int P, int q0, double* dst, int t) {
  const int r = (t * PER) >> 6;
  const int cb = (t * PER) & 63;
  const bool rok = q0 + r < P;
  const double* src = G + static_cast<int64_t>(q0 + r) * P + q0 + cb;
  double v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = (rok && q0 + cb + j < P) ? src[j] : 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) dst[r * 65 + cb + j] = v[j];
}


// Thresholds of the pairs [i0, i0 + 64) by one wave: lane l holds b^2, b and
// u of pair i0 + l in registers; the recursion runs on uniform values read
// with readlane (no memory access on the serial path) and lane i keeps the
// threshold of pair i0 + i.  The only serial operation besides fma / max is
// sqrt(sigma^2); the hardware fp64 square root is used (its error is far
// below the 1e-6 decision margins that matter).

__global__ __launch_bounds__(256) void halving_sweep_kernel(SweepLaunch a) {
  extern __shared__ double smem[];
  const int z = blockIdx.x;
  const int P = a.N / 2;
  const int unit = z / a.bins_per_unit;
  const int lb = z % a.bins_per_unit;
  const double* G = a.G + static_cast<int64_t>(z) * P * P;
  double* s_thr = smem;               // P   thresholds (formed by the pair-Gram launch)
  double* s_alpha = s_thr + P;        // P
  double* s_eta = s_alpha + P;        // P   (+1 / -1)
  double* s_G = s_eta + P;            // 2 x 64 x 65

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  for (int i = tid; i < P; i += 256) {
    s_thr[i] = G[thr_slot(i, P)];
    s_alpha[i] = 0.0;
  }
  const int np = (P + 63) / 64;
  stage_block<16>(G, P, 0, s_G, tid);   // panel 0's diagonal block
  __syncthreads();

  const int32_t* in = a.idx_in + static_cast<int64_t>(unit) * a.in_unit_stride + static_cast<int64_t>(lb) * a.in_stride;
  int32_t* out = a.idx_out + static_cast<int64_t>(z) * a.out_stride;
  int32_t* pout = a.row_out ? a.row_out + static_cast<int64_t>(z) * a.out_stride : nullptr;
  uint8_t* dec = a.dec ? a.dec + static_cast<int64_t>(unit) * a.dec_per_unit + dec_offset(a, lb, P) : nullptr;
  for (int p = 0; p < np; ++p) {
    const int p0 = 64 * p;
    const int rows = min(64, P - p0);
    const double* blk = s_G + (p & 1) * 64 * 65;
    if (w == 0) {
      double alpha = s_alpha[p0 + lane < P ? p0 + lane : 0];
      const double thr = lane < rows ? s_thr[p0 + lane] : 0.0;
      double g[64];   // g[cc] = G[p0 + cc][p0 + lane]: the upper triangle holds it for cc < lane
#pragma unroll
      for (int cc = 0; cc < 64; ++cc) g[cc] = blk[cc * 65 + lane];
      // decision j is lane j's: its sign eta_j = +1 (keep the first point)
      // or -1 comes to every lane as the high word of a double through
      // readlane, and alpha += eta_j g[j] is one fma with that scalar operand
      // (exact product, the same rounding as the add); the decision bits come
      // from the same compare's lane mask, off the dependent chain
      uint64_t bits = 0;
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        const bool lt = alpha < thr;
        bits |= __ballot(lt) & (1ull << j);
        const uint32_t hj = __builtin_amdgcn_readlane(lt ? 0x3FF00000u : 0xBFF00000u, j);
        alpha = fma(__hiloint2double(static_cast<int>(hj), 0), g[j], alpha);
      }
      if (lane < rows) {
        const int i = p0 + lane;
        const bool first = (bits >> lane) & 1ull;
        s_eta[i] = first ? 1.0 : -1.0;
        out[i] = in[2 * i + (first ? 0 : 1)];
        if (pout) pout[i] = kept_row(a, z, 2 * i + (first ? 0 : 1));
        if (dec) dec[i] = first ? 1 : 0;
      }
    } else if (w <= 2 && p + 1 < np) {
      // waves 1 and 2 stage the next diagonal block
      stage_block<32>(G, P, p0 + 64, s_G + ((p + 1) & 1) * 64 * 65, tid - 64);
    }
    __syncthreads();
    // the panel's contribution to every later pair i: sum_j eta_j G[p0 + j][i],
    // row segments of the upper triangle, read coalesced across the lanes
    if (p + 1 < np) {
      for (int i = p0 + 64 + tid; i < P; i += 256) {
        const double* col = G + static_cast<int64_t>(p0) * P + i;
        double gv[64];                       // full panel: rows == 64 here; all loads in flight
#pragma unroll
        for (int j = 0; j < 64; ++j) gv[j] = col[static_cast<int64_t>(j) * P];
        double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
        for (int j = 0; j < 64; j += 2) {
          acc0 += s_eta[p0 + j] * gv[j];
          acc1 += s_eta[p0 + j + 1] * gv[j + 1];
        }
        s_alpha[i] += acc0 + acc1;
      }
      __syncthreads();
    }
  }
}

// Bins of at most 64 pairs: one wave per bin, four bins per workgroup.
// Lane i holds pair i: its threshold, alpha_i and row i of G (lower part)
// in registers; lane 0 runs the sigma recursion reading b_i from lane i.
template <int PMAX>
__global__ __launch_bounds__(256) void halving_sweep_small_kernel(SweepLaunch a) {
  const int P = a.N / 2;
  const int lane = threadIdx.x & 63;
  const int z = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (z >= a.nbins) return;   // whole wave: no barrier in this kernel
  const int unit = z / a.bins_per_unit;
  const int lb = z % a.bins_per_unit;
  const double* G = a.G + static_cast<int64_t>(z) * P * P;
  const bool mine = lane < P;
  double g[PMAX];
#pragma unroll
  for (int j = 0; j < PMAX; ++j) g[j] = (mine && j < lane) ? G[static_cast<int64_t>(j) * P + lane] : 0.0;   // upper triangle
  // thresholds of at most 64 pairs, formed here (b^2 from the Gram diagonal)
  const double u = mine ? philox_uniform(static_cast<uint64_t>(lane), a.bin_base + lb, static_cast<uint64_t>(unit),
                                         a.tag, a.seed)
                        : 0.0;
  const double b2 = mine ? fmax(G[static_cast<int64_t>(lane) * P + lane], 0.0) : 0.0;
  const double c = sqrt(2.0 * log(2.0 * a.N / a.delta));
  double s2 = 0.0;
  const double thr =
      step_threshold(a.greedy, sigma_steps(s2, b2, sqrt(b2), P, c, 1.0 + 1.0 / (c * c), 2.0 / c), u);
  double alpha = 0.0;
  uint64_t bits = 0;
#pragma unroll
  for (int j = 0; j < PMAX; ++j) {
    if (j >= P) continue;   // uniform: P is the same for the whole wave
    const uint64_t m = __ballot(alpha < thr);
    const bool first = (m >> j) & 1ull;
    bits |= static_cast<uint64_t>(first) << j;
    alpha += first ? g[j] : -g[j];
  }
  if (mine) {
    const bool first = (bits >> lane) & 1ull;
    const int32_t* in = a.idx_in + static_cast<int64_t>(unit) * a.in_unit_stride + static_cast<int64_t>(lb) * a.in_stride;
    a.idx_out[static_cast<int64_t>(z) * a.out_stride + lane] = in[2 * lane + (first ? 0 : 1)];
    if (a.row_out) a.row_out[static_cast<int64_t>(z) * a.out_stride + lane] = kept_row(a, z, 2 * lane + (first ? 0 : 1));
    if (a.dec) a.dec[static_cast<int64_t>(unit) * a.dec_per_unit + dec_offset(a, lb, P) + lane] = first ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Index bookkeeping.
// ---------------------------------------------------------------------------
__global__ void iota_kernel(int32_t* out, int64_t units, int64_t n, int64_t stride) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= units * n) return;
  out[(i / n) * stride + (i % n)] = static_cast<int32_t>(i % n);
}

// Uniform subsampling of the thin phase: batch k of epoch e = k / 3 + 1
// (m = 4^e, r = m / 2) covers tokens [4^e n (1 + k % 3), 4^e n (2 + k % 3))
// in 2n aligned groups of r tokens; each group contributes the token at
// offset floor(u r), u from counter (group, log2 r, unit, subsample tag).
// One random point per stratum of r consecutive list entries (base subsampling
// ahead of the Compress; the strata are the Compress base blocks' sub-blocks).
__global__ void base_sample_kernel(const int32_t* list, int64_t L, int units, int64_t r, uint64_t seed, int32_t* out) {
  const int64_t Lp = L / r;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= Lp * units) return;
  const int unit = static_cast<int>(i / Lp);
  const int64_t t = i % Lp;
  const double u = philox_uniform(static_cast<uint64_t>(t), 0, static_cast<uint64_t>(unit), kTagBaseSample, seed);
  const int64_t off = min(static_cast<int64_t>(floor(u * static_cast<double>(r))), r - 1);
  const int64_t pos = t * r + off;
  out[i] = list ? list[static_cast<int64_t>(unit) * L + pos] : static_cast<int32_t>(pos);
}

__global__ void express_reps_kernel(ExpressView ev, int units, uint64_t seed, int32_t* reps) {
  const int64_t per_unit = static_cast<int64_t>(ev.n_batches_alloc) * 2 * ev.n;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per_unit * units) return;
  const int unit = static_cast<int>(i / per_unit);
  const int64_t rem = i % per_unit;
  const int k = static_cast<int>(rem / (2 * ev.n));
  const int slot = static_cast<int>(rem % (2 * ev.n));
  const int e = k / 3 + 1;
  const int log2m = 2 * e;
  const int log2r = log2m - 1;
  const int64_t start = (static_cast<int64_t>(ev.n) << log2m) * (1 + k % 3);
  const int64_t g = (start >> log2r) + slot;
  const uint64_t word = philox_word0(static_cast<uint64_t>(g), static_cast<uint64_t>(log2r),
                                     static_cast<uint64_t>(unit), kTagSubsample, seed);
  const int64_t off = static_cast<int64_t>(word >> (64 - log2r));
  reps[i] = static_cast<int32_t>((g << log2r) + off);
}

// Input list of HALVE e: the first 4n tokens (e = 0), else the output of
// HALVE e-1 followed by the three batches of epoch e; with rows.out (e >= 1),
// also the points' digit-scratch rows, from the same places of rows.halve and
// rows.batch.
__global__ void halve_input_kernel(ExpressView ev, int units, int e, int32_t* halve_in, HalveRows rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per = 4LL * ev.n;
  if (i >= per * units) return;
  const int unit = static_cast<int>(i / per);
  const int j = static_cast<int>(i % per);
  int32_t val;
  if (e == 0) {
    val = j;
  } else if (j < ev.n) {
    const int64_t at = (static_cast<int64_t>(unit) * ev.n_halves + (e - 1)) * ev.n + j;
    val = ev.halve_out[at];
    if (rows.out) rows.out[i] = rows.halve[at];
  } else {
    const int64_t at = (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (e - 1)) * ev.n + (j - ev.n);
    val = ev.batch_out[at];
    if (rows.out) rows.out[i] = rows.batch[at];
  }
  halve_in[i] = val;
}

// Final causal coreset of a unit: the cache and buffer after every full block,
// then the trailing partial block (weight 1), padded with -1 / 0.
__device__ void express_state_after(const ExpressView& ev, int unit, int beta, int& n_halve_pts,
                                    const int32_t*& halve_pts, int& n_batch_pts, const int32_t*& batch_pts,
                                    int& n_rep, const int32_t*& rep_pts, int& raw_prefix, float& wm, float& wr) {
  n_halve_pts = n_batch_pts = n_rep = 0;
  halve_pts = batch_pts = rep_pts = nullptr;
  raw_prefix = 0;
  wm = 1.0f;
  wr = 1.0f;
  if (beta < 4) {
    raw_prefix = beta * ev.n;
    return;
  }
  int E = 1;
  while ((1LL << (2 * (E + 1))) <= beta) ++E;
  const int m = 1 << (2 * E);
  const int since = beta - m;
  const int nbc = since / m;
  const int rem = since % m;
  wm = static_cast<float>(m);
  wr = static_cast<float>(m / 2);
  n_halve_pts = ev.n;
  halve_pts = ev.halve_out + (static_cast<int64_t>(unit) * ev.n_halves + (E - 1)) * ev.n;
  n_batch_pts = nbc * ev.n;
  batch_pts = ev.batch_out + (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (E - 1)) * ev.n;
  n_rep = static_cast<int>((static_cast<int64_t>(rem) * 2 * ev.n) / m);
  rep_pts = ev.reps + (static_cast<int64_t>(unit) * ev.n_batches_alloc + 3 * (E - 1) + nbc) * 2 * ev.n;
}

__global__ void express_final_kernel(ExpressView ev, int units, int S, int32_t* idx, float* w, int32_t* len,
                                     int64_t cap) {
  const int unit = blockIdx.x;
  int nh, nb, nr, raw;
  const int32_t *hp, *bp, *rp;
  float wm, wr;
  express_state_after(ev, unit, ev.nblk, nh, hp, nb, bp, nr, rp, raw, wm, wr);
  const int tail_start = ev.nblk * ev.n;
  const int n_raw = raw + (S - tail_start);   // raw prefix (exact phase) + trailing block
  const int total = nh + nb + nr + n_raw;
  int32_t* oi = idx ? idx + static_cast<int64_t>(unit) * cap : nullptr;
  float* ow = w ? w + static_cast<int64_t>(unit) * cap : nullptr;
  for (int j = threadIdx.x; j < cap; j += blockDim.x) {
    int32_t id = -1;
    float wt = 0.0f;
    if (j < nh) {
      id = hp[j];
      wt = wm;
    } else if (j < nh + nb) {
      id = bp[j - nh];
      wt = wm;
    } else if (j < nh + nb + nr) {
      id = rp[j - nh - nb];
      wt = wr;
    } else if (j < total) {
      const int r = j - nh - nb - nr;
      id = r < raw ? r : tail_start + (r - raw);
      wt = 1.0f;
    }
    if (oi) oi[j] = id;
    if (ow) ow[j] = wt;
  }
  if (len && threadIdx.x == 0) len[unit] = total;
}

__global__ void fill_coreset_kernel(const int32_t* src, int64_t src_stride, int units, int n, float wv,
                                    int32_t* idx, float* w, int32_t* len) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(units) * n) return;
  const int64_t u = i / n, j = i % n;
  if (idx) idx[i] = src ? src[u * src_stride + j] : static_cast<int32_t>(j);
  if (w) w[i] = wv;
  if (len && j == 0) len[u] = n;
}

__global__ void sanitize_indices_kernel(const int32_t* in, int64_t n, int32_t S, int32_t* out, int* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t x = in[i];
  const bool bad = static_cast<uint32_t>(x) >= static_cast<uint32_t>(S);
  out[i] = bad ? (x < 0 ? 0 : S - 1) : x;
  if (bad && err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ void philox_words_kernel(const uint64_t* ctr, int64_t n, uint64_t seed, uint64_t* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t x[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  philox4x64_10(x, seed, 0);
  out[4 * i] = x[0];
  out[4 * i + 1] = x[1];
  out[4 * i + 2] = x[2];
  out[4 * i + 3] = x[3];
}

// ---------------------------------------------------------------------------
// Bins of at most 16 points: Gram, thresholds and walk in one launch.  A wave
// takes a tile of 16 points of one unit -- 16 / N whole bins -- and forms
// their point Gram X X^T, keys and values apart, on the fp64 MFMA 16x16x4
// (A[i][k] at lane i + 16 k, B[k][j] at lane j + 16 k, D[i][j] in lane
// j + 16 (i % 4), element i / 4): for X X^T the A and B operands are the same
// register, lane l holding a feature of point l % 16 from quarter l / 16 of
// the features.  kappa of every point pair goes to LDS (products across bins
// are formed and never read).  Bins of 4 or 8 points use the 4x4x4 form
// instead, which forms only products inside a bin.  Lane q then takes pair q of the tile: its
// pair-Gram column (the same expression as the tiles), the sigma recursion
// of its bin up to itself, its threshold, and the walk, one ballot per step
// for all the tile's bins together.
// ---------------------------------------------------------------------------
constexpr int kSmallN = 16;   // points per tile (and largest bin of the fused path)


// Eight features of one point kept raw (fp8: one 8-byte load, bf16: one
// 16-byte load, fp32: two) until their MFMAs, then widened one at a time.
template <int ET>
struct SmallRaw {
  u32x4_t w[ET == kF32 ? 2 : 1];
  __device__ __forceinline__ void load(const unsigned char* p) {
    if constexpr (ET == kFP8) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0][0] = x.x;
      w[0][1] = x.y;
    } else {
      w[0] = *reinterpret_cast<const u32x4_t*>(p);
    }
    if constexpr (ET == kF32) w[1] = *reinterpret_cast<const u32x4_t*>(p + 16);
  }
  __device__ __forceinline__ double operator[](int f) const {
    if constexpr (ET == kFP8) return static_cast<double>(fp8_byte_to_float(w[0][f >> 2], f & 3));
    else if constexpr (ET == kBF16) return static_cast<double>(__uint_as_float((f & 1) ? (w[0][f >> 1] & 0xffff0000u) : (w[0][f >> 1] << 16)));
    else return static_cast<double>(__uint_as_float(w[f >> 2][f & 3]));
  }
};
constexpr int kSmallBatch = 8;   // loads of eight features in flight per lane

// <x_i, x_j> over the F features of row `row` of every point: lane l takes
// the blocks of eight features 4 g + l / 16 of its point, one per load (F a
// multiple of 32; the four lanes of a point read 64 contiguous bytes).
// Loads go out kSmallBatch at a time before their MFMAs, and four
// accumulators keep four MFMAs in flight.
template <int ET>
__device__ __forceinline__ f64x4_t small_gram(const unsigned char* row, int F) {
  const int quarter = (threadIdx.x & 63) >> 4;
  const int elt = elt_size<ET>();
  const unsigned char* p = row + quarter * 8 * elt;   // lane quarter q: feature blocks 4 g + q of 8
  const int groups = F / 32;   // loads of eight features per lane
  f64x4_t acc[4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  for (int g0 = 0; g0 < groups; g0 += kSmallBatch) {
    SmallRaw<ET> x[kSmallBatch];
#pragma unroll
    for (int j = 0; j < kSmallBatch; ++j) x[j].load(p + min(g0 + j, groups - 1) * 32 * elt);   // (repeats are not used)
#pragma unroll
    for (int j = 0; j < kSmallBatch; ++j) {
      if (g0 + j >= groups) break;   // uniform
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const double v = x[j][f];
        acc[f & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64(v, v, acc[f & 3], 0, 0, 0);
      }
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Bins of 4 or 8 points on the fp64 MFMA 4x4x4 with four blocks (A[m][k] at
// lane 16 k + 4 b + m, B[k][n] at lane 16 k + 4 b + n, D[m][n] at lane
// 16 m + 4 b + n): lane l holds point l % 16 = 4 b + (l % 4) of the tile, so
// block b with A = B = that register is the 4 x 4 Gram of quad b (d0), and
// with B = the point of quad b ^ 1 (PAIR) the products of quads b and b ^ 1
// (d1).  Nothing is formed across bins.
template <int ET, bool PAIR>
__device__ __forceinline__ void small_gram44(const unsigned char* row, const unsigned char* prow, int F, double& d0,
                                             double& d1) {
  const int quarter = (threadIdx.x & 63) >> 4;
  const int elt = elt_size<ET>();
  const int off = quarter * 8 * elt;   // feature blocks 4 g + quarter of 8, as in small_gram
  const int groups = F / 32;
  constexpr int BATCH = PAIR ? kSmallBatch / 2 : kSmallBatch;
  double a0[2] = {0.0, 0.0}, a1[2] = {0.0, 0.0};
  for (int g0 = 0; g0 < groups; g0 += BATCH) {
    SmallRaw<ET> x[BATCH], y[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int gj = min(g0 + j, groups - 1);   // (repeats are not used)
      x[j].load(row + off + gj * 32 * elt);
      if constexpr (PAIR) y[j].load(prow + off + gj * 32 * elt);
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (g0 + j >= groups) break;   // uniform
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const double v = x[j][f];
        a0[f & 1] = __builtin_amdgcn_mfma_f64_4x4x4f64(v, v, a0[f & 1], 0, 0, 0);
        if constexpr (PAIR) a1[f & 1] = __builtin_amdgcn_mfma_f64_4x4x4f64(v, y[j][f], a1[f & 1], 0, 0, 0);
      }
    }
  }
  d0 = a0[0] + a0[1];
  d1 = a1[0] + a1[1];
}

template <int ET>
__global__ __launch_bounds__(256) void small_halving_kernel(GramLaunch g, SweepLaunch a) {
  __shared__ double s_kap[4][kSmallN][kSmallN + 1];   // kappa of the tile's point pairs, per wave
  const int N = g.N, P = N / 2;
  const int bpt = kSmallN / N;                        // whole bins per tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int units = g.nbins / g.bins_per_unit;
  const int tpu = (g.bins_per_unit + bpt - 1) / bpt;   // tiles per unit
  const int t = blockIdx.x * 4 + w;
  if (t >= units * tpu) return;   // whole wave: no barrier in this kernel
  const int unit = t / tpu, bin0 = (t % tpu) * bpt;
  const int b = unit / g.src.H_kv, h = unit % g.src.H_kv;

  // the row of point pt of the tile (points past the tile's bins read its first point)
  const int elt = elt_size<ET>();
  auto point_row = [&](int pt) -> int64_t {
    const int pb = pt / N;
    const bool ok = pb < bpt && bin0 + pb < g.bins_per_unit;
    const int tok = g.idx[static_cast<int64_t>(unit) * g.idx_unit_stride +
                          static_cast<int64_t>(ok ? bin0 + pb : bin0) * g.idx_stride + (ok ? pt % N : 0)];
    return (static_cast<int64_t>(b) * g.src.S + tok) * g.src.H_kv + h;
  };
  const unsigned char* K = static_cast<const unsigned char*>(g.src.k);
  const unsigned char* V = static_cast<const unsigned char*>(g.src.v);
  const int64_t row = point_row(lane & 15);
  if (N <= 8) {   // 4x4x4: the quad Grams (and, for 8 points, quad b against quad b ^ 1)
    const int m = lane >> 4, qb = (lane >> 2) & 3, n = lane & 3;
    double kd0, kd1, vd0, vd1;
    if (N == 8) {
      const int64_t prow = point_row((lane & 15) ^ 4);
      small_gram44<ET, true>(K + row * g.src.E * elt, K + prow * g.src.E * elt, g.src.E, kd0, kd1);
      small_gram44<ET, true>(V + row * g.src.D * elt, V + prow * g.src.D * elt, g.src.D, vd0, vd1);
      s_kap[w][4 * qb + m][4 * (qb ^ 1) + n] = exp_f64(g.scale * kd1) * (vd1 + 1.0);
    } else {
      small_gram44<ET, false>(K + row * g.src.E * elt, nullptr, g.src.E, kd0, kd1);
      small_gram44<ET, false>(V + row * g.src.D * elt, nullptr, g.src.D, vd0, vd1);
    }
    s_kap[w][4 * qb + m][4 * qb + n] = exp_f64(g.scale * kd0) * (vd0 + 1.0);
  } else {        // 16x16x4: every point pair of the tile
    const f64x4_t kd = small_gram<ET>(K + row * g.src.E * elt, g.src.E);
    const f64x4_t vd = small_gram<ET>(V + row * g.src.D * elt, g.src.D);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_kap[w][(lane >> 4) + 4 * i][lane & 15] = exp_f64(g.scale * kd[i]) * (vd[i] + 1.0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // lane q: pair i of bin bq of the tile
  const int bq = lane / P, i = lane % P;
  const bool mine = lane < bpt * P && bin0 + bq < g.bins_per_unit;
  const int lb = bin0 + (mine ? bq : 0);
  const int o = (mine ? bq : 0) * N;   // the bin's first point in the tile
  auto gpair = [&](int r, int c) -> double {   // pair-Gram entry (row pair r, column pair c) of the lane's bin
    const double* k0 = s_kap[w][o + 2 * r];
    const double* k1 = s_kap[w][o + 2 * r + 1];
    return (k0[o + 2 * c] - k0[o + 2 * c + 1]) - (k1[o + 2 * c] - k1[o + 2 * c + 1]);
  };
  double gcol[kSmallN / 2];
#pragma unroll
  for (int j = 0; j < kSmallN / 2; ++j) gcol[j] = (mine && j < i) ? gpair(j, i) : 0.0;
  // sigma recursion of the bin through pair i (the arithmetic of sigma_steps)
  const double c = sqrt(2.0 * log(2.0 * N / g.delta));
  const double k1 = 1.0 + 1.0 / (c * c), k2 = 2.0 / c;
  double s2 = 0.0, al = 0.0;
  for (int k = 0; k <= i; ++k) {
    const double b2 = fmax(gpair(k, k), 0.0), bk = sqrt(b2);
    const double cb = c * bk, b2k1 = b2 * k1, k2b = k2 * bk;
    const double sg = __builtin_amdgcn_sqrt(s2);
    const double bsc = cb * sg;
    const double grow = s2 + fmax(0.0, fma(-k2b, sg, b2k1));
    const double keep = fmax(s2, b2);
    al = fmax(bsc, b2);
    s2 = bsc >= b2 ? grow : keep;
  }
  const double u = mine ? philox_uniform(static_cast<uint64_t>(i), a.bin_base + lb, static_cast<uint64_t>(unit), a.tag,
                                         a.seed)
                        : 0.0;
  const double thr = step_threshold(a.greedy, al, u);
  double alpha = 0.0;
  uint32_t bits = 0;
  const int first_lane = lane - i;   // pair 0 of the lane's bin
#pragma unroll
  for (int j = 0; j < kSmallN / 2; ++j) {
    if (j >= P) continue;   // uniform
    const uint64_t m = __ballot(alpha < thr);
    const bool first = (m >> ((first_lane + j) & 63)) & 1ull;   // (lanes past the bins read any bit)
    bits |= static_cast<uint32_t>(first) << j;
    alpha += first ? gcol[j] : -gcol[j];
  }
  if (mine) {
    const bool first = (bits >> i) & 1u;
    const int z = unit * g.bins_per_unit + lb;
    const int32_t* in = a.idx_in + static_cast<int64_t>(unit) * a.in_unit_stride + static_cast<int64_t>(lb) * a.in_stride;
    a.idx_out[static_cast<int64_t>(z) * a.out_stride + i] = in[2 * i + (first ? 0 : 1)];
    if (a.row_out) a.row_out[static_cast<int64_t>(z) * a.out_stride + i] = kept_row(a, z, 2 * i + (first ? 0 : 1));
    if (a.dec) a.dec[static_cast<int64_t>(unit) * a.dec_per_unit + dec_offset(a, lb, P) + i] = first ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Bins of 20 to 32 points (a multiple of 4): one workgroup per bin.  The
// bin's rows go to LDS (one spare 16-byte piece per row spreads the operand
// reads over the banks); its point Gram is formed in 4 x 4 blocks of quads,
// the upper triangle of the quad grid, four blocks per fp64 MFMA 4x4x4 (block
// b of lane 16 k + 4 b + j: A = its row quad's point j, B = its column quad's
// point j), the blocks dealt round-robin to the waves; kappa goes to LDS for
// (i, j) and (j, i).  Wave 0 then runs the walk exactly as the small sweep.
// ---------------------------------------------------------------------------
constexpr int kMediumN = 32;   // (64-point bins ran faster on the tiles)

// Eight features at p (LDS), widened.
template <int ET>
__device__ __forceinline__ void medium_features(const lds_byte* p, double x[8]) {
  typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) const u32x2_t lds_u2;
  if constexpr (ET == kFP8) {
    const u32x2_t w = *reinterpret_cast<lds_u2*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = static_cast<double>(fp8_byte_to_float(w[0], j));
      x[4 + j] = static_cast<double>(fp8_byte_to_float(w[1], j));
    }
  } else if constexpr (ET == kBF16) {
    const u32x4_t w = *reinterpret_cast<lds_u4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = static_cast<double>(__uint_as_float(w[j] << 16));
      x[2 * j + 1] = static_cast<double>(__uint_as_float(w[j] & 0xffff0000u));
    }
  } else {
    const u32x4_t w0 = reinterpret_cast<lds_u4*>(p)[0], w1 = reinterpret_cast<lds_u4*>(p)[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = static_cast<double>(__uint_as_float(w0[j]));
      x[4 + j] = static_cast<double>(__uint_as_float(w1[j]));
    }
  }
}

template <int ET>
__global__ __launch_bounds__(256) void medium_halving_kernel(GramLaunch g, SweepLaunch a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_rows[];
  __shared__ double s_kap[kMediumN][kMediumN + 1];
  const int N = g.N, P = N / 2, Q = N / 4;
  const int z = blockIdx.x;
  const int unit = z / g.bins_per_unit, lb = z % g.bins_per_unit;
  const int b = unit / g.src.H_kv, h = unit % g.src.H_kv;
  const int elt = elt_size<ET>();
  const int KP = g.src.E * elt / 16, VP = g.src.D * elt / 16;   // 16-byte pieces of a K / V row
  const int RS = (KP + VP + 1) * 16;                            // staged row stride (bytes)
  lds_byte* rows = (lds_byte*)s_rows;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // the bin's rows into LDS, up to 16 pieces per thread in flight
  {
    const int32_t* list = g.idx + static_cast<int64_t>(unit) * g.idx_unit_stride + static_cast<int64_t>(lb) * g.idx_stride;
    const uint4* K = static_cast<const uint4*>(g.src.k);
    const uint4* V = static_cast<const uint4*>(g.src.v);
    const int pieces = N * (KP + VP);
    for (int x0 = 0; x0 < pieces; x0 += 16 * 256) {
      uint4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int x = min(x0 + 256 * i + tid, pieces - 1);
        const int pt = x / (KP + VP), c = x % (KP + VP);
        const int64_t row = (static_cast<int64_t>(b) * g.src.S + list[pt]) * g.src.H_kv + h;
        v[i] = c < KP ? K[row * KP + c] : V[row * VP + (c - KP)];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int x = x0 + 256 * i + tid;
        if (x < pieces) {
          const int pt = x / (KP + VP), c = x % (KP + VP);
          *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(rows + pt * RS + 16 * c) = u32x4_t{v[i].x, v[i].y, v[i].z, v[i].w};
        }
      }
    }
  }
  __syncthreads();

  // kappa of the upper quad blocks
  {
    const int nblk = Q * (Q + 1) / 2, ngroups = (nblk + 3) / 4;
    const int m = lane >> 4, beta = (lane >> 2) & 3, j = lane & 3;
    for (int gi = w; gi < ngroups; gi += 4) {
      const int blk = min(4 * gi + beta, nblk - 1);   // (spare blocks of the last group repeat the last one)
      int rq = 0, rem = blk;
      while (rem >= Q - rq) {
        rem -= Q - rq;
        ++rq;
      }
      const int cq = rq + rem;
      const lds_byte* pa = rows + (4 * rq + j) * RS + m * 8 * elt;   // feature blocks 4 t + m of eight
      const lds_byte* pb = rows + (4 * cq + j) * RS + m * 8 * elt;
      double kd[2] = {0.0, 0.0}, vd[2] = {0.0, 0.0};
      for (int t = 0; t < g.src.E / 32; ++t) {
        double xa[8], xb[8];
        medium_features<ET>(pa + t * 32 * elt, xa);
        medium_features<ET>(pb + t * 32 * elt, xb);
#pragma unroll
        for (int f = 0; f < 8; ++f) kd[f & 1] = __builtin_amdgcn_mfma_f64_4x4x4f64(xa[f], xb[f], kd[f & 1], 0, 0, 0);
      }
      for (int t = 0; t < g.src.D / 32; ++t) {
        double xa[8], xb[8];
        medium_features<ET>(pa + KP * 16 + t * 32 * elt, xa);
        medium_features<ET>(pb + KP * 16 + t * 32 * elt, xb);
#pragma unroll
        for (int f = 0; f < 8; ++f) vd[f & 1] = __builtin_amdgcn_mfma_f64_4x4x4f64(xa[f], xb[f], vd[f & 1], 0, 0, 0);
      }
      // D[m][n] of block beta sits in lane 16 m + 4 beta + n: points (4 rq + m, 4 cq + n)
      const double kap = exp_f64(g.scale * (kd[0] + kd[1])) * ((vd[0] + vd[1]) + 1.0);
      if (4 * gi + beta < nblk) {
        s_kap[4 * rq + m][4 * cq + j] = kap;
        s_kap[4 * cq + j][4 * rq + m] = kap;
      }
    }
  }
  __syncthreads();
  if (w != 0) return;   // the walk: one wave

  auto gpair = [&](int r, int c) -> double {   // pair-Gram entry (row pair r, column pair c)
    return (s_kap[2 * r][2 * c] - s_kap[2 * r][2 * c + 1]) - (s_kap[2 * r + 1][2 * c] - s_kap[2 * r + 1][2 * c + 1]);
  };
  const bool mine = lane < P;
  double gc[kMediumN / 2];
#pragma unroll
  for (int j = 0; j < kMediumN / 2; ++j) gc[j] = (mine && j < lane) ? gpair(j, lane) : 0.0;
  const double u = mine ? philox_uniform(static_cast<uint64_t>(lane), a.bin_base + lb, static_cast<uint64_t>(unit),
                                         a.tag, a.seed)
                        : 0.0;
  const double b2 = mine ? fmax(gpair(lane, lane), 0.0) : 0.0;
  const double c = sqrt(2.0 * log(2.0 * a.N / a.delta));
  double s2 = 0.0;
  const double thr =
      step_threshold(a.greedy, sigma_steps(s2, b2, sqrt(b2), P, c, 1.0 + 1.0 / (c * c), 2.0 / c), u);
  double alpha = 0.0;
  uint64_t bits = 0;
#pragma unroll
  for (int j = 0; j < kMediumN / 2; ++j) {
    if (j >= P) continue;   // uniform
    const uint64_t mb = __ballot(alpha < thr);
    const bool first = (mb >> j) & 1ull;
    bits |= static_cast<uint64_t>(first) << j;
    alpha += first ? gc[j] : -gc[j];
  }
  if (mine) {
    const bool first = (bits >> lane) & 1ull;
    const int32_t* in = a.idx_in + static_cast<int64_t>(unit) * a.in_unit_stride + static_cast<int64_t>(lb) * a.in_stride;
    a.idx_out[static_cast<int64_t>(z) * a.out_stride + lane] = in[2 * lane + (first ? 0 : 1)];
    if (a.row_out) a.row_out[static_cast<int64_t>(z) * a.out_stride + lane] = kept_row(a, z, 2 * lane + (first ? 0 : 1));
    if (a.dec) a.dec[static_cast<int64_t>(unit) * a.dec_per_unit + dec_offset(a, lb, P) + lane] = first ? 1 : 0;
  }
}

inline unsigned grid1d(int64_t n, int block) { return static_cast<unsigned>((n + block - 1) / block); }

}  // namespace

hipError_t launch_pair_gram(const GramLaunch& a, hipStream_t s) {
  if (gram8_runs(a)) return launch_pair_gram8(a, s);
  const int P = a.N / 2;
  int64_t blocks;
  if (P < 32 && (32 % P) == 0) {
    blocks = static_cast<int64_t>(a.nbins / a.bins_per_unit) * ((a.bins_per_unit * P + 31) / 32);
  } else {
    const int nt = (P + 31) / 32;
    blocks = static_cast<int64_t>(nt) * (nt + 1) / 2 * a.nbins;
  }
  if (blocks == 0) return hipSuccess;
  int nthr, per_wave;
  threshold_groups(a, nthr, per_wave);
  dim3 grid(static_cast<unsigned>(blocks + nthr));
  if (a.src.dtype == kFP8)
    hipLaunchKernelGGL(pair_gram_kernel<kFP8>, grid, dim3(256), 0, s, a, nthr, per_wave);
  else if (a.src.dtype == kBF16)
    hipLaunchKernelGGL(pair_gram_kernel<kBF16>, grid, dim3(256), 0, s, a, nthr, per_wave);
  else
    hipLaunchKernelGGL(pair_gram_kernel<kF32>, grid, dim3(256), 0, s, a, nthr, per_wave);
  return hipGetLastError();
}

size_t sweep_lds_bytes(int N) { return (3 * static_cast<size_t>(N / 2) + 2 * 64 * 65) * sizeof(double); }

hipError_t launch_halving_sweep(const SweepLaunch& a, hipStream_t s, hipEvent_t done) {
  if (a.N / 2 <= 16) {
    launch_signal(halving_sweep_small_kernel<16>, dim3((a.nbins + 3) / 4), dim3(256), 0, s, done, a);
    return hipGetLastError();
  }
  if (a.N / 2 <= 64) {
    launch_signal(halving_sweep_small_kernel<64>, dim3((a.nbins + 3) / 4), dim3(256), 0, s, done, a);
    return hipGetLastError();
  }
  const size_t lds = sweep_lds_bytes(a.N);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(halving_sweep_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  launch_signal(halving_sweep_kernel, dim3(a.nbins), dim3(256), static_cast<uint32_t>(lds), s, done, a);
  return hipGetLastError();
}

bool small_halving_supported(int N, int E, int D) {
  return N >= 2 && N <= kSmallN && N % 2 == 0 && E % 32 == 0 && D % 32 == 0;
}

hipError_t launch_small_halving(const GramLaunch& g, const SweepLaunch& a, hipStream_t s) {
  if (!small_halving_supported(g.N, g.src.E, g.src.D) || g.N != a.N || g.nbins != a.nbins ||
      g.bins_per_unit != a.bins_per_unit)
    return hipErrorInvalidValue;
  if (g.nbins == 0) return hipSuccess;
  const int bpt = kSmallN / g.N;
  const int64_t waves = static_cast<int64_t>(g.nbins / g.bins_per_unit) * ((g.bins_per_unit + bpt - 1) / bpt);
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
  if (g.src.dtype == kFP8)
    hipLaunchKernelGGL(small_halving_kernel<kFP8>, grid, dim3(256), 0, s, g, a);
  else if (g.src.dtype == kBF16)
    hipLaunchKernelGGL(small_halving_kernel<kBF16>, grid, dim3(256), 0, s, g, a);
  else
    hipLaunchKernelGGL(small_halving_kernel<kF32>, grid, dim3(256), 0, s, g, a);
  return hipGetLastError();
}

static size_t medium_rows_lds(int N, int E, int D, int dtype) {
  const int elt = dtype == kF32 ? 4 : (dtype == kBF16 ? 2 : 1);
  return static_cast<size_t>(N) * ((E + D) * elt + 16);
}

bool medium_halving_supported(int N, int E, int D, int dtype) {
  return N > kSmallN && N <= kMediumN && N % 4 == 0 && E % 32 == 0 && D % 32 == 0 &&
         medium_rows_lds(N, E, D, dtype) <= 96 * 1024;
}

hipError_t launch_medium_halving(const GramLaunch& g, const SweepLaunch& a, hipStream_t s) {
  if (!medium_halving_supported(g.N, g.src.E, g.src.D, g.src.dtype) || g.N != a.N || g.nbins != a.nbins ||
      g.bins_per_unit != a.bins_per_unit)
    return hipErrorInvalidValue;
  if (g.nbins == 0) return hipSuccess;
  const size_t lds = medium_rows_lds(g.N, g.src.E, g.src.D, g.src.dtype);
  const void* fn = g.src.dtype == kFP8 ? reinterpret_cast<const void*>(medium_halving_kernel<kFP8>)
                   : g.src.dtype == kBF16 ? reinterpret_cast<const void*>(medium_halving_kernel<kBF16>)
                                          : reinterpret_cast<const void*>(medium_halving_kernel<kF32>);
  if (lds > 64 * 1024) {
    static bool set[64][3];   // once per device and element type (for the largest size)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!set[dev][g.src.dtype]) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
      if (e != hipSuccess) return e;
      set[dev][g.src.dtype] = true;
    }
  }
  if (g.src.dtype == kFP8)
    hipLaunchKernelGGL(medium_halving_kernel<kFP8>, dim3(g.nbins), dim3(256), lds, s, g, a);
  else if (g.src.dtype == kBF16)
    hipLaunchKernelGGL(medium_halving_kernel<kBF16>, dim3(g.nbins), dim3(256), lds, s, g, a);
  else
    hipLaunchKernelGGL(medium_halving_kernel<kF32>, dim3(g.nbins), dim3(256), lds, s, g, a);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* out, int64_t units, int64_t n, int64_t stride, hipStream_t s) {
  if (units * n == 0) return hipSuccess;
  hipLaunchKernelGGL(iota_kernel, dim3(grid1d(units * n, 256)), dim3(256), 0, s, out, units, n, stride);
  return hipGetLastError();
}

hipError_t launch_base_sample(const int32_t* list, int64_t L, int units, int64_t r, uint64_t seed, int32_t* out,
                              hipStream_t s) {
  const int64_t total = static_cast<int64_t>(units) * (L / r);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(base_sample_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, list, L, units, r, seed, out);
  return hipGetLastError();
}

hipError_t launch_express_reps(const ExpressView& ev, int units, uint64_t seed, int32_t* reps, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(units) * ev.n_batches_alloc * 2 * ev.n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(express_reps_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, ev, units, seed, reps);
  return hipGetLastError();
}

hipError_t launch_halve_input(const ExpressView& ev, int units, int e, int32_t* halve_in, hipStream_t s,
                              const HalveRows& rows) {
  const int64_t total = static_cast<int64_t>(units) * 4 * ev.n;
  hipLaunchKernelGGL(halve_input_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, ev, units, e, halve_in, rows);
  return hipGetLastError();
}

hipError_t launch_express_final(const ExpressView& ev, int units, int S, int32_t* idx, float* w, int32_t* len,
                                int64_t cap, hipStream_t s) {
  if (!idx && !w && !len) return hipSuccess;
  hipLaunchKernelGGL(express_final_kernel, dim3(units), dim3(256), 0, s, ev, units, S, idx, w, len, cap);
  return hipGetLastError();
}

hipError_t launch_fill_coreset(const int32_t* src, int64_t src_stride, int units, int n, float w, int32_t* idx,
                               float* wout, int32_t* len, hipStream_t s) {
  if (!idx && !wout && !len) return hipSuccess;
  const int64_t total = static_cast<int64_t>(units) * n;
  hipLaunchKernelGGL(fill_coreset_kernel, dim3(grid1d(total, 256)), dim3(256), 0, s, src, src_stride, units, n, w,
                     idx, wout, len);
  return hipGetLastError();
}

hipError_t launch_sanitize_indices(const int32_t* in, int64_t n, int32_t S, int32_t* out, int* err, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sanitize_indices_kernel, dim3(grid1d(n, 256)), dim3(256), 0, s, in, n, S, out, err);
  return hipGetLastError();
}

hipError_t launch_philox_words(const uint64_t* ctr, int64_t n, uint64_t seed, uint64_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(philox_words_kernel, dim3(grid1d(n, 256)), dim3(256), 0, s, ctr, n, seed, out);
  return hipGetLastError();
}

ExpressSchedule express_schedule(int64_t S, int n) {
  ExpressSchedule sc{};
  sc.n = n;
  sc.nblk = static_cast<int>(S / n);
  // HALVE e happens after 4^(e+1) blocks; epoch e >= 1 holds three batches of 4^e blocks.
  int halves = 0;
  while ((1LL << (2 * (halves + 1))) <= sc.nblk) ++halves;
  sc.n_halves = halves;
  int done = 0, alloc = 0;
  for (int e = 1;; ++e) {
    const int64_t m = 1LL << (2 * e);
    const int64_t epoch_start = m;            // blocks
    if (epoch_start >= sc.nblk) break;
    for (int j = 0; j < 3; ++j) {
      const int64_t bstart = epoch_start + j * m;
      if (bstart < sc.nblk) ++alloc;
      if (bstart + m <= sc.nblk) ++done;
    }
  }
  sc.n_batches_done = done;
  sc.n_batches_alloc = alloc;
  sc.decisions = static_cast<int64_t>(3) * n * halves + static_cast<int64_t>(n) * done;
  return sc;
}

}  // namespace thin
