// Weighted-coreset softmax attention on gfx950 (MFMA for Q K^T and P V only).
//
// out(q) = sum_j w_j exp(s <q, k_j>) v_j / sum_j w_j exp(s <q, k_j>) over the
// keys a query sees ("Express Language Modeling": attention against a small
// weighted summary of the keys and values).  ln w_j is folded into the
// logit, the softmax is taken online (running maximum and sum), and the
// accumulation is fp32.
//
// A query sees a list of segments.  A segment is either a list of token
// indices (a coreset, the EXPRESS cache or buffer) with one log-weight or
// per-point weights, or a raw token range with weight 1 and, for the block
// being streamed, a causal mask.  Unmasked attention uses one segment per
// unit; Thinformer Express uses the cache / buffer segments of the state
// before the query's block plus the raw causal block.
//
// Layout: one workgroup = 4 waves x 16 queries of one (b, h); keys are
// staged 32 at a time in LDS (K row-major, V transposed for bf16).  The
// products are computed transposed: S^T = K Q^T puts one query per lane
// column (lane % 16), so the softmax statistics and the O^T = V^T P^T
// accumulator of a query live in the same lanes and rescaling needs no lane
// exchange.

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace thin {

namespace {

constexpr int kQT = 64;   // queries per workgroup
constexpr int kKC = 32;   // keys per LDS chunk
constexpr float kLog2e = 1.4426950408889634f;

struct Seg {
  const int32_t* idx;   // nullptr: raw token range
  int start;            // first entry of idx, or first token of the range
  int count;
  float lnw2;           // log2 of the weight when w == nullptr
  const float* w;       // per-point weights (indexed like idx), or nullptr
  int causal;           // raw range streamed causally: key visible iff key <= query
};

template <bool BF16, int E, int D>
struct Smem;

template <int E, int D>
struct Smem<true, E, D> {
  uint16_t k[kKC][E + 8];
  uint16_t vt[D][40];          // V^T, key slots permuted to the P^T operand order
  float lnw2[kKC];
  int pos[kKC];
};

template <int E, int D>
struct Smem<false, E, D> {
  float k[kKC][E + 4];
  float v[kKC][D + 4];
  float lnw2[kKC];
  int pos[kKC];
};

// key kk of a 32-key chunk -> its slot in the bf16 P^T / V^T operands:
// lane group g holds keys 4g..4g+3 of each 16-key half as slots 8g..8g+7.
__device__ __forceinline__ int bf16_slot(int kk) { return 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3); }

template <bool BF16, int E, int D>
struct Attn {
  static constexpr int NQ = BF16 ? E / 32 : E / 4;   // Q fragments per lane
  static constexpr int ND = D / 16;                  // output blocks of 16 dims

  using QFrag = typename std::conditional<BF16, bf16x8_t, float>::type;

  const AttnLaunch& a;
  Smem<BF16, E, D>& sm;
  int b, h, hk, unit;
  int lane, g, qr;   // my query row (token index)
  bool row_live;
  QFrag qf[NQ];
  f32x4_t o[ND];
  float m_run, l_run;

  __device__ Attn(const AttnLaunch& la, Smem<BF16, E, D>& s, int q0, int bh) : a(la), sm(s) {
    b = bh / a.H;
    h = bh % a.H;
    hk = h / (a.H / a.H_kv);
    unit = b * a.H_kv + hk;
    lane = threadIdx.x & 63;
    g = lane >> 4;
    qr = q0 + 16 * (threadIdx.x >> 6) + (lane & 15);
    row_live = qr < a.T;
    const int64_t qrow = ((static_cast<int64_t>(b) * a.T + (row_live ? qr : 0)) * a.H + h) * E;
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      if constexpr (BF16) {
        const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(static_cast<const uint16_t*>(a.q) + qrow + kk * 32 + 8 * g);
        qf[kk] = row_live ? *src : bf16x8_t{};
      } else {
        qf[kk] = row_live ? static_cast<const float*>(a.q)[qrow + kk * 4 + g] : 0.0f;
      }
    }
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }

  __device__ __forceinline__ int key_token(const Seg& s, int j) const { return s.idx ? s.idx[s.start + j] : s.start + j; }

  // A chunk of 32 keys travels global -> registers -> LDS, so that the next
  // chunk's loads are in flight while the current one is consumed.
  static constexpr int KPT = BF16 ? (kKC * E / 8 + 255) / 256 : (kKC * E / 4 + 255) / 256;   // 16-byte pieces / thread
  static constexpr int VPT = BF16 ? (kKC * D / 8 + 255) / 256 : (kKC * D / 4 + 255) / 256;
  struct Chunk {
    uint4 k[KPT];
    uint4 v[VPT];
    int pos;
    float l2;
  };

  __device__ __forceinline__ void load(const Seg& s, int c0, int nk, Chunk& ch) const {
    const int tid = threadIdx.x;
    const int64_t kv_base = static_cast<int64_t>(b) * a.S;
    constexpr int KP = BF16 ? E / 8 : E / 4;
    constexpr int VP = BF16 ? D / 8 : D / 4;
    constexpr int ELT = BF16 ? 2 : 4;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = tid + 256 * j;
      const int r = p / KP, c = p % KP;
      ch.k[j] = uint4{0, 0, 0, 0};
      if (p < kKC * KP && r < nk) {
        const int64_t row = (kv_base + key_token(s, c0 + r)) * a.H_kv + hk;
        ch.k[j] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k) + (row * E + c * (16 / ELT)) * ELT);
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int p = tid + 256 * j;
      const int r = p / VP, c = p % VP;
      ch.v[j] = uint4{0, 0, 0, 0};
      if (p < kKC * VP && r < nk) {
        const int64_t row = (kv_base + key_token(s, c0 + r)) * a.H_kv + hk;
        ch.v[j] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v) + (row * D + c * (16 / ELT)) * ELT);
      }
    }
    ch.pos = 0x7fffffff;
    ch.l2 = -INFINITY;
    if (tid < kKC && tid < nk) {
      ch.pos = key_token(s, c0 + tid);
      ch.l2 = s.w ? log2f(s.w[s.start + c0 + tid]) : s.lnw2;
    }
  }

  __device__ __forceinline__ void store(const Chunk& ch) {
    const int tid = threadIdx.x;
    constexpr int KP = BF16 ? E / 8 : E / 4;
    constexpr int VP = BF16 ? D / 8 : D / 4;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = tid + 256 * j;
      if (p >= kKC * KP) break;
      const int r = p / KP, c = p % KP;
      if constexpr (BF16)
        *reinterpret_cast<uint4*>(&sm.k[r][c * 8]) = ch.k[j];
      else
        *reinterpret_cast<uint4*>(&sm.k[r][c * 4]) = ch.k[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int p = tid + 256 * j;
      if (p >= kKC * VP) break;
      const int r = p / VP, c = p % VP;
      if constexpr (BF16) {
        const int slot = bf16_slot(r);
        const uint32_t wv[4] = {ch.v[j].x, ch.v[j].y, ch.v[j].z, ch.v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sm.vt[c * 8 + 2 * q][slot] = static_cast<uint16_t>(wv[q] & 0xffffu);
          sm.vt[c * 8 + 2 * q + 1][slot] = static_cast<uint16_t>(wv[q] >> 16);
        }
      } else {
        *reinterpret_cast<uint4*>(&sm.v[r][c * 4]) = ch.v[j];
      }
    }
    if (tid < kKC) {
      sm.pos[tid] = ch.pos;
      sm.lnw2[tid] = ch.l2;
    }
  }

  // One chunk of 32 staged keys for this wave's 16 queries.
  __device__ void consume(const Seg& s, bool row_ok) {
    f32x4_t st[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) {
        if constexpr (BF16) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&sm.k[c * 16 + (lane & 15)][kk * 32 + 8 * g]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], acc, 0, 0, 0);
        } else {
          const float kf = sm.k[c * 16 + (lane & 15)][kk * 4 + g];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf, qf[kk], acc, 0, 0, 0);
        }
      }
      st[c] = acc;
    }
    // logits (base 2), masks
    const float sc = a.scale * kLog2e;
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = c * 16 + 4 * g + i;
        const bool vis = row_ok && (!s.causal || sm.pos[kk] <= qr);
        const float l2 = sm.lnw2[kk];
        const float val = vis ? st[c][i] * sc + l2 : -INFINITY;
        x[c][i] = val;
        mx = fmaxf(mx, val);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[2][4];
    float rs = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[c][i] = __builtin_amdgcn_exp2f(x[c][i] - m_use);
        rs += p[c][i];
      }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] *= alpha;
    if constexpr (BF16) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<__bf16>(p[0][i]);
        pb[4 + i] = static_cast<__bf16>(p[1][i]);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(&sm.vt[16 * d + (lane & 15)][8 * g]);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[d], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const float vf = sm.v[c * 16 + 4 * g + i][16 * d + (lane & 15)];
            o[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, p[c][i], o[d], 0, 0, 0);
          }
    }
  }

  __device__ void run_segment(const Seg s, bool row_ok) {
    if (s.count <= 0) return;
    Chunk ch;
    load(s, 0, min(kKC, s.count), ch);
    for (int c0 = 0; c0 < s.count; c0 += kKC) {
      store(ch);
      __syncthreads();
      if (c0 + kKC < s.count) load(s, c0 + kKC, min(kKC, s.count - c0 - kKC), ch);
      consume(s, row_ok);
      __syncthreads();
    }
  }

  __device__ void store() {
    if (!row_live) return;
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    const int64_t orow = ((static_cast<int64_t>(b) * a.T + qr) * a.H + h) * D;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int col = 16 * d + 4 * g;
      if constexpr (BF16) {
        uint16_t* dst = static_cast<uint16_t*>(a.out) + orow + col;
        const uint32_t lo = float_to_bf16_bits(o[d][0] * inv) | (static_cast<uint32_t>(float_to_bf16_bits(o[d][1] * inv)) << 16);
        const uint32_t hi = float_to_bf16_bits(o[d][2] * inv) | (static_cast<uint32_t>(float_to_bf16_bits(o[d][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
      } else {
        float* dst = static_cast<float*>(a.out) + orow + col;
        *reinterpret_cast<float4*>(dst) = float4{o[d][0] * inv, o[d][1] * inv, o[d][2] * inv, o[d][3] * inv};
      }
    }
  }
};

// Attend to the Express state after beta blocks, then to the raw causal block.
// Segments: HALVE output (weight m), completed batches of the epoch (m),
// representatives of the current batch (m / 2), raw tokens (1, causal).
template <class A>
__device__ void express_block(A& at, const ExpressView& ev, int beta, int S, int key_end, bool row_ok) {
  const int unit = at.unit;
  if (beta < 4) {   // exact phase: every earlier token and the block itself, weight 1
    at.run_segment(Seg{nullptr, 0, min(key_end, S), 0.f, nullptr, 1}, row_ok);
    return;
  }
  int E = 1;
  while ((1LL << (2 * (E + 1))) <= beta) ++E;
  const int m = 1 << (2 * E);
  const int since = beta - m;
  const int nbc = since / m;
  const int rem = since % m;
  const float lm = static_cast<float>(2 * E);        // log2 m
  at.run_segment(Seg{ev.halve_out + (static_cast<int64_t>(unit) * ev.n_halves + (E - 1)) * ev.n, 0, ev.n, lm,
                     nullptr, 0},
                 row_ok);
  if (nbc > 0)
    at.run_segment(Seg{ev.batch_out + (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (E - 1)) * ev.n, 0,
                       nbc * ev.n, lm, nullptr, 0},
                   row_ok);
  const int n_rep = static_cast<int>((static_cast<int64_t>(rem) * 2 * ev.n) / m);
  if (n_rep > 0)
    at.run_segment(Seg{ev.reps + (static_cast<int64_t>(unit) * ev.n_batches_alloc + 3 * (E - 1) + nbc) * 2 * ev.n, 0,
                       n_rep, lm - 1.0f, nullptr, 0},
                   row_ok);
  const int bn = beta * ev.n;
  at.run_segment(Seg{nullptr, bn, min(key_end, S) - bn, 0.f, nullptr, 1}, row_ok);
}

template <bool BF16, int E, int D>
__global__ __launch_bounds__(256) void seg_attention_kernel(AttnLaunch a) {
  __shared__ Smem<BF16, E, D> sm;
  const int64_t tile = xcd_remap(blockIdx.y * static_cast<int64_t>(gridDim.x) + blockIdx.x,
                                 static_cast<int64_t>(gridDim.x) * gridDim.y);
  const int q0 = static_cast<int>(tile % gridDim.x) * kQT;
  const int bh = static_cast<int>(tile / gridDim.x);
  Attn<BF16, E, D> at(a, sm, q0, bh);
  if (!a.causal) {
    const int b = bh / a.H, hk = (bh % a.H) / (a.H / a.H_kv);
    const int unit = b * a.H_kv + hk;
    if (a.cs_idx)
      at.run_segment(Seg{a.cs_idx + unit * a.cs_stride, 0, a.cs_n, a.cs_lnw * kLog2e,
                         a.cs_w ? a.cs_w + unit * a.cs_stride : nullptr, 0},
                     true);
    else
      at.run_segment(Seg{nullptr, 0, a.S, a.cs_lnw * kLog2e, nullptr, 0}, true);
  } else {
    const int n = a.ev.n;
    const int q_last = min(q0 + kQT - 1, a.T - 1);
    const int beta_lo = q0 / n, beta_hi = q_last / n;
    for (int beta = beta_lo; beta <= beta_hi; ++beta) {
      const int key_end = min(q_last + 1, (beta + 1) * n);
      express_block(at, a.ev, beta, a.S, key_end, (at.qr / n) == beta);
    }
  }
  at.store();
}

template <bool BF16, int E, int D>
hipError_t launch_one(const AttnLaunch& a, hipStream_t s) {
  dim3 grid((a.T + kQT - 1) / kQT, a.B * a.H);
  hipLaunchKernelGGL((seg_attention_kernel<BF16, E, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int bf16, int E, int D) {
  if (bf16) return (E == 64 && (D == 64 || D == 128 || D == 256)) || (E == 128 && (D == 128 || D == 64));
  return (E == 64 && (D == 64 || D == 128)) || (E == 128 && D == 128);
}

hipError_t launch_attention(const AttnLaunch& a, int bf16, int E, int D, hipStream_t s) {
  if (a.T == 0 || a.B * a.H == 0) return hipSuccess;
  if (bf16) {
    return launch_attention_bf16(a, E, D, s);
  } else {
    if (E == 64 && D == 64) return launch_one<false, 64, 64>(a, s);
    if (E == 64 && D == 128) return launch_one<false, 64, 128>(a, s);
    if (E == 128 && D == 128) return launch_one<false, 128, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace thin
