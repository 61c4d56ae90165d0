// Weighted-coreset / Express attention for bfloat16 inputs on gfx950.
//
// Same definition as the fp32 kernel (attn.hip): for every query the
// visible keys form segments (coreset or cache / buffer index lists with a
// log-weight, raw token ranges with weight 1, the block being streamed with a
// causal mask); out = sum w e^{s<q,k>} v / sum w e^{s<q,k>}, ln w folded into
// the logit, online softmax, fp32 accumulation, MFMA for Q K^T and P V.
//
// Layout for bf16 (MFMA v_mfma_f32_16x16x32_bf16):
//  * one workgroup = 8 waves x 16 queries of one (b, h), all sharing each
//    staged key chunk;
//  * keys are staged 64 at a time in LDS, K and V both row-major (16-byte
//    global loads and LDS writes); the next chunk is loaded into registers
//    while the current one is consumed;
//  * the V operand of P V is read with the gfx950 transposing LDS read
//    (ds_read_tr16_b64): within each 16-lane group, lane j receives element
//    j % 4 of the 8-byte pieces addressed by lanes j/4 + 4k (k = 0..3), so
//    lanes addressing V[k0 + i/4][d0 + 4 (i % 4)] deliver V[k0..k0+3][d0 + j]
//    to lane j: four keys of one dimension, as the MFMA operand wants;
//  * the index list of a gathered segment is staged in LDS once, so chunk
//    loads never wait on a dependent global index read;
//  * S^T = K Q^T keeps one query per lane column, so softmax statistics and
//    the O^T = V^T P^T accumulator of a query share lanes.

#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace thin {

namespace {

constexpr int kQ = 128;       // queries per workgroup
constexpr int kThreads = 512; // 8 waves x 16 queries
constexpr int NQG = 1;        // 16-query groups per wave
constexpr int kC = 64;        // keys per chunk
constexpr int kIdxCap = 1024; // index entries staged per pass
constexpr float kLog2eB = 1.4426950408889634f;

struct SegB {
  const int32_t* idx;   // nullptr: raw token range
  int start;
  int count;
  float lnw2;
  const float* w;
  int causal;
};

template <int E, int D>
struct SmemB {
  uint16_t k[kC][E + 8];
  uint16_t v[kC][D + 16];      // row stride D + 16 keeps the transposing reads conflict-free
  float lnw2[kC];
  int pos[kC];
  int idx[kIdxCap];
};

template <int E, int D>
struct AttnB {
  static constexpr int NK = E / 32;   // k-steps of Q K^T
  static constexpr int ND = D / 16;   // 16-dim output blocks
  static constexpr int KPT = kC * E / 8 / kThreads;   // 16-byte pieces per thread
  static constexpr int VPT = kC * D / 8 / kThreads;

  const AttnLaunch& a;
  SmemB<E, D>& sm;
  int b, h, hk, unit, lane, g;
  int qr[NQG];
  bool live[NQG];
  bf16x8_t qf[NQG][NK];
  f32x4_t o[NQG][ND];
  float m_run[NQG], l_run[NQG];

  struct Chunk {
    uint4 k[KPT];
    uint4 v[VPT];
    int pos;
    float l2;
  };

  __device__ AttnB(const AttnLaunch& la, SmemB<E, D>& s, int q0, int bh) : a(la), sm(s) {
    b = bh / a.H;
    h = bh % a.H;
    hk = h / (a.H / a.H_kv);
    unit = b * a.H_kv + hk;
    lane = threadIdx.x & 63;
    g = lane >> 4;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      qr[qg] = q0 + 16 * NQG * w + 16 * qg + (lane & 15);
      live[qg] = qr[qg] < a.T;
      const int64_t qrow = ((static_cast<int64_t>(b) * a.T + (live[qg] ? qr[qg] : 0)) * a.H + h) * E;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(static_cast<const uint16_t*>(a.q) + qrow + kk * 32 + 8 * g);
        qf[qg][kk] = live[qg] ? *src : bf16x8_t{};
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) o[qg][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_run[qg] = -INFINITY;
      l_run[qg] = 0.f;
    }
  }

  __device__ __forceinline__ int token(const SegB& s, int base, int j) const {
    return s.idx ? sm.idx[j] : s.start + base + j;
  }

  __device__ __forceinline__ void load(const SegB& s, int base, int c0, int nk, Chunk& ch) const {
    const int tid = threadIdx.x;
    const int64_t kv_base = static_cast<int64_t>(b) * a.S;
    constexpr int KP = E / 8;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = tid + kThreads * j;
      const int r = p / KP, c = p % KP;
      ch.k[j] = uint4{0, 0, 0, 0};
      if (r < nk) {
        const int64_t row = (kv_base + token(s, base, c0 + r)) * a.H_kv + hk;
        ch.k[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + row * E + c * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int p = tid + kThreads * j;
      const int r = p / (D / 8), c = p % (D / 8);
      ch.v[j] = uint4{0, 0, 0, 0};
      if (r < nk) {
        const int64_t row = (kv_base + token(s, base, c0 + r)) * a.H_kv + hk;
        ch.v[j] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + row * D + c * 8);
      }
    }
    ch.pos = 0x7fffffff;
    ch.l2 = -INFINITY;
    if (tid < kC && tid < nk) {
      ch.pos = token(s, base, c0 + tid);
      ch.l2 = s.w ? log2f(s.w[s.start + base + c0 + tid]) : s.lnw2;
    }
  }

  __device__ __forceinline__ void store(const Chunk& ch) {
    const int tid = threadIdx.x;
    constexpr int KP = E / 8;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = tid + kThreads * j;
      const int r = p / KP, c = p % KP;
      *reinterpret_cast<uint4*>(&sm.k[r][c * 8]) = ch.k[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int p = tid + kThreads * j;
      const int r = p / (D / 8), c = p % (D / 8);
      *reinterpret_cast<uint4*>(&sm.v[r][c * 8]) = ch.v[j];
    }
    if (tid < kC) {
      sm.pos[tid] = ch.pos;
      sm.lnw2[tid] = ch.l2;
    }
  }

  __device__ void consume(const SegB& s, const bool row_ok[NQG]) {
    f32x4_t st[NQG][4];
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) st[qg][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&sm.k[kb * 16 + (lane & 15)][kk * 32 + 8 * g]);
#pragma unroll
        for (int qg = 0; qg < NQG; ++qg)
          st[qg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qg][kk], st[qg][kb], 0, 0, 0);
      }
    const float sc = a.scale * kLog2eB;
    bf16x8_t pb[NQG][2];
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      float x[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kb * 16 + 4 * g + i;
          const bool vis = row_ok[qg] && (!s.causal || sm.pos[kk] <= qr[qg]);
          const float val = vis ? st[qg][kb][i] * sc + sm.lnw2[kk] : -INFINITY;
          x[kb][i] = val;
          mx = fmaxf(mx, val);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[qg], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qg] - m_use);
      float rs = 0.f;
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(x[kb][i] - m_use);
          rs += p[kb][i];
        }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run[qg] = l_run[qg] * alpha + rs;
      m_run[qg] = m_new;
#pragma unroll
      for (int d = 0; d < ND; ++d) o[qg][d] *= alpha;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[qg][hh][i] = static_cast<__bf16>(p[2 * hh][i]);
          pb[qg][hh][4 + i] = static_cast<__bf16>(p[2 * hh + 1][i]);
        }
    }
    // O^T += V^T P^T: lane group g's operand slots 0-3 / 4-7 are keys
    // 32hh + 4g + (0..3) and 32hh + 16 + 4g + (0..3) (the S^T layout)
    const int i16 = lane & 15;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)&sm.v[32 * hh + 4 * g + (i16 >> 2)][16 * d + 4 * (i16 & 3)]);
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)&sm.v[32 * hh + 16 + 4 * g + (i16 >> 2)][16 * d + 4 * (i16 & 3)]);
        const bf16x8_t vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qg = 0; qg < NQG; ++qg)
          o[qg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[qg][hh], o[qg][d], 0, 0, 0);
      }
  }

  __device__ void run_segment(const SegB s, const bool row_ok[NQG]) {
    for (int base = 0; base < s.count; base += kIdxCap) {
      const int cnt = min(kIdxCap, s.count - base);
      if (s.idx) {
        __syncthreads();
        for (int j = threadIdx.x; j < cnt; j += kThreads) sm.idx[j] = s.idx[s.start + base + j];
        __syncthreads();
      }
      Chunk ch;
      load(s, base, 0, min(kC, cnt), ch);
      for (int c0 = 0; c0 < cnt; c0 += kC) {
        __syncthreads();
        store(ch);
        __syncthreads();
        if (c0 + kC < cnt) load(s, base, c0 + kC, min(kC, cnt - c0 - kC), ch);
        consume(s, row_ok);
      }
    }
  }

  __device__ void finish() {
#pragma unroll
    for (int qg = 0; qg < NQG; ++qg) {
      if (!live[qg]) continue;
      const float inv = l_run[qg] > 0.f ? 1.0f / l_run[qg] : 0.f;
      const int64_t orow = ((static_cast<int64_t>(b) * a.T + qr[qg]) * a.H + h) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        uint16_t* dst = static_cast<uint16_t*>(a.out) + orow + 16 * d + 4 * g;
        const uint32_t lo = float_to_bf16_bits(o[qg][d][0] * inv) |
                            (static_cast<uint32_t>(float_to_bf16_bits(o[qg][d][1] * inv)) << 16);
        const uint32_t hi = float_to_bf16_bits(o[qg][d][2] * inv) |
                            (static_cast<uint32_t>(float_to_bf16_bits(o[qg][d][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
      }
    }
  }
};

template <int E, int D>
__device__ void express_block_b(AttnB<E, D>& at, const ExpressView& ev, int beta, int S, int key_end) {
  bool row_ok[NQG];
  for (int qg = 0; qg < NQG; ++qg) row_ok[qg] = (at.qr[qg] / ev.n) == beta;
  const int unit = at.unit;
  if (beta < 4) {
    at.run_segment(SegB{nullptr, 0, min(key_end, S), 0.f, nullptr, 1}, row_ok);
    return;
  }
  int Ep = 1;
  while ((1LL << (2 * (Ep + 1))) <= beta) ++Ep;
  const int m = 1 << (2 * Ep);
  const int since = beta - m;
  const int nbc = since / m;
  const int rem = since % m;
  const float lm = static_cast<float>(2 * Ep);
  at.run_segment(SegB{ev.halve_out + (static_cast<int64_t>(unit) * ev.n_halves + (Ep - 1)) * ev.n, 0, ev.n, lm,
                      nullptr, 0},
                 row_ok);
  if (nbc > 0)
    at.run_segment(SegB{ev.batch_out + (static_cast<int64_t>(unit) * ev.n_batches_done + 3 * (Ep - 1)) * ev.n, 0,
                        nbc * ev.n, lm, nullptr, 0},
                   row_ok);
  const int n_rep = static_cast<int>((static_cast<int64_t>(rem) * 2 * ev.n) / m);
  if (n_rep > 0)
    at.run_segment(SegB{ev.reps + (static_cast<int64_t>(unit) * ev.n_batches_alloc + 3 * (Ep - 1) + nbc) * 2 * ev.n,
                        0, n_rep, lm - 1.0f, nullptr, 0},
                   row_ok);
  const int bn = beta * ev.n;
  at.run_segment(SegB{nullptr, bn, min(key_end, S) - bn, 0.f, nullptr, 1}, row_ok);
}

template <int E, int D>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnLaunch a) {
  __shared__ SmemB<E, D> sm;
  const int64_t tile = xcd_remap(blockIdx.y * static_cast<int64_t>(gridDim.x) + blockIdx.x,
                                 static_cast<int64_t>(gridDim.x) * gridDim.y);
  const int q0 = static_cast<int>(tile % gridDim.x) * kQ;
  AttnB<E, D> at(a, sm, q0, static_cast<int>(tile / gridDim.x));
  if (!a.causal) {
    bool ok[NQG];
    for (int qg = 0; qg < NQG; ++qg) ok[qg] = true;
    if (a.cs_idx)
      at.run_segment(SegB{a.cs_idx + at.unit * a.cs_stride, 0, a.cs_n, a.cs_lnw * kLog2eB,
                          a.cs_w ? a.cs_w + at.unit * a.cs_stride : nullptr, 0},
                     ok);
    else
      at.run_segment(SegB{nullptr, 0, a.S, a.cs_lnw * kLog2eB, nullptr, 0}, ok);
  } else {
    const int n = a.ev.n;
    const int q_last = min(q0 + kQ - 1, a.T - 1);
    for (int beta = q0 / n; beta <= q_last / n; ++beta)
      express_block_b(at, a.ev, beta, a.S, min(q_last + 1, (beta + 1) * n));
  }
  at.finish();
}

template <int E, int D>
hipError_t launch_b(const AttnLaunch& a, hipStream_t s) {
  dim3 grid((a.T + kQ - 1) / kQ, a.B * a.H);
  hipLaunchKernelGGL((attn_bf16_kernel<E, D>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const AttnLaunch& a, int E, int D, hipStream_t s) {
  if (E == 64 && D == 64) return launch_b<64, 64>(a, s);
  if (E == 64 && D == 128) return launch_b<64, 128>(a, s);
  if (E == 64 && D == 256) return launch_b<64, 256>(a, s);
  if (E == 128 && D == 128) return launch_b<128, 128>(a, s);
  if (E == 128 && D == 64) return launch_b<128, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace thin
