// gdn_span_chunked: the gated delta rule over a long chain span (prefill
// length), chunk by chunk.
//
// Recurrence (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025):
//   S_t = a_t S_{t-1} + w_t k_t^T,  w_t = b_t (v_t - a_t S_{t-1} k_t),  o_t = S_t q_t.
// The only sequential dependency of the plain recurrence is w_t on S_{t-1}
// k_t. The chunked form (the paper's hardware-efficient chunkwise algorithm,
// WY/UT representation of the products of Householder-like factors) removes
// it inside a chunk of C positions starting from state S_0: with
// G[t][j] = a_{j+1} ... a_t (G[t][t] = 1) and g_t = a_0 ... a_t,
//   w_t + sum_{j<t} b_t G[t][j] (k_t . k_j) w_j = b_t (v_t - g_t S_0 k_t),
// a unit lower-triangular system (I + A) W = Y for all value rows at once.
// After solving it the states and outputs follow from the cheap rank-1
// recurrence S_t = a_t S_{t-1} + w_t k_t^T, which has no dot product on its
// critical path.
//
// The outputs need no state either: o_t = g_t S_0 q_t + sum_{j<=t} G[t][j]
// (q_t . k_j) w_j.
//
// MI355X design. One block of 4 waves per (request, value head, 16 state
// rows); each lane keeps 8 columns of one row of S in VGPRs across all
// chunks (the layout of gdn_verify_span). Per chunk of 64 positions:
//  1. k, q and the block's v rows staged in LDS as f32 from registers that
//     were loaded while the previous chunk was processed;
//  2. K K^T and Q K^T (64 x 64 each) on the matrix cores (bf16 inputs:
//     32x32x16 MFMA, exact products and f32 accumulation, one 32x32 tile of
//     each per wave; f32 inputs: vector FMA), and X = K S_0^T, QS = Q S_0^T
//     for the block's rows (16x16x4 f32 MFMA, one 16-position tile per wave);
//  3. G, g, A = strictly lower (b_t G[t][j] (K K^T)[t][j]) and P = lower
//     (G[t][j] (Q K^T)[t][j]) by running products, four lanes per row
//     (16 columns each, the decays above a lane's segment from the other
//     lanes; no division, no logarithm: zero and tiny decays are exact);
//  4. Y = b (V - g X), then (I + A) W = Y by blocks of 16 positions: a
//     block-row update by all threads, then forward substitution inside the
//     16 x 16 diagonal block with one lane per state row;
//  5. outputs O = g QS + P W;
//  6. with capture, states S_t = a_t S_{t-1} + w_t k_t^T (8 FMAs per lane
//     and position, no dot product), each stored with nontemporal 16-byte
//     stores; without, only the chunk-end state S_C = g S_0 + (G_C W)^T K on
//     the matrix cores.
// Positions past the end of the span are padded with a = 1, b = 0, k = q =
// v = 0 (identity steps) and never streamed.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.h"
#include "internal.h"

namespace hrs {
namespace {

constexpr int kC = 64;          // positions per chunk
constexpr int kDK = 128;        // d_k = d_v (the built size)
constexpr int kRows = 16;       // state rows per block
constexpr int kThreads = 256;   // 4 waves
constexpr int kLPR = 16;        // lanes per state row in the streaming pass
constexpr int kNCH = kDK / (4 * kLPR);   // float4 chunks per lane (2)
constexpr int kKS = kDK + 4;    // LDS row stride of k and q (spreads 4 rows over banks)
constexpr int kSS = kDK + 4;    // LDS row stride of the state rows (16-byte rows, 4-bank offsets)
constexpr int kAS = kC + 4;     // LDS row stride of K K^T / A and Q K^T / P (16-byte rows)

// LDS layout, in floats.
constexpr int kOffK = 0;
constexpr int kOffQ = kOffK + kC * kKS;
constexpr int kOffV = kOffQ + kC * kKS;           // [C][16] v rows of the block
constexpr int kOffS0 = kOffV + kC * kRows;        // [16][kSS] S_0 rows
constexpr int kOffA = kOffS0 + kRows * kSS;       // [C][kAS] K K^T, then A
constexpr int kOffP = kOffA + kC * kAS;           // [C][kAS] Q K^T, then P = G (Q K^T), lower incl.
constexpr int kOffX = kOffP + kC * kAS;           // [C][16] X, then Y, then W
constexpr int kOffQS = kOffX + kC * kRows;        // [C][16] Q S_0^T
constexpr int kOffGC = kOffQS + kC * kRows;       // [C] G[n-1][t]: decay from position t to the chunk end
constexpr int kOffG = kOffGC + kC;                // [C] g_t
constexpr int kOffAv = kOffG + kC;                // [C] a_t
constexpr int kOffBv = kOffAv + kC;               // [C] b_t
constexpr int kTS = 20;                           // LDS row stride of the diagonal-block inverses
constexpr int kOffTb = kOffBv + kC;               // [4][16][kTS] (I + A_bb)^-1 of the 16 x 16 diagonal blocks
constexpr int kOffRb = kOffTb + 4 * 16 * kTS;     // [16][16] right-hand side of one block
constexpr int kLdsFloats = kOffRb + 16 * kRows;
constexpr size_t kLdsBytes = static_cast<size_t>(kLdsFloats) * sizeof(float);

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* a;
  const void* b;
  float* state;
  float* ckpt;
  void* out;       // float or bf16 (OUTBF)
  int32_t n_pos;
  int32_t n_kheads;
  int32_t n_vheads;
  int32_t group;   // Hv / Hk
  float q_scale;
};

// K K^T and Q K^T of the chunk into A and P (64 x 64 each). bf16 inputs:
// 32 x 32 tiles on the matrix cores, operands read from the bf16 inputs
// (exact products, f32 accumulation); each wave computes one tile of each.
// f32 inputs: vector FMA from the staged rows.
// Eight staged f32 values that are bf16-exact, packed back into bf16 pairs
// (the upper halves of their bit patterns).
__device__ __forceinline__ bf16x8 pack_bf16(const float* p) {
  const u32x4 x = *reinterpret_cast<const u32x4*>(p);
  const u32x4 y = *reinterpret_cast<const u32x4*>(p + 4);
  u32x4 r;
  r.x = (x.x >> 16) | (x.y & 0xFFFF0000u);
  r.y = (x.z >> 16) | (x.w & 0xFFFF0000u);
  r.z = (y.x >> 16) | (y.y & 0xFFFF0000u);
  r.w = (y.z >> 16) | (y.w & 0xFFFF0000u);
  return __builtin_bit_cast(bf16x8, r);
}

// K K^T and Q K^T of the staged chunk into A and P (64 x 64 each; q is
// staged unscaled). bf16 inputs: 32 x 32 tiles on the matrix cores, operands
// packed back to bf16 from the staged rows (exact), f32 accumulation; each
// wave computes one tile of each. f32 inputs: vector FMA.
template <typename TIn>
__device__ __forceinline__ void gram(float* lds) {
  float* const A = lds + kOffA;
  float* const P = lds + kOffP;
  const float* const K = lds + kOffK;
  const float* const Q = lds + kOffQ;
  const int tid = threadIdx.x;
  if constexpr (sizeof(TIn) == 2) {
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ti = wave >> 1, tj = wave & 1;
    const int ra = 32 * ti + (lane & 31);
    const int rb = 32 * tj + (lane & 31);
    const int ko = 8 * (lane >> 5);
    f32x16 acc_k = {}, acc_q = {};
#pragma unroll
    for (int kk = 0; kk < kDK; kk += 16) {
      const bf16x8 b8 = pack_bf16(K + rb * kKS + kk + ko);
      acc_k = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack_bf16(K + ra * kKS + kk + ko), b8, acc_k, 0, 0, 0);
      acc_q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pack_bf16(Q + ra * kKS + kk + ko), b8, acc_q, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * ti + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      A[row * kAS + 32 * tj + (lane & 31)] = acc_k[r];
      P[row * kAS + 32 * tj + (lane & 31)] = acc_q[r];
    }
  } else {
    // 2 x 8 register tiles.
    for (int tile = tid; tile < (kC / 2) * (kC / 8); tile += kThreads) {
      const int t0 = (tile / (kC / 8)) * 2;
      const int j0 = (tile % (kC / 8)) * 8;
      float ak[2][8] = {}, aq[2][8] = {};
      for (int c = 0; c < kDK; c += 4) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(K + t0 * kKS + c);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(K + (t0 + 1) * kKS + c);
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(Q + t0 * kKS + c);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(Q + (t0 + 1) * kKS + c);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 y = *reinterpret_cast<const f32x4*>(K + (j0 + j) * kKS + c);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            ak[0][j] = __builtin_fmaf(x0[u], y[u], ak[0][j]);
            ak[1][j] = __builtin_fmaf(x1[u], y[u], ak[1][j]);
            aq[0][j] = __builtin_fmaf(z0[u], y[u], aq[0][j]);
            aq[1][j] = __builtin_fmaf(z1[u], y[u], aq[1][j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        A[t0 * kAS + j0 + j] = ak[0][j];
        A[(t0 + 1) * kAS + j0 + j] = ak[1][j];
        P[t0 * kAS + j0 + j] = aq[0][j];
        P[(t0 + 1) * kAS + j0 + j] = aq[1][j];
      }
    }
  }
}

// One chunk's inputs as loaded from memory (raw bits), so the loads of chunk
// c + 1 can be issued before chunk c is processed and consumed afterwards.
template <typename TIn> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void widen(float* o) const {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
  __device__ __forceinline__ void widen(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

constexpr int kKQItems = kC * (kDK / 8) / kThreads;   // k (and q) 8-element items per thread (4)

template <typename TIn>
struct ChunkRegs {
  Raw8<TIn> k[kKQItems], q[kKQItems], v;
  float a, b;
};

// Issue the loads of the chunk starting at c0 (n positions) into registers.
template <typename TIn, bool LOGG>
__device__ __forceinline__ void fetch_chunk(const ChunkArgs& args, ChunkRegs<TIn>& rg, int r, int h, int g, int row0,
                                            int c0, int n) {
  const int T = args.n_pos;
  const int tid = threadIdx.x;
  const TIn* qg = static_cast<const TIn*>(args.q);
  const TIn* kg = static_cast<const TIn*>(args.k);
  const TIn* vg = static_cast<const TIn*>(args.v);
#pragma unroll
  for (int i = 0; i < kKQItems; ++i) {
    const int e = tid + i * kThreads;
    const int t = e / (kDK / 8);
    const int j = (e % (kDK / 8)) * 8;
    if (t < n) {
      const size_t src = ((static_cast<size_t>(r) * T + c0 + t) * args.n_kheads + g) * kDK + j;
      rg.k[i].load(kg + src);
      rg.q[i].load(qg + src);
    } else {
      rg.k[i].zero();
      rg.q[i].zero();
    }
  }
  {
    const int t = tid / (kRows / 8);
    const int i0 = (tid % (kRows / 8)) * 8;
    if (tid < kC * (kRows / 8) && t < n)
      rg.v.load(vg + ((static_cast<size_t>(r) * T + c0 + t) * args.n_vheads + h) * kDK + row0 + i0);
    else
      rg.v.zero();
  }
  rg.a = 1.0f;
  rg.b = 0.0f;
  if (tid < n) {
    const size_t src = (static_cast<size_t>(r) * T + c0 + tid) * args.n_vheads + h;
    rg.a = load_elem<TIn>(static_cast<const TIn*>(args.a), src);   // the log decay with log gates
    rg.b = load_elem<TIn>(static_cast<const TIn*>(args.b), src);
  }
}

// Write a fetched chunk into the staging buffers (f32; q unscaled).
template <typename TIn, bool LOGG>
__device__ __forceinline__ void stage_chunk(float* lds, const ChunkRegs<TIn>& rg, int n) {
  const int tid = threadIdx.x;
  float* const Kl = lds + kOffK;
  float* const Ql = lds + kOffQ;
#pragma unroll
  for (int i = 0; i < kKQItems; ++i) {
    const int e = tid + i * kThreads;
    const int t = e / (kDK / 8);
    const int j = (e % (kDK / 8)) * 8;
    float x[8];
    rg.k[i].widen(x);
    *reinterpret_cast<f32x4*>(Kl + t * kKS + j) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(Kl + t * kKS + j + 4) = f32x4{x[4], x[5], x[6], x[7]};
    rg.q[i].widen(x);
    *reinterpret_cast<f32x4*>(Ql + t * kKS + j) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(Ql + t * kKS + j + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
  if (tid < kC * (kRows / 8)) {
    float x[8];
    rg.v.widen(x);
    float* const lv = lds + kOffV + (tid / (kRows / 8)) * kRows + (tid % (kRows / 8)) * 8;
    *reinterpret_cast<f32x4*>(lv) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(lv + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
  if (tid < kC) {
    // Log-space gates: a_t = exp(g_t) (positions past the span end keep a = 1).
    lds[kOffAv + tid] = (LOGG && tid < n) ? expf(rg.a) : rg.a;
    lds[kOffBv + tid] = rg.b;
  }
}

// One output rounded to the nearest bf16 (ties to even; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// LOGG: `a` holds log decays; OUTBF: outputs are written as bf16.
template <typename TIn, bool CAPTURE, bool LOGG, bool OUTBF>
__global__ __launch_bounds__(kThreads) void gdn_chunked_kernel(const ChunkArgs args) {
  extern __shared__ float lds[];
  const int T = args.n_pos;
  const int Hv = args.n_vheads;
  const int nrb = kDK / kRows;
  const int W = blockIdx.x;
  const int row0 = (W % nrb) * kRows;
  const int h = (W / nrb) % Hv;
  const int r = W / (nrb * Hv);
  const int g = h / args.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane % kLPR;
  const int row_blk = (tid >> 6) * (64 / kLPR) + lane / kLPR;   // 0..15
  const size_t head_elems = static_cast<size_t>(kDK) * kDK;
  const size_t pos_stride = static_cast<size_t>(Hv) * head_elems;
  float* const Kl = lds + kOffK;
  float* const Ql = lds + kOffQ;
  float* const Vl = lds + kOffV;
  float* const S0 = lds + kOffS0;
  float* const A = lds + kOffA;
  float* const P = lds + kOffP;
  float* const X = lds + kOffX;
  float* const QS = lds + kOffQS;
  float* const GC = lds + kOffGC;
  float* const Tb = lds + kOffTb;
  float* const Rb = lds + kOffRb;
  float* const Gv = lds + kOffG;
  float* const Av = lds + kOffAv;
  float* const Bv = lds + kOffBv;
  // q is staged unscaled; q_scale enters P and QS.
  const float p_scale = args.q_scale;

  float* const state_row = args.state + (static_cast<size_t>(r) * Hv + h) * head_elems +
                           static_cast<size_t>(row0 + row_blk) * kDK;
  float* const ckpt_row0 = CAPTURE ? args.ckpt + static_cast<size_t>(r) * T * pos_stride +
                                         static_cast<size_t>(h) * head_elems +
                                         static_cast<size_t>(row0 + row_blk) * kDK
                                   : nullptr;
  const size_t out_h = (static_cast<size_t>(r) * T * Hv + h) * kDK + row0;   // element offset

  f32x4 s[kNCH];
#pragma unroll
  for (int m = 0; m < kNCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(state_row + 4 * (li + kLPR * m));

  ChunkRegs<TIn> rg;
  fetch_chunk<TIn, LOGG>(args, rg, r, h, g, row0, 0, min(kC, T));
  for (int c0 = 0; c0 < T; c0 += kC) {
    const int n = min(kC, T - c0);
    __syncthreads();   // the previous chunk's LDS reads are done
    // 1. Stage the fetched chunk (k, q unscaled, the block's v rows, gates)
    //    and the current state rows, then fetch the next chunk: its loads
    //    complete while this one is processed.
    stage_chunk<TIn, LOGG>(lds, rg, n);
#pragma unroll
    for (int m = 0; m < kNCH; ++m) *reinterpret_cast<f32x4*>(S0 + row_blk * kSS + 4 * (li + kLPR * m)) = s[m];
    if (c0 + kC < T) fetch_chunk<TIn, LOGG>(args, rg, r, h, g, row0, c0 + kC, min(kC, T - c0 - kC));
    __syncthreads();
    // 2. K K^T and Q K^T (matrix cores for bf16), X = K S_0^T and
    //    QS = Q S_0^T.
    gram<TIn>(lds);
    {
      // X and QS on the matrix cores (16x16x4 f32 MFMA, exact f32 products):
      // wave w takes positions [16 w, 16 w + 16) for all 16 state rows. In
      // each step of 4 MFMAs over 16 columns, lane group kq = lane / 16
      // supplies columns [c + 4 kq, c + 4 kq + 4), so a lane reads its
      // operands as 16-byte LDS loads.
      const int wave = tid >> 6;
      const int lane = tid & 63;
      const int row = 16 * wave + (lane & 15);    // position (A operand row)
      const int srow = lane & 15;                  // state row (B operand column)
      const int kq = lane >> 4;
      f32x4 xk = {}, xq = {};
#pragma unroll 2
      for (int c = 0; c < kDK; c += 16) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(Kl + row * kKS + c + 4 * kq);
        const f32x4 qv = *reinterpret_cast<const f32x4*>(Ql + row * kKS + c + 4 * kq);
        const f32x4 sv = *reinterpret_cast<const f32x4*>(S0 + srow * kSS + c + 4 * kq);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xk = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u], sv[u], xk, 0, 0, 0);
          xq = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[u], sv[u], xq, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 16 * wave + 4 * kq + u;
        X[t * kRows + srow] = xk[u];
        QS[t * kRows + srow] = xq[u];
      }
    }
    __syncthreads();
    // 3. Row t: A[t][j] = b_t G[t][j] (K K^T)[t][j] for j < t, P[t][j] =
    //    G[t][j] (q_t . k_j) for j <= t, and g_t, where G[t][j] = a_{j+1}
    //    ... a_t (1 for j >= t). Four lanes share a row, each 16 columns
    //    [16 s, 16 s + 16): a lane multiplies the decays of its own segment
    //    into running products from the segment's top down (no division, no
    //    logarithm: zero and tiny decays are exact), and the product of the
    //    decays above its segment comes from the other three lanes.
    {
      const int t = tid >> 2;
      const int sg = tid & 3;
      const int j0 = 16 * sg;
      float av[16];   // a_{j0} .. a_{j0 + 15}
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(Av + j0 + j);
        av[j] = x.x; av[j + 1] = x.y; av[j + 2] = x.z; av[j + 3] = x.w;
      }
      // Product of this segment's decays with index <= t (the factor that
      // every column of the segments below needs).
      float own = 1.0f;
#pragma unroll
      for (int i = 15; i >= 0; --i) own *= (j0 + i <= t) ? av[i] : 1.0f;
      // Product of the segments above (lanes sg + 1 .. 3 of this row),
      // highest first.
      const int base = tid & ~3;
      float above = 1.0f;
#pragma unroll
      for (int k = 3; k >= 1; --k) {
        const float o = __shfl(own, base + k);
        if (k > sg) above *= o;
      }
      const float bt = Bv[t];
      float* const arow = A + t * kAS;
      float* const prow = P + t * kAS;
      const bool last = t == n - 1;   // this row's products are the decays to the chunk end
      float gp = above;               // G[t][j] for the current j
#pragma unroll
      for (int j = 12; j >= 0; j -= 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(arow + j0 + j);
        const f32x4 qv = *reinterpret_cast<const f32x4*>(prow + j0 + j);
        f32x4 ka, qa, gc;
#pragma unroll
        for (int u = 3; u >= 0; --u) {
          const int jj = j0 + j + u;   // column
          if (j + u < 15) gp *= (jj < t) ? av[j + u + 1] : 1.0f;
          ka[u] = bt * gp * kv[u];
          qa[u] = (p_scale * gp) * qv[u];
          gc[u] = gp;
        }
        *reinterpret_cast<f32x4*>(arow + j0 + j) = ka;
        *reinterpret_cast<f32x4*>(prow + j0 + j) = qa;
        if (last) *reinterpret_cast<f32x4*>(GC + j0 + j) = gc;
      }
      if (sg == 0) Gv[t] = av[0] * gp;   // g_t = a_0 G[t][0]
    }
    __syncthreads();
    // 4. Y = b (V - g X) in place of X (waves 1-3) while wave 0 inverts the
    //    four 16 x 16 diagonal blocks of I + A (one lane per column of one
    //    block, forward substitution in registers); then (I + A) W = Y block
    //    by block: R = Y_b - A_b,<b W_<b, W_b = (I + A_bb)^-1 R, W in place of Y.
    if (tid < 64) {
      const int bi = tid >> 4;
      const int col = tid & 15;
      const float* ab = A + (16 * bi) * kAS + 16 * bi;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float r[16];
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(ab + i * kAS + j);
          r[j] = v4.x; r[j + 1] = v4.y; r[j + 2] = v4.z; r[j + 3] = v4.w;
        }
        float acc0 = (i == col) ? 1.0f : 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int j = 0; j < i; ++j) {
          if (j & 1) acc1 = __builtin_fmaf(-r[j], x[j], acc1);
          else acc0 = __builtin_fmaf(-r[j], x[j], acc0);
        }
        x[i] = acc0 + acc1;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Tb[(bi * 16 + i) * kTS + col] = x[i];
    } else {
      for (int e = tid - 64; e < kC * kRows; e += kThreads - 64) {
        const int t = e / kRows;
        X[e] = Bv[t] * __builtin_fmaf(-Gv[t], X[e], Vl[e]);
      }
    }
    __syncthreads();
    for (int blk = 0; blk < kC / 16; ++blk) {
      const int i = tid >> 4;          // row inside the block
      const int col = tid & 15;
      const int t = 16 * blk + i;
      {
        float acc0 = X[t * kRows + col], acc1 = 0.0f;
        for (int j = 0; j < 16 * blk; j += 4) {
          const f32x4 av4 = *reinterpret_cast<const f32x4*>(A + t * kAS + j);
          acc0 = __builtin_fmaf(-av4.x, X[j * kRows + col], acc0);
          acc1 = __builtin_fmaf(-av4.y, X[(j + 1) * kRows + col], acc1);
          acc0 = __builtin_fmaf(-av4.z, X[(j + 2) * kRows + col], acc0);
          acc1 = __builtin_fmaf(-av4.w, X[(j + 3) * kRows + col], acc1);
        }
        Rb[i * kRows + col] = acc0 + acc1;
      }
      __syncthreads();
      {
        const float* trow = Tb + (blk * 16 + i) * kTS;
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(trow + j);
          acc0 = __builtin_fmaf(t4.x, Rb[j * kRows + col], acc0);
          acc1 = __builtin_fmaf(t4.y, Rb[(j + 1) * kRows + col], acc1);
          acc0 = __builtin_fmaf(t4.z, Rb[(j + 2) * kRows + col], acc0);
          acc1 = __builtin_fmaf(t4.w, Rb[(j + 3) * kRows + col], acc1);
        }
        X[t * kRows + col] = acc0 + acc1;
      }
      __syncthreads();
    }
    // 5. Outputs: o_t = g_t (q_t . S_0 rows) + sum_{j <= t} P[t][j] w_j; a
    //    thread takes 4 state rows of one position.
    {
      const int t = tid >> 2;
      const int c4 = (tid & 3) * 4;
      if (t < n) {
        const f32x4 qs = *reinterpret_cast<const f32x4*>(QS + t * kRows + c4);
        const float gt = Gv[t] * args.q_scale;
        f32x4 acc = {gt * qs.x, gt * qs.y, gt * qs.z, gt * qs.w};
        for (int j = 0; j <= t; j += 4) {
          const f32x4 p4 = *reinterpret_cast<const f32x4*>(P + t * kAS + j);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            // Entries past the diagonal (j + u > t) are skipped; the block's
            // positions past the span end have w = 0 (b = 0).
            const float pv = (j + u <= t) ? p4[u] : 0.0f;
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(X + (j + u) * kRows + c4);
            acc.x = __builtin_fmaf(pv, w4.x, acc.x);
            acc.y = __builtin_fmaf(pv, w4.y, acc.y);
            acc.z = __builtin_fmaf(pv, w4.z, acc.z);
            acc.w = __builtin_fmaf(pv, w4.w, acc.w);
          }
        }
        const size_t o = out_h + static_cast<size_t>(c0 + t) * Hv * kDK + c4;
        if constexpr (OUTBF) {
          u32x2 w;
          w.x = bf16_rne(acc.x) | (bf16_rne(acc.y) << 16);
          w.y = bf16_rne(acc.z) | (bf16_rne(acc.w) << 16);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(args.out) + o) = w;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(args.out) + o) = acc;
        }
      }
    }
    if constexpr (CAPTURE) {
      // 6. States: S_t = a_t S_{t-1} + w_t k_t^T, each checkpointed; 8
      //    positions at a time so their LDS reads are issued together.
      for (int t0 = 0; t0 < n; t0 += 8) {
        float at[8], wt[8];
        f32x4 kk[8][kNCH];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          at[u] = Av[t0 + u];
          wt[u] = X[(t0 + u) * kRows + row_blk];
#pragma unroll
          for (int m = 0; m < kNCH; ++m)
            kk[u][m] = *reinterpret_cast<const f32x4*>(Kl + (t0 + u) * kKS + 4 * (li + kLPR * m));
        }
        const int un = min(8, n - t0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (un == 8 || u < un) {
#pragma unroll
            for (int m = 0; m < kNCH; ++m) {
              s[m].x = __builtin_fmaf(wt[u], kk[u][m].x, at[u] * s[m].x);
              s[m].y = __builtin_fmaf(wt[u], kk[u][m].y, at[u] * s[m].y);
              s[m].z = __builtin_fmaf(wt[u], kk[u][m].z, at[u] * s[m].z);
              s[m].w = __builtin_fmaf(wt[u], kk[u][m].w, at[u] * s[m].w);
            }
            float* dst = ckpt_row0 + static_cast<size_t>(c0 + t0 + u) * pos_stride;
#pragma unroll
            for (int m = 0; m < kNCH; ++m)
              __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(dst + 4 * (li + kLPR * m)));
          }
        }
      }
    } else {
      // 6. State at the chunk end only: S_C = g_{n-1} S_0 + sum_t G[n-1][t]
      //    w_t k_t^T on the matrix cores (16x16x4 f32 MFMA; wave w takes
      //    columns [32 w, 32 w + 32)), written over S_0 and read back into
      //    the lanes' registers.
      const int wave = tid >> 6;
      const int lane = tid & 63;
      const int i = lane & 15;
      const int kq = lane >> 4;
      f32x4 d0 = {}, d1 = {};
#pragma unroll
      for (int tb = 0; tb < kC; tb += 16) {
        const int tq = tb + 4 * kq;
        const f32x4 gc = *reinterpret_cast<const f32x4*>(GC + tq);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float wv = gc[u] * X[(tq + u) * kRows + i];
          const float* krow = Kl + (tq + u) * kKS + 32 * wave + (lane & 15);
          d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(wv, krow[0], d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(wv, krow[16], d1, 0, 0, 0);
        }
      }
      const float gn = Gv[n - 1];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float* e0 = S0 + (4 * kq + u) * kSS + 32 * wave + (lane & 15);
        e0[0] = __builtin_fmaf(gn, e0[0], d0[u]);
        e0[16] = __builtin_fmaf(gn, e0[16], d1[u]);
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < kNCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(S0 + row_blk * kSS + 4 * (li + kLPR * m));
    }
  }
  if (!CAPTURE) {
#pragma unroll
    for (int m = 0; m < kNCH; ++m) *reinterpret_cast<f32x4*>(state_row + 4 * (li + kLPR * m)) = s[m];
  }
}

template <typename TIn, bool CAPTURE, bool LOGG>
hipError_t launch_out(const ChunkArgs& args, int blocks, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL((gdn_chunked_kernel<TIn, CAPTURE, LOGG, true>), dim3(blocks), dim3(kThreads), kLdsBytes, s,
                       args);
  else
    hipLaunchKernelGGL((gdn_chunked_kernel<TIn, CAPTURE, LOGG, false>), dim3(blocks), dim3(kThreads), kLdsBytes, s,
                       args);
  return launch_error();
}

template <typename TIn>
hipError_t launch_chunked(const ChunkArgs& args, int blocks, bool capture, bool log_gates, bool out_bf16,
                          hipStream_t s) {
  if (capture)
    return log_gates ? launch_out<TIn, true, true>(args, blocks, out_bf16, s)
                     : launch_out<TIn, true, false>(args, blocks, out_bf16, s);
  return log_gates ? launch_out<TIn, false, true>(args, blocks, out_bf16, s)
                   : launch_out<TIn, false, false>(args, blocks, out_bf16, s);
}

}  // namespace
}  // namespace hrs

using namespace hrs;

extern "C" int gdn_span_chunked(const hrs_chunked_desc* cd, const void* q, const void* k, const void* v,
                                const void* a, const void* b, float* state, float* ckpt, void* out, void* stream) {
  if (cd == nullptr) return HRS_EINVAL;
  const hrs_gdn_desc* d = &cd->gdn;
  if (d->n_req < 1 || d->n_kheads < 1 || d->n_vheads < 1 || d->d_k < 1 || d->d_v < 1) return HRS_EINVAL;
  if (d->n_vheads % d->n_kheads != 0) return HRS_EINVAL;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(cd->out_dtype)) return HRS_EINVAL;
  if (d->topo != HRS_CHAIN) return d->topo == HRS_TREE ? HRS_EUNSUPPORTED : HRS_EINVAL;
  if (d->n_pos < 1 || d->n_pos > HRS_MAX_CHUNKED_POS) return HRS_EINVAL;
  if (!q || !k || !v || !a || !b || !state || !out) return HRS_EINVAL;
  if (static_cast<int64_t>(d->n_req) * d->n_vheads * (kDK / kRows) > (1 << 30)) return HRS_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) || !aligned16(state) ||
      !aligned16(out) || (ckpt && !aligned16(ckpt)))
    return HRS_EALIGN;
  if (d->d_k != kDK || d->d_v != kDK) return HRS_EUNSUPPORTED;

  ChunkArgs args;
  args.q = q; args.k = k; args.v = v; args.a = a; args.b = b;
  args.state = state; args.ckpt = ckpt; args.out = out;
  args.n_pos = d->n_pos; args.n_kheads = d->n_kheads; args.n_vheads = d->n_vheads;
  args.group = d->n_vheads / d->n_kheads; args.q_scale = d->q_scale;
  const int blocks = d->n_req * d->n_vheads * (kDK / kRows);
  const bool logg = cd->log_gates != 0;
  const bool obf = cd->out_dtype == HRS_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const hipError_t e = d->in_dtype == HRS_BF16
                           ? launch_chunked<uint16_t>(args, blocks, ckpt != nullptr, logg, obf, s)
                           : launch_chunked<float>(args, blocks, ckpt != nullptr, logg, obf, s);
  return e == hipSuccess ? HRS_OK : HRS_EDEVICE;
}
