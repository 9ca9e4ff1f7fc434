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
//  1. k, q (times q_scale) and the block's v rows staged in LDS as f32;
//  2. K K^T and Q K^T (64 x 64 each) on the matrix cores (bf16 inputs:
//     32x32x16 MFMA, exact products and f32 accumulation, one 32x32 tile of
//     each per wave; f32 inputs: vector FMA), and X = K S_0^T, QS = Q S_0^T
//     for the block's rows (16x16x4 f32 MFMA, one 16-position tile per wave);
//  3. G, g, A = strictly lower (b_t G[t][j] (K K^T)[t][j]) and P = lower
//     (G[t][j] (Q K^T)[t][j]) by running products (no division, no
//     logarithm: zero and tiny decays are exact);
//  4. Y = b (V - g X), then (I + A) W = Y by blocks of 16 positions: a
//     block-row update by all threads, then forward substitution inside the
//     16 x 16 diagonal block with one lane per state row;
//  5. outputs O = g QS + P W;
//  6. states S_t = a_t S_{t-1} + w_t k_t^T (8 FMAs per lane and position, no
//     dot product), each stored with nontemporal 16-byte stores when
//     captured.
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
constexpr int kOffGC = kOffQS + kC * kRows;       // [C] unused pad (keeps g_t 16-byte aligned)
constexpr int kOffG = kOffGC + kC;                // [C] g_t
constexpr int kOffAv = kOffG + kC;                // [C] a_t
constexpr int kOffBv = kOffAv + kC;               // [C] b_t
constexpr int kLdsFloats = kOffBv + kC;
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
  float* out;
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
template <typename TIn>
__device__ __forceinline__ void gram(const ChunkArgs& args, float* lds, const TIn* kbase, const TIn* qbase, int n) {
  float* const A = lds + kOffA;
  float* const P = lds + kOffP;
  const int tid = threadIdx.x;
  if constexpr (sizeof(TIn) == 2) {
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ti = wave >> 1, tj = wave & 1;
    // Rows past the span end read row 0 (in bounds); those results are never
    // used (b = 0 there, and outputs past the end are not written).
    const int ra = 32 * ti + (lane & 31);
    const int rb = 32 * tj + (lane & 31);
    const size_t stride = static_cast<size_t>(args.n_kheads) * kDK;
    const size_t oa = static_cast<size_t>(ra < n ? ra : 0) * stride + 8 * (lane >> 5);
    const size_t ob = static_cast<size_t>(rb < n ? rb : 0) * stride + 8 * (lane >> 5);
    f32x16 acc_k = {}, acc_q = {};
#pragma unroll
    for (int kk = 0; kk < kDK; kk += 16) {
      const u32x4 wa = *reinterpret_cast<const u32x4*>(kbase + oa + kk);
      const u32x4 wq = *reinterpret_cast<const u32x4*>(qbase + oa + kk);
      const u32x4 wb = *reinterpret_cast<const u32x4*>(kbase + ob + kk);
      const bf16x8 b8 = __builtin_bit_cast(bf16x8, wb);
      acc_k = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wa), b8, acc_k, 0, 0, 0);
      acc_q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wq), b8, acc_q, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * ti + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      A[row * kAS + 32 * tj + (lane & 31)] = acc_k[r];
      P[row * kAS + 32 * tj + (lane & 31)] = acc_q[r];
    }
  } else {
    // 2 x 8 register tiles from the staged k and q (the staged q already
    // carries q_scale).
    const float* K = lds + kOffK;
    const float* Q = lds + kOffQ;
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

template <typename TIn, bool CAPTURE>
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
  const TIn* qg = static_cast<const TIn*>(args.q);
  const TIn* kg = static_cast<const TIn*>(args.k);
  const TIn* vg = static_cast<const TIn*>(args.v);
  const TIn* ag = static_cast<const TIn*>(args.a);
  const TIn* bg = static_cast<const TIn*>(args.b);
  float* const Kl = lds + kOffK;
  float* const Ql = lds + kOffQ;
  float* const Vl = lds + kOffV;
  float* const S0 = lds + kOffS0;
  float* const A = lds + kOffA;
  float* const P = lds + kOffP;
  float* const X = lds + kOffX;
  float* const QS = lds + kOffQS;
  float* const Gv = lds + kOffG;
  float* const Av = lds + kOffAv;
  float* const Bv = lds + kOffBv;
  // Q K^T from the raw bf16 inputs lacks q_scale; the f32 path forms it from
  // the staged (scaled) q.
  const float p_scale = sizeof(TIn) == 2 ? args.q_scale : 1.0f;

  float* const state_row = args.state + (static_cast<size_t>(r) * Hv + h) * head_elems +
                           static_cast<size_t>(row0 + row_blk) * kDK;
  float* const ckpt_row0 = CAPTURE ? args.ckpt + static_cast<size_t>(r) * T * pos_stride +
                                         static_cast<size_t>(h) * head_elems +
                                         static_cast<size_t>(row0 + row_blk) * kDK
                                   : nullptr;
  float* const out_h = args.out + (static_cast<size_t>(r) * T * Hv + h) * kDK + row0;

  f32x4 s[kNCH];
#pragma unroll
  for (int m = 0; m < kNCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(state_row + 4 * (li + kLPR * m));

  for (int c0 = 0; c0 < T; c0 += kC) {
    const int n = min(kC, T - c0);
    __syncthreads();   // the previous chunk's LDS reads are done
    // 1. Stage k, q (scaled), the block's v rows and the gates; the current
    //    state rows go to S0.
    for (int e = tid; e < kC * (kDK / 8); e += kThreads) {
      const int t = e / (kDK / 8);
      const int j = (e % (kDK / 8)) * 8;
      float kv[8] = {}, qv[8] = {};
      if (t < n) {
        const size_t src = ((static_cast<size_t>(r) * T + c0 + t) * args.n_kheads + g) * kDK + j;
        load8<TIn>(kg + src, kv);
        load8<TIn>(qg + src, qv);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Kl[t * kKS + j + i] = kv[i];
        Ql[t * kKS + j + i] = qv[i] * args.q_scale;
      }
    }
    for (int e = tid; e < kC * (kRows / 8); e += kThreads) {
      const int t = e / (kRows / 8);
      const int i0 = (e % (kRows / 8)) * 8;
      float vv[8] = {};
      if (t < n) load8<TIn>(vg + ((static_cast<size_t>(r) * T + c0 + t) * Hv + h) * kDK + row0 + i0, vv);
#pragma unroll
      for (int i = 0; i < 8; ++i) Vl[t * kRows + i0 + i] = vv[i];
    }
    if (tid < kC) {
      const size_t src = (static_cast<size_t>(r) * T + c0 + tid) * Hv + h;
      Av[tid] = tid < n ? load_elem<TIn>(ag, src) : 1.0f;
      Bv[tid] = tid < n ? load_elem<TIn>(bg, src) : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < kNCH; ++m) *reinterpret_cast<f32x4*>(S0 + row_blk * kSS + 4 * (li + kLPR * m)) = s[m];
    __syncthreads();
    // 2. K K^T and Q K^T (matrix cores for bf16), X = K S_0^T and
    //    QS = Q S_0^T (vector FMA, 2 x 2 register tiles per product).
    {
      const size_t base = ((static_cast<size_t>(r) * T + c0) * args.n_kheads + g) * kDK;
      gram<TIn>(args, lds, kg + base, qg + base, n);
    }
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
    //    G[t][j] (q_t . k_j) for j <= t, and g_t, by running products from
    //    the diagonal down (the decays are read into registers first).
    if (tid < kC) {
      const int t = tid;
      float av[kC];
#pragma unroll
      for (int j = 0; j < kC; j += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(Av + j);
        av[j] = x.x; av[j + 1] = x.y; av[j + 2] = x.z; av[j + 3] = x.w;
      }
      const float bt = Bv[t];
      float* const arow = A + t * kAS;
      float* const prow = P + t * kAS;
      // Branch-free: the running product stays 1 until j < t, and entries
      // with j > t (unused) are scaled by 1 as well.
      float gp = 1.0f;   // G[t][j] for the current j
#pragma unroll
      for (int j = kC - 4; j >= 0; j -= 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(arow + j);
        const f32x4 qv = *reinterpret_cast<const f32x4*>(prow + j);
        f32x4 ka, qa;
#pragma unroll
        for (int u = 3; u >= 0; --u) {
          const int jj = j + u;
          if (jj + 1 < kC) gp *= (jj < t) ? av[jj + 1] : 1.0f;
          ka[u] = bt * gp * kv[u];
          qa[u] = (p_scale * gp) * qv[u];
        }
        *reinterpret_cast<f32x4*>(arow + j) = ka;
        *reinterpret_cast<f32x4*>(prow + j) = qa;
      }
      Gv[t] = av[0] * gp;   // g_t = a_0 G[t][0]
    }
    __syncthreads();
    // 4. Y = b (V - g X) in place of X, then (I + A) W = Y by 16-position
    //    blocks, W in place of Y.
    for (int e = tid; e < kC * kRows; e += kThreads) {
      const int t = e / kRows;
      X[e] = Bv[t] * __builtin_fmaf(-Gv[t], X[e], Vl[e]);
    }
    __syncthreads();
    for (int blk = 0; blk < kC / 16; ++blk) {
      if (blk > 0) {
        // Subtract the contribution of the solved positions [0, 16 blk).
        const int t = 16 * blk + (tid >> 4);
        const int col = tid & 15;
        float acc0 = X[t * kRows + col], acc1 = 0.0f;
        for (int j = 0; j < 16 * blk; j += 4) {
          const f32x4 av4 = *reinterpret_cast<const f32x4*>(A + t * kAS + j);
          acc0 = __builtin_fmaf(-av4.x, X[j * kRows + col], acc0);
          acc1 = __builtin_fmaf(-av4.y, X[(j + 1) * kRows + col], acc1);
          acc0 = __builtin_fmaf(-av4.z, X[(j + 2) * kRows + col], acc0);
          acc1 = __builtin_fmaf(-av4.w, X[(j + 3) * kRows + col], acc1);
        }
        X[t * kRows + col] = acc0 + acc1;
        __syncthreads();
      }
      if (tid < kRows) {
        // Forward substitution inside the diagonal block, one lane per column.
        const int col = tid;
        const int base = 16 * blk;
        float wv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc0 = X[(base + i) * kRows + col], acc1 = 0.0f;
#pragma unroll
          for (int j = 0; j < i; ++j) {
            if (j & 1) acc1 = __builtin_fmaf(-A[(base + i) * kAS + base + j], wv[j], acc1);
            else acc0 = __builtin_fmaf(-A[(base + i) * kAS + base + j], wv[j], acc0);
          }
          wv[i] = acc0 + acc1;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) X[(base + i) * kRows + col] = wv[i];
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
        const float gt = Gv[t];
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
        *reinterpret_cast<f32x4*>(out_h + static_cast<size_t>(c0 + t) * Hv * kDK + c4) = acc;
      }
    }
    // 6. States: S_t = a_t S_{t-1} + w_t k_t^T (checkpoint each with capture),
    //    8 positions at a time so their LDS reads are issued together.
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
          if (CAPTURE) {
            float* dst = ckpt_row0 + static_cast<size_t>(c0 + t0 + u) * pos_stride;
#pragma unroll
            for (int m = 0; m < kNCH; ++m)
              __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(dst + 4 * (li + kLPR * m)));
          }
        }
      }
    }
  }
  if (!CAPTURE) {
#pragma unroll
    for (int m = 0; m < kNCH; ++m) *reinterpret_cast<f32x4*>(state_row + 4 * (li + kLPR * m)) = s[m];
  }
}

template <typename TIn>
hipError_t launch_chunked(const ChunkArgs& args, int blocks, bool capture, hipStream_t s) {
  if (capture)
    hipLaunchKernelGGL((gdn_chunked_kernel<TIn, true>), dim3(blocks), dim3(kThreads), kLdsBytes, s, args);
  else
    hipLaunchKernelGGL((gdn_chunked_kernel<TIn, false>), dim3(blocks), dim3(kThreads), kLdsBytes, s, args);
  return launch_error();
}

}  // namespace
}  // namespace hrs

using namespace hrs;

extern "C" int gdn_span_chunked(const hrs_gdn_desc* d, const void* q, const void* k, const void* v, const void* a,
                                const void* b, float* state, float* ckpt, float* out, void* stream) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_req < 1 || d->n_kheads < 1 || d->n_vheads < 1 || d->d_k < 1 || d->d_v < 1) return HRS_EINVAL;
  if (d->n_vheads % d->n_kheads != 0) return HRS_EINVAL;
  if (!dtype_ok(d->in_dtype)) return HRS_EINVAL;
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const hipError_t e = d->in_dtype == HRS_BF16 ? launch_chunked<uint16_t>(args, blocks, ckpt != nullptr, s)
                                               : launch_chunked<float>(args, blocks, ckpt != nullptr, s);
  return e == hipSuccess ? HRS_OK : HRS_EDEVICE;
}
