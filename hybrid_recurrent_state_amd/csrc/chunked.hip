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
// a unit lower-triangular system (I + A) W = Y for all value rows at once, so
// W = T Y with T = (I + A)^-1. The outputs need no state either:
//   o_t = g_t S_0 q_t + sum_{j<=t} P[t][j] w_j,  P[t][j] = G[t][j] (q_t . k_j),
// i.e. O = g QS + (P T) Y; and the chunk-end state is
//   S_C = g_{C-1} S_0 + sum_t G[C-1][t] w_t k_t^T.
// T, P T, g and G[C-1][.] depend on k, q and the gates only, not on S_0.
//
// MI355X design: two kernels per segment of up to 32 chunks.
//  * Pre-pass, one block of 4 waves per (request, value head, chunk), all
//    chunks in parallel: K K^T and Q K^T on the matrix cores (bf16 inputs:
//    32x32x16 MFMA, exact products, f32 accumulation), the decay products
//    (running products, four lanes per row, no division or logarithm: zero
//    and tiny decays are exact), T = (I + A)^-1 by 16 x 16 blocks (the
//    diagonal blocks by forward substitution, four lanes per column joined by
//    DPP; the blocks below them level by level on 16x16x4 f32 MFMA) and P T
//    (16x16x4 f32 MFMA); the record is written to the caller's workspace in
//    the order the sequential kernel's operand registers read it.
//  * Sequential kernel, one block of 4 waves per (request, value head, 16
//    state rows); each lane keeps 8 columns of one row of S in VGPRs across
//    all chunks (the layout of gdn_verify_span). Per chunk: X = K S_0^T and
//    QS = Q S_0^T, Y = b (V - g X), then W = T Y and P T Y from T and P T in
//    registers (16x16x4 f32 MFMA), the outputs, and the state: with capture
//    S_t = a_t S_{t-1} + w_t k_t^T (8 FMAs per lane and position, no dot
//    product), each stored with nontemporal 16-byte stores; without, the
//    chunk-end state on the matrix cores. With bf16 inputs X, QS and the
//    chunk-end state are bf16 products (16x16x32 MFMA): the f32 factor (S_0,
//    or G[C-1][t] w_t) is split into three bf16 parts whose sum is exactly the
//    f32 value, so every product is exact and the sums are f32; f32 inputs
//    use 16x16x4 f32 MFMA. The next chunk's inputs and pre-pass record are
//    loaded while a chunk is processed: for a segment of several bf16 chunks
//    by 4 producer waves, which stage them into the other of two LDS
//    buffers; otherwise by the 4 compute waves into their registers (a
//    single chunk keeps the smaller LDS footprint, two blocks per CU, and two
//    f32 input buffers would not fit in LDS). Blocks are ordered so
//    that the 8 row blocks of one head fall on one XCD (workgroups go to XCDs
//    round robin), where they share the head's k, q and record through that
//    XCD's L2.
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
constexpr int kRows = 16;       // state rows per sequential block
constexpr int kRowBlocks = kDK / kRows;
constexpr int kThreads = 256;   // 4 waves
constexpr int kLPR = 16;        // lanes per state row in the streaming pass
constexpr int kNCH = kDK / (4 * kLPR);   // float4 chunks per lane (2)
constexpr int kKS = kDK + 4;    // LDS row stride of k and q (spreads 4 rows over banks)
constexpr int kSS = kDK + 4;    // LDS row stride of the state rows (16-byte rows, 4-bank offsets)
constexpr int kTS = kC + 4;     // LDS row stride of the 64-wide matrices (16-byte rows)
constexpr int kSegChunks = 32;  // chunks per pre-pass + sequential launch pair

// Pre-pass record of one (request, value head, chunk) in the workspace, in
// floats: the 10 lower 16 x 16 tiles of T = (I + A)^-1, then those of P T
// (both are lower triangular), then g_t and G[C-1][t]. A tile (i, j), j <= i,
// sits at index i (i + 1) / 2 + j, in the order the sequential kernel's
// matrix-core operands read it: lane l = 16 kq + r of wave i holds row
// 16 i + r, columns 16 j + 4 kq .. + 3, as floats [4 l, 4 l + 4) of the tile.
constexpr int kTiles = 10;
constexpr int kRecT = 0;
constexpr int kRecPT = kRecT + kTiles * 256;
constexpr int kRecG = kRecPT + kTiles * 256;
constexpr int kRecGC = kRecG + kC;
constexpr int kRecFloats = kRecGC + kC;

__host__ __device__ constexpr int tile_index(int i, int j) { return i * (i + 1) / 2 + j; }

// Sequential kernel LDS layout, in bytes: one chunk's inputs (k, q, the
// block's v rows and the gates; in the producer/consumer form, PC, two such
// buffers, each also holding the chunk's pre-pass record), then the compute
// waves' own arrays. BF (bf16 inputs): k and q staged as bf16, and the
// chunk's starting state also as three bf16 parts whose sum is the f32 value
// (the operands of the bf16 products); f32 inputs: k and q as f32. Without
// PC, T and P T never go through LDS: each wave loads its own 16 rows
// straight into its matrix-core operand registers.
template <bool BF, bool PC = false>
struct SeqLds {
  static constexpr int kKRow = BF ? (kDK + 8) * 2 : kKS * 4;   // bytes per k or q row (16-byte rows)
  static constexpr int kSplRow = (kDK + 8) * 2;                // bytes per row of one state part
  // Offsets within an input buffer.
  static constexpr int K = 0;                                  // [C] rows of k
  static constexpr int Q = K + kC * kKRow;                     // [C] rows of q (unscaled)
  static constexpr int V = Q + kC * kKRow;                     // f32 [C][16] v rows of the block
  static constexpr int AV = V + kC * kRows * 4;                // f32 [C] a_t
  static constexpr int BV = AV + kC * 4;                       // f32 [C] b_t
  static constexpr int REC = BV + kC * 4;                      // PC: the chunk's pre-pass record
  static constexpr int IN = REC + (PC ? kRecFloats * 4 : 0);   // bytes of one input buffer
  // The compute waves' arrays, after the input buffer(s).
  static constexpr int S0 = (PC ? 2 : 1) * IN;                 // f32 [16][kSS] S_0 rows
  static constexpr int SPL = S0 + kRows * kSS * 4;             // BF: bf16 [3][16] S_0 parts
  static constexpr int Y = SPL + (BF ? 3 * kRows * kSplRow : 0);   // f32 [16][kTS] Y^T (state row, position)
  static constexpr int W = Y + kRows * kTS * 4;                // f32 [16][kTS] W^T
  static constexpr int G = W + kRows * kTS * 4;                // f32 [C] g_t
  static constexpr int GC = G + kC * 4;                        // f32 [C] G[n-1][t] (follows g_t, as in the record)
  static constexpr int kWpRow = (kC + 8) * 2;                  // bytes per row of one part of G[n-1][t] w_t
  static constexpr int WP = GC + kC * 4;                       // BF: bf16 [3][16] parts of G[n-1][t] w_t
  static constexpr int BYTES = WP + (BF ? 3 * kRows * kWpRow : 0);
  static_assert(Q % 16 == 0 && V % 16 == 0 && REC % 16 == 0 && IN % 16 == 0 && S0 % 16 == 0 && SPL % 16 == 0 &&
                    Y % 16 == 0 && W % 16 == 0 && WP % 16 == 0 && kWpRow % 16 == 0, "16-byte LDS rows");
};

// Pre-pass LDS layout: k and q staged first; A, P, T and T^T take their
// place once the Gram products are in registers.
constexpr int kPOffK = 0;
constexpr int kPOffQ = kC * kKS;
// bf16 inputs stage k and q as their bf16 bits instead: rows of kPKRowB bytes
// (16-byte rows, a 4-bank shift per row), q after k.
constexpr int kPOffKB = 0;
constexpr int kPKRowB = (kDK + 8) * 2;
constexpr int kPQOffB = kC * kPKRowB;
static_assert(2 * kPQOffB <= kC * kKS * 2 * 4, "bf16 k and q fit where the f32 rows would");
constexpr int kPOffA = 0;
constexpr int kPOffP = kC * kTS;
constexpr int kPOffT = 2 * kC * kTS;
constexpr int kPOffTt = 3 * kC * kTS;
constexpr int kPOffAv = (2 * kC * kKS > 4 * kC * kTS) ? 2 * kC * kKS : 4 * kC * kTS;
constexpr int kPOffBv = kPOffAv + kC;
constexpr int kPOffG = kPOffBv + kC;
constexpr int kPOffGC = kPOffG + kC;
constexpr int kPLdsFloats = kPOffGC + kC;
constexpr size_t kPLdsBytes = static_cast<size_t>(kPLdsFloats) * sizeof(float);

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
  int32_t n_req;
  int32_t n_pos;
  int32_t n_kheads;
  int32_t n_vheads;
  int32_t group;   // Hv / Hk
  float q_scale;
};

// K K^T and Q K^T of the staged chunk (q unscaled), computed into registers
// and then written over the staging area as A and P (64 x 64 each, row
// stride kTS); the block barrier between the two keeps every read of k and
// q ahead of the writes. bf16 inputs: 32 x 32 tiles on the matrix cores,
// operands read straight from the staged bf16 rows (staged as f32 and packed
// back at each read, the pre-pass took 1.5-2% longer per prefill), f32
// accumulation, one tile of each per wave. f32 inputs: vector FMA, 2 x 8
// outputs of each per thread.
template <typename TIn>
__device__ __forceinline__ void gram(float* lds) {
  const float* const K = lds + kPOffK;
  const float* const Q = lds + kPOffQ;
  float* const A = lds + kPOffA;
  float* const P = lds + kPOffP;
  const int tid = threadIdx.x;
  if constexpr (sizeof(TIn) == 2) {
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ti = wave >> 1, tj = wave & 1;
    const int ra = 32 * ti + (lane & 31);
    const int rb = 32 * tj + (lane & 31);
    const int ko = 8 * (lane >> 5);
    const char* const Kb = reinterpret_cast<const char*>(lds) + kPOffKB;
    auto op = [&](int q, int row, int kk) {   // 8 bf16 of k (q = 0) or q (q = 1)
      return *reinterpret_cast<const bf16x8*>(Kb + q * kPQOffB + row * kPKRowB + 2 * (kk + ko));
    };
    f32x16 acc_k = {}, acc_q = {};
#pragma unroll
    for (int kk = 0; kk < kDK; kk += 16) {
      const bf16x8 b8 = op(0, rb, kk);
      acc_k = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(0, ra, kk), b8, acc_k, 0, 0, 0);
      acc_q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(1, ra, kk), b8, acc_q, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * ti + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      A[row * kTS + 32 * tj + (lane & 31)] = acc_k[r];
      P[row * kTS + 32 * tj + (lane & 31)] = acc_q[r];
    }
  } else {
    static_assert((kC / 2) * (kC / 8) == kThreads, "one 2 x 8 tile per thread");
    const int t0 = (tid / (kC / 8)) * 2;
    const int j0 = (tid % (kC / 8)) * 8;
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
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      A[t0 * kTS + j0 + j] = ak[0][j];
      A[(t0 + 1) * kTS + j0 + j] = ak[1][j];
      P[t0 * kTS + j0 + j] = aq[0][j];
      P[(t0 + 1) * kTS + j0 + j] = aq[1][j];
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

// The gates are kept as loaded (bf16 bits or f32) and widened when staged:
// widening at the load would wait for it there, and with it for every load
// issued before it (the memory counter drains in order).
template <typename TIn>
struct ChunkRegs {
  Raw8<TIn> k[kKQItems], q[kKQItems], v;
  TIn a, b;
};

template <typename TIn> __device__ __forceinline__ TIn gate_one();
template <> __device__ __forceinline__ float gate_one<float>() { return 1.0f; }
template <> __device__ __forceinline__ uint16_t gate_one<uint16_t>() { return 0x3F80; }   // bf16 1.0
template <typename TIn> __device__ __forceinline__ float gate_widen(TIn x);
template <> __device__ __forceinline__ float gate_widen<float>(float x) { return x; }
template <> __device__ __forceinline__ float gate_widen<uint16_t>(uint16_t x) { return bf16_one(x); }

// Issue the loads of the chunk starting at c0 (n positions) into registers:
// k and q of key head g, the gates of value head h, and with WITHV the 16 v
// rows from row0 of value head h.
template <typename TIn, bool WITHV>
__device__ __forceinline__ void fetch_chunk(const ChunkArgs& args, ChunkRegs<TIn>& rg, int r, int h, int g, int row0,
                                            int c0, int n, int tid) {
  const int T = args.n_pos;
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
  if constexpr (WITHV) {
    const int t = tid / (kRows / 8);
    const int i0 = (tid % (kRows / 8)) * 8;
    if (tid < kC * (kRows / 8) && t < n)
      rg.v.load(vg + ((static_cast<size_t>(r) * T + c0 + t) * args.n_vheads + h) * kDK + row0 + i0);
    else
      rg.v.zero();
  }
  rg.a = gate_one<TIn>();
  rg.b = TIn(0);
  if (tid < n) {
    const size_t src = (static_cast<size_t>(r) * T + c0 + tid) * args.n_vheads + h;
    rg.a = static_cast<const TIn*>(args.a)[src];   // the log decay with log gates
    rg.b = static_cast<const TIn*>(args.b)[src];
  }
}

// Pre-pass staging: a fetched chunk's k and q (unscaled) into LDS as f32,
// and a_t, b_t at av/bv.
template <typename TIn, bool LOGG>
__device__ __forceinline__ void stage_chunk(float* lds, const ChunkRegs<TIn>& rg, int n, float* av, float* bv) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kKQItems; ++i) {
    const int e = tid + i * kThreads;
    const int t = e / (kDK / 8);
    const int j = (e % (kDK / 8)) * 8;
    if constexpr (sizeof(TIn) == 2) {
      // bf16: the loaded bits, in rows of kPKRowB bytes (the Gram products
      // read them as their operands).
      char* const Kb = reinterpret_cast<char*>(lds) + kPOffKB;
      *reinterpret_cast<u32x4*>(Kb + t * kPKRowB + 2 * j) = rg.k[i].v;
      *reinterpret_cast<u32x4*>(Kb + kPQOffB + t * kPKRowB + 2 * j) = rg.q[i].v;
    } else {
      float* const Kl = lds + kPOffK;
      float* const Ql = lds + kPOffQ;
      float x[8];
      rg.k[i].widen(x);
      *reinterpret_cast<f32x4*>(Kl + t * kKS + j) = f32x4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f32x4*>(Kl + t * kKS + j + 4) = f32x4{x[4], x[5], x[6], x[7]};
      rg.q[i].widen(x);
      *reinterpret_cast<f32x4*>(Ql + t * kKS + j) = f32x4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f32x4*>(Ql + t * kKS + j + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
  }
  if (tid < kC) {
    // Log-space gates: a_t = exp(g_t) (positions past the span end keep a = 1).
    const float a = gate_widen<TIn>(rg.a);
    av[tid] = (LOGG && tid < n) ? expf(a) : a;
    bv[tid] = gate_widen<TIn>(rg.b);
  }
}

// One output rounded to the nearest bf16 (ties to even; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Pre-pass: one block per (request, value head, chunk) of the segment that
// starts at chunk chunk0 and holds n_seg chunks; record
// ((r * Hv + h) * n_seg + chunk - chunk0) of ws.
template <typename TIn, bool LOGG>
__global__ __launch_bounds__(kThreads) void gdn_chunk_prep_kernel(const ChunkArgs args, float* ws, int chunk0,
                                                                  int n_seg) {
  extern __shared__ float lds[];
  const int T = args.n_pos;
  const int Hv = args.n_vheads;
  const int cl = blockIdx.x % n_seg;
  const int h = (blockIdx.x / n_seg) % Hv;
  const int r = blockIdx.x / (n_seg * Hv);
  const int c0 = (chunk0 + cl) * kC;
  const int n = min(kC, T - c0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  float* const A = lds + kPOffA;
  float* const P = lds + kPOffP;
  float* const Tl = lds + kPOffT;
  float* const Tt = lds + kPOffTt;
  float* const Av = lds + kPOffAv;
  float* const Bv = lds + kPOffBv;
  float* const Gv = lds + kPOffG;
  float* const GC = lds + kPOffGC;
  float* const rec = ws + (static_cast<size_t>(r) * Hv + h) * n_seg * kRecFloats +
                     static_cast<size_t>(cl) * kRecFloats;
  const float p_scale = args.q_scale;

  {
    ChunkRegs<TIn> rg;
    fetch_chunk<TIn, false>(args, rg, r, h, h / args.group, 0, c0, n, threadIdx.x);
    stage_chunk<TIn, LOGG>(lds, rg, n, Av, Bv);
  }
  __syncthreads();
  gram<TIn>(lds);
  __syncthreads();
  // Row t: A[t][j] = b_t G[t][j] (K K^T)[t][j] for j < t (0 elsewhere),
  // P[t][j] = q_scale G[t][j] (q_t . k_j) for j <= t (0 elsewhere), and g_t,
  // where G[t][j] = a_{j+1} ... a_t (1 for j >= t). Four lanes share a row,
  // each 16 columns [16 s, 16 s + 16): a lane multiplies the decays of its
  // own segment into running products from the segment's top down (no
  // division, no logarithm: zero and tiny decays are exact), and the product
  // of the decays above its segment comes from the other three lanes.
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
    float own = 1.0f;   // this segment's decays with index <= t
#pragma unroll
    for (int i = 15; i >= 0; --i) own *= (j0 + i <= t) ? av[i] : 1.0f;
    const int base = tid & ~3;
    float above = 1.0f;   // the segments above, highest first
#pragma unroll
    for (int k = 3; k >= 1; --k) {
      const float o = __shfl(own, base + k);
      if (k > sg) above *= o;
    }
    const float bt = Bv[t];
    float* const arow = A + t * kTS;
    float* const prow = P + t * kTS;
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
        ka[u] = (jj < t) ? bt * gp * kv[u] : 0.0f;
        qa[u] = (jj <= t) ? (p_scale * gp) * qv[u] : 0.0f;
        gc[u] = gp;
      }
      *reinterpret_cast<f32x4*>(arow + j0 + j) = ka;
      *reinterpret_cast<f32x4*>(prow + j0 + j) = qa;
      if (last) *reinterpret_cast<f32x4*>(GC + j0 + j) = gc;
    }
    if (sg == 0) Gv[t] = av[0] * gp;   // g_t = a_0 G[t][0]
  }
  __syncthreads();
  // T = (I + A)^-1 by blocks of 16: T_ii = (I + A_ii)^-1 for the four
  // diagonal blocks (wave i, forward substitution, column j = lane / 4 by the
  // four lanes of a quad: lane s sums the terms k in [4 s, 4 s + 4) and keeps
  // T[k][j] for those k, DPP joins the partial sums), then the blocks below
  // the diagonal level by level, T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, on
  // the matrix cores. Entries of A on and above the diagonal are 0. T is
  // kept row-major and transposed (T^T rows are the columns the products
  // read as 16-byte loads).
  {
    const int col = lane >> 2;
    const int sub = lane & 3;
    const int d0 = 16 * wave;
    float xs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = 0.0f;
      if (i > 0) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(A + (d0 + i) * kTS + d0 + 4 * sub);
        p = __builtin_fmaf(a4.x, xs[0], __builtin_fmaf(a4.y, xs[1], __builtin_fmaf(a4.z, xs[2], a4.w * xs[3])));
      }
      const float x = ((i == col) ? 1.0f : 0.0f) - group_sum<4>(p);
      if (sub == (i >> 2)) xs[i & 3] = x;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) Tl[(d0 + 4 * sub + m) * kTS + d0 + col] = xs[m];
    *reinterpret_cast<f32x4*>(Tt + (d0 + col) * kTS + d0 + 4 * sub) = f32x4{xs[0], xs[1], xs[2], xs[3]};
    // The blocks above the diagonal are never read (the record holds the
    // lower tiles only), so they are left unwritten.
  }
  __syncthreads();
  {
    const int ii = lane & 15;
    const int kq = lane >> 4;
    for (int lev = 1; lev < 4; ++lev) {
      if (wave < 4 - lev) {
        const int bi = wave + lev, bj = wave;
        f32x4 m = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int bk = bj; bk < bi; ++bk) {
          const f32x4 av = *reinterpret_cast<const f32x4*>(A + (16 * bi + ii) * kTS + 16 * bk + 4 * kq);
          const f32x4 tv = *reinterpret_cast<const f32x4*>(Tt + (16 * bj + ii) * kTS + 16 * bk + 4 * kq);
#pragma unroll
          for (int u = 0; u < 4; ++u) m = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], tv[u], m, 0, 0, 0);
        }
        // The product's lanes hold M[4 kq + u][ii], the B operand of the
        // next product in the same lane order.
        const f32x4 td = *reinterpret_cast<const f32x4*>(Tl + (16 * bi + ii) * kTS + 16 * bi + 4 * kq);
        f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) o = __builtin_amdgcn_mfma_f32_16x16x4f32(td[u], m[u], o, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) Tl[(16 * bi + 4 * kq + u) * kTS + 16 * bj + ii] = -o[u];
        *reinterpret_cast<f32x4*>(Tt + (16 * bj + ii) * kTS + 16 * bi + 4 * kq) = f32x4{-o.x, -o.y, -o.z, -o.w};
      }
      __syncthreads();
    }
  }
  // The record: T's lower tiles, g and G[n-1][.] copied out in the reader's
  // order; P T on the matrix cores (16x16x4 f32 MFMA) as the transposed
  // product T^T P^T, whose output lanes hold exactly the reader's 4-column
  // pieces of P T: tile (i, j) sums over the blocks k in [j, i], 20 block
  // products over the 10 tiles, 5 per wave.
  {
    const int i = lane & 15;
    const int kq = lane >> 4;
    for (int c = 0; c <= wave; ++c)
      *reinterpret_cast<f32x4*>(rec + kRecT + tile_index(wave, c) * 256 + 4 * lane) =
          *reinterpret_cast<const f32x4*>(Tl + (16 * wave + i) * kTS + 16 * c + 4 * kq);
    if (tid < 2 * kC / 4)
      *reinterpret_cast<f32x4*>(rec + kRecG + 4 * tid) = *reinterpret_cast<const f32x4*>(Gv + 4 * tid);
  }
  {
    // Tiles per wave, (i, j) packed as 4 i + j; 16 ends a list.
    constexpr uint8_t kPtTiles[4][4] = {{12, 0, 16, 16}, {8, 4, 16, 16}, {13, 9, 16, 16}, {14, 5, 10, 15}};
    const int i = lane & 15;
    const int kq = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tile = kPtTiles[wave][e];
      if (tile == 16) break;
      const int ti = tile >> 2, tj = tile & 3;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int c = 16 * tj; c < 16 * ti + 16; c += 16) {
        const f32x4 tv = *reinterpret_cast<const f32x4*>(Tt + (16 * tj + i) * kTS + c + 4 * kq);
        const f32x4 pv = *reinterpret_cast<const f32x4*>(P + (16 * ti + i) * kTS + c + 4 * kq);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[u], pv[u], acc, 0, 0, 0);
      }
      *reinterpret_cast<f32x4*>(rec + kRecPT + tile_index(ti, tj) * 256 + 4 * lane) = acc;
    }
  }
}

// The pre-pass record of one chunk in registers, in the layout of the
// matrix-core operands that read it: wave w's lane (i, kq) = (lane % 16,
// lane / 16) holds T[16 w + i][16 c + 4 kq + u] for the column blocks c <= w
// and P T[16 (3 - w) + i][16 c + 4 kq + u] for c <= 3 - w (wave w computes
// W for its own positions and the outputs for the mirrored block, w + 1 and
// 4 - w tiles: five per wave); one coalesced 16-byte load per lane and tile.
// The first 32 threads also hold g and G[n-1][.] (4 values each).
struct RecRegs {
  f32x4 t[4], pt[4], g;
};

__device__ __forceinline__ void fetch_rec(const float* rec, RecRegs& rr) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c <= wave) rr.t[c] = *reinterpret_cast<const f32x4*>(rec + kRecT + tile_index(wave, c) * 256 + 4 * lane);
    if (c <= 3 - wave)
      rr.pt[c] = *reinterpret_cast<const f32x4*>(rec + kRecPT + tile_index(3 - wave, c) * 256 + 4 * lane);
  }
  if (tid < 2 * kC / 4) rr.g = *reinterpret_cast<const f32x4*>(rec + kRecG + 4 * tid);
}

// The producer/consumer form's copy of a chunk's pre-pass record into LDS:
// loaded by the 256 producer threads (ptid) into registers, written to the
// input buffer unchanged.
constexpr int kRecVec = kRecFloats / 4;                          // float4 per record
constexpr int kRecVecPerThread = (kRecVec + kThreads - 1) / kThreads;
static_assert(kRecFloats % 4 == 0, "whole float4 records");

__device__ __forceinline__ void fetch_rec_pc(const float* rec, f32x4 (&rr)[kRecVecPerThread], int ptid) {
#pragma unroll
  for (int k = 0; k < kRecVecPerThread; ++k) {
    const int i = ptid + k * kThreads;
    if (i < kRecVec) rr[k] = reinterpret_cast<const f32x4*>(rec)[i];
  }
}

__device__ __forceinline__ void stage_rec_pc(float* recl, const f32x4 (&rr)[kRecVecPerThread], int ptid) {
#pragma unroll
  for (int k = 0; k < kRecVecPerThread; ++k) {
    const int i = ptid + k * kThreads;
    if (i < kRecVec) reinterpret_cast<f32x4*>(recl)[i] = rr[k];
  }
}

// Sequential staging of a fetched chunk into an input buffer: k and q (bf16
// as loaded, or f32), the block's v rows and a_t, b_t as f32 (tid: the
// staging thread, 0 .. kThreads - 1).
template <typename TIn, bool LOGG>
__device__ __forceinline__ void stage_seq(char* lds, const ChunkRegs<TIn>& rg, int n, int tid) {
  using L = SeqLds<sizeof(TIn) == 2>;
#pragma unroll
  for (int i = 0; i < kKQItems; ++i) {
    const int e = tid + i * kThreads;
    const int t = e / (kDK / 8);
    const int j = (e % (kDK / 8)) * 8;
    char* const kd = lds + L::K + t * L::kKRow;
    char* const qd = lds + L::Q + t * L::kKRow;
    if constexpr (sizeof(TIn) == 2) {
      *reinterpret_cast<u32x4*>(kd + 2 * j) = rg.k[i].v;
      *reinterpret_cast<u32x4*>(qd + 2 * j) = rg.q[i].v;
    } else {
      *reinterpret_cast<f32x4*>(kd + 4 * j) = rg.k[i].a;
      *reinterpret_cast<f32x4*>(kd + 4 * j + 16) = rg.k[i].b;
      *reinterpret_cast<f32x4*>(qd + 4 * j) = rg.q[i].a;
      *reinterpret_cast<f32x4*>(qd + 4 * j + 16) = rg.q[i].b;
    }
  }
  if (tid < kC * (kRows / 8)) {
    float x[8];
    rg.v.widen(x);
    float* const lv = reinterpret_cast<float*>(lds + L::V) + (tid / (kRows / 8)) * kRows + (tid % (kRows / 8)) * 8;
    *reinterpret_cast<f32x4*>(lv) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(lv + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
  if (tid < kC) {
    // Log-space gates: a_t = exp(g_t) (positions past the span end keep a = 1).
    const float a = gate_widen<TIn>(rg.a);
    reinterpret_cast<float*>(lds + L::AV)[tid] = (LOGG && tid < n) ? expf(a) : a;
    reinterpret_cast<float*>(lds + L::BV)[tid] = gate_widen<TIn>(rg.b);
  }
}

// f32 x as hi + mid + lo, three bf16 values whose sum is x exactly (x
// finite): hi keeps the top 8 significant bits, x - hi (exact) the next 16,
// split the same way; the last 8 bits fit a bf16 as they are.
__device__ __forceinline__ void split3(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t hb = __float_as_uint(x) & 0xFFFF0000u;
  const float r1 = x - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mb);
  h = hb >> 16;
  m = mb >> 16;
  l = __float_as_uint(r2) >> 16;
}

// One value of row t of the staged k, column c, as f32.
template <bool BF>
__device__ __forceinline__ float k_at(const char* lds, int t, int c) {
  using L = SeqLds<BF>;
  if constexpr (BF)
    return bf16_one(*reinterpret_cast<const uint16_t*>(lds + L::K + t * L::kKRow + 2 * c));
  else
    return *reinterpret_cast<const float*>(lds + L::K + t * L::kKRow + 4 * c);
}

// Four consecutive values of row t of the staged k from column c (c % 4 == 0).
template <bool BF>
__device__ __forceinline__ f32x4 k4_at(const char* lds, int t, int c) {
  using L = SeqLds<BF>;
  if constexpr (BF) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(lds + L::K + t * L::kKRow + 2 * c);
    return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  } else {
    return *reinterpret_cast<const f32x4*>(lds + L::K + t * L::kKRow + 4 * c);
  }
}

// Four 16-bit values by the gfx950 transposing LDS read (ds_read_b64_tr_b16):
// within each group of 16 lanes, lane i receives, as its j-th value, element
// i % 4 of the four consecutive 16-bit values that lane 4 j + i / 4 of the
// group addresses (p: 8-byte aligned, in LDS).
__device__ __forceinline__ u32x2 ds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Sequential pass over the segment's chunks. init: the state the segment
// starts from, request r's rows at init + r * init_rstride (the state
// buffer, or with capture the checkpoint before the segment). LOGG: `a`
// holds log decays; OUTBF: outputs are written as bf16. PC: 4 further
// producer waves load chunk c + 2 and stage chunk c + 1 into the other of two
// input buffers while the 4 compute waves process chunk c (the staging then
// leaves the compute waves' path; every barrier is shared by both roles).
template <typename TIn, bool CAPTURE, bool LOGG, bool OUTBF, bool PC>
__global__ __launch_bounds__(PC ? 2 * kThreads : kThreads) void gdn_chunked_kernel(const ChunkArgs args,
                                                                                  const float* ws, int chunk0,
                                                                                  int n_seg, const float* init,
                                                                                  size_t init_rstride) {
  constexpr bool BF = sizeof(TIn) == 2;
  static_assert(!PC || BF, "two f32 input buffers do not fit in LDS");
  using L = SeqLds<BF, PC>;
  extern __shared__ float lds_f[];
  char* const lds = reinterpret_cast<char*>(lds_f);
  const int T = args.n_pos;
  const int Hv = args.n_vheads;
  const int n_heads = args.n_req * Hv;
  // Block order: head-major with the 8 row blocks of a head on one XCD when
  // the head count allows it (block b runs on XCD b % 8).
  int hh, rb;
  if ((n_heads & 7) == 0) {
    const int x = blockIdx.x & 7;
    const int sl = blockIdx.x >> 3;
    hh = x + 8 * (sl >> 3);
    rb = sl & 7;
  } else {
    hh = blockIdx.x / kRowBlocks;
    rb = blockIdx.x % kRowBlocks;
  }
  const int row0 = rb * kRows;
  const int h = hh % Hv;
  const int r = hh / Hv;
  const int g = h / args.group;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane % kLPR;
  const int kq = lane >> 4;
  const int srow = lane & 15;
  const int row_blk = wave * (64 / kLPR) + lane / kLPR;   // 0..15
  const size_t head_elems = static_cast<size_t>(kDK) * kDK;
  const size_t pos_stride = static_cast<size_t>(Hv) * head_elems;
  const bool compute = !PC || tid < kThreads;   // wave-uniform
  const int ptid = tid - kThreads;              // producer index (PC)
  float* const S0 = reinterpret_cast<float*>(lds + L::S0);
  float* const Yt = reinterpret_cast<float*>(lds + L::Y);
  float* const Wt = reinterpret_cast<float*>(lds + L::W);
  float* const GvC = reinterpret_cast<float*>(lds + L::G);   // without PC: g_t and G[n-1][t] of the chunk
  float* const GCC = reinterpret_cast<float*>(lds + L::GC);
  const float* const rec0 = ws + (static_cast<size_t>(r) * Hv + h) * n_seg * kRecFloats;

  const size_t row_off = static_cast<size_t>(h) * head_elems + static_cast<size_t>(row0 + row_blk) * kDK;
  const float* const init_row = init + r * init_rstride + row_off;
  float* const state_row = args.state + static_cast<size_t>(r) * pos_stride + row_off;
  float* const ckpt_row0 = CAPTURE ? args.ckpt + static_cast<size_t>(r) * T * pos_stride + row_off : nullptr;
  const size_t out_h = (static_cast<size_t>(r) * T * Hv + h) * kDK + row0;   // element offset

  f32x4 s[kNCH];
  if (compute) {
#pragma unroll
    for (int m = 0; m < kNCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(init_row + 4 * (li + kLPR * m));
  }

  // A chunk's outputs wait in registers until the next chunk is staged:
  // stored right away they would sit in the memory counter in front of the
  // next chunk's prefetched loads, and staging would wait for them too.
  f32x4 o_pend = {0.0f, 0.0f, 0.0f, 0.0f};
  size_t o_elem = 0;   // element of the first pending output
  int o_cnt = 0;       // pending outputs (positions of this lane still in the span)
  auto store_pending = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < o_cnt) {
        const size_t e = o_elem + static_cast<size_t>(u) * Hv * kDK;
        if constexpr (OUTBF)
          static_cast<uint16_t*>(args.out)[e] = static_cast<uint16_t>(bf16_rne(o_pend[u]));
        else
          static_cast<float*>(args.out)[e] = o_pend[u];
      }
    }
  };

  ChunkRegs<TIn> rg;
  RecRegs cur, nxt;                       // without PC: this chunk's and the next chunk's record
  f32x4 rr[kRecVecPerThread];             // PC producers: the record being prefetched
  if constexpr (PC) {
    // The producers stage the first chunk and its record, and fetch the second.
    if (!compute) {
      fetch_chunk<TIn, true>(args, rg, r, h, g, row0, chunk0 * kC, min(kC, T - chunk0 * kC), ptid);
      fetch_rec_pc(rec0, rr, ptid);
      stage_seq<TIn, LOGG>(lds, rg, min(kC, T - chunk0 * kC), ptid);
      stage_rec_pc(reinterpret_cast<float*>(lds + L::REC), rr, ptid);
      if (n_seg > 1) {
        fetch_chunk<TIn, true>(args, rg, r, h, g, row0, (chunk0 + 1) * kC, min(kC, T - (chunk0 + 1) * kC), ptid);
        fetch_rec_pc(rec0 + kRecFloats, rr, ptid);
      }
    }
  } else {
    fetch_chunk<TIn, true>(args, rg, r, h, g, row0, chunk0 * kC, min(kC, T - chunk0 * kC), tid);
    fetch_rec(rec0, nxt);
  }
  for (int cl = 0; cl < n_seg; ++cl) {
    const int c0 = (chunk0 + cl) * kC;
    const int n = min(kC, T - c0);
    // This chunk's input buffer.
    char* const inb = lds + (PC ? (cl & 1) * L::IN : 0);
    const float* const Vl = reinterpret_cast<const float*>(inb + L::V);
    const float* const Av = reinterpret_cast<const float*>(inb + L::AV);
    const float* const Bv = reinterpret_cast<const float*>(inb + L::BV);
    const float* const recl = reinterpret_cast<const float*>(inb + L::REC);   // PC: the chunk's record
    const float* const Gv = PC ? recl + kRecG : GvC;
    const float* const GC = PC ? recl + kRecGC : GCC;
    __syncthreads();   // the previous chunk's LDS reads are done (PC: this chunk is staged)
    // 1. Stage the fetched chunk (PC: staged already), its decays and the
    //    current state rows (as f32 and, for the bf16 products, as three
    //    bf16 parts), take over the record's T and P T rows, then fetch the
    //    next chunk: its loads complete while this one is processed.
    if constexpr (!PC) stage_seq<TIn, LOGG>(lds, rg, n, tid);
    if (compute) {
      if constexpr (!PC) {
        cur = nxt;
        if (tid < 2 * kC / 4) *reinterpret_cast<f32x4*>(GvC + 4 * tid) = cur.g;
      }
      // The starting state: from the lanes' registers with capture (the
      // rank-1 recurrence keeps it there) and at the segment's first chunk;
      // otherwise the previous chunk's end left it, and its parts, in LDS.
      if (CAPTURE || cl == 0) {
#pragma unroll
        for (int m = 0; m < kNCH; ++m) {
          *reinterpret_cast<f32x4*>(S0 + row_blk * kSS + 4 * (li + kLPR * m)) = s[m];
          if constexpr (BF) {
            uint32_t hp[4], mp[4], lp[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split3(s[m][e], hp[e], mp[e], lp[e]);
            char* const sp = lds + L::SPL + row_blk * L::kSplRow + 2 * 4 * (li + kLPR * m);
            *reinterpret_cast<u32x2*>(sp) = u32x2{hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16)};
            *reinterpret_cast<u32x2*>(sp + kRows * L::kSplRow) =
                u32x2{mp[0] | (mp[1] << 16), mp[2] | (mp[3] << 16)};
            *reinterpret_cast<u32x2*>(sp + 2 * kRows * L::kSplRow) =
                u32x2{lp[0] | (lp[1] << 16), lp[2] | (lp[3] << 16)};
          }
        }
      }
      if constexpr (!PC) {
        if (cl + 1 < n_seg) {
          fetch_chunk<TIn, true>(args, rg, r, h, g, row0, c0 + kC, min(kC, T - c0 - kC), tid);
          fetch_rec(rec0 + static_cast<size_t>(cl + 1) * kRecFloats, nxt);
        }
      }
    }
    __syncthreads();
    const int tb = 16 * wave + 4 * kq;         // this lane's 4 positions of the wave's W tile
    const int tq = 16 * (3 - wave) + 4 * kq;   // and of its output tile (the mirrored block)
    f32x4 qsg;
    if (compute) {
      store_pending();
      // 2. X = K S_0^T and QS = Q S_0^T: wave w takes positions [16 w,
      //    16 w + 16) for all 16 state rows. bf16 inputs: three bf16 products
      //    per operand pair (16x16x32 MFMA: k and q are bf16, S_0 = hi + mid +
      //    lo exactly, each product exact, f32 accumulation); f32 inputs: f32
      //    products (16x16x4 MFMA), lane group kq supplying columns [c + 4 kq,
      //    c + 4 kq + 4) of each 16, so a lane reads its operands as 16-byte
      //    LDS loads. Then Y = b (V - g X), stored transposed, and q_scale g QS
      //    kept in the lanes that hold it.
      {
        const int row = 16 * wave + srow;
        const int qrow = 16 * (3 - wave) + srow;
        f32x4 xk, xq;
        if constexpr (BF) {
          f32x4 xh = {}, xm = {}, xl = {}, qh = {}, qm = {}, ql = {};
#pragma unroll
          for (int c = 0; c < kDK; c += 32) {
            const int col = 2 * (c + 8 * kq);
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(inb + L::K + row * L::kKRow + col);
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(inb + L::Q + qrow * L::kKRow + col);
            const char* const sp = lds + L::SPL + srow * L::kSplRow + col;
            const bf16x8 sh = *reinterpret_cast<const bf16x8*>(sp);
            const bf16x8 sm = *reinterpret_cast<const bf16x8*>(sp + kRows * L::kSplRow);
            const bf16x8 sl = *reinterpret_cast<const bf16x8*>(sp + 2 * kRows * L::kSplRow);
            xh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, sh, xh, 0, 0, 0);
            qh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, sh, qh, 0, 0, 0);
            xm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, sm, xm, 0, 0, 0);
            qm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, sm, qm, 0, 0, 0);
            xl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, sl, xl, 0, 0, 0);
            ql = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, sl, ql, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            xk[u] = (xl[u] + xm[u]) + xh[u];
            xq[u] = (ql[u] + qm[u]) + qh[u];
          }
        } else {
          xk = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          xq = xk;
#pragma unroll 2
          for (int c = 0; c < kDK; c += 16) {
            const f32x4 kv = *reinterpret_cast<const f32x4*>(inb + L::K + row * L::kKRow + 4 * (c + 4 * kq));
            const f32x4 qv = *reinterpret_cast<const f32x4*>(inb + L::Q + qrow * L::kKRow + 4 * (c + 4 * kq));
            const f32x4 sv = *reinterpret_cast<const f32x4*>(S0 + srow * kSS + c + 4 * kq);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              xk = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[u], sv[u], xk, 0, 0, 0);
              xq = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[u], sv[u], xq, 0, 0, 0);
            }
          }
        }
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(Gv + tb);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(Bv + tb);
        const f32x4 gq = *reinterpret_cast<const f32x4*>(Gv + tq);
        f32x4 y;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          y[u] = b4[u] * __builtin_fmaf(-g4[u], xk[u], Vl[(tb + u) * kRows + srow]);
          qsg[u] = (gq[u] * args.q_scale) * xq[u];
        }
        *reinterpret_cast<f32x4*>(Yt + srow * kTS + tb) = y;
      }
    } else if constexpr (PC) {
      // Producers, spread over three barrier intervals so that none of them
      // outlasts the compute waves' step in it: the next chunk's inputs into
      // the other buffer (its reads ended at this chunk's first barrier)...
      if (cl + 1 < n_seg) stage_seq<TIn, LOGG>(lds + ((cl + 1) & 1) * L::IN, rg, min(kC, T - c0 - kC), ptid);
    }
    __syncthreads();
    if (compute) {
      // 3. W = T Y and P T Y in one pass over Y (16x16x4 f32 MFMA), T and
      //    P T lower triangular in 16-position blocks: wave w takes W for its
      //    positions [16 w, 16 w + 16) (column blocks c <= w) and P T Y for
      //    the mirrored block 3 - w (c <= 3 - w), five tiles per wave (the
      //    same block for both took 2, 4, 6 and 8); its T and P T rows are in
      //    registers, PC: read from the staged record. Outputs o = q_scale g
      //    QS + P T Y, stored after the next chunk is staged.
      {
        f32x4 wacc = {}, oacc = {};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool wt = c <= wave, ot = c <= 3 - wave;   // wave-uniform
          if (wt || ot) {
            const f32x4 yv = *reinterpret_cast<const f32x4*>(Yt + srow * kTS + 16 * c + 4 * kq);
            if (wt) {
              const f32x4 tc = PC ? *reinterpret_cast<const f32x4*>(recl + kRecT + tile_index(wave, c) * 256 + 4 * lane)
                                  : cur.t[c];
#pragma unroll
              for (int u = 0; u < 4; ++u) wacc = __builtin_amdgcn_mfma_f32_16x16x4f32(tc[u], yv[u], wacc, 0, 0, 0);
            }
            if (ot) {
              const f32x4 pc = PC ? *reinterpret_cast<const f32x4*>(recl + kRecPT + tile_index(3 - wave, c) * 256 +
                                                                    4 * lane)
                                  : cur.pt[c];
#pragma unroll
              for (int u = 0; u < 4; ++u) oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(pc[u], yv[u], oacc, 0, 0, 0);
            }
          }
        }
        *reinterpret_cast<f32x4*>(Wt + srow * kTS + tb) = wacc;
        if constexpr (BF && !CAPTURE) {
          // The chunk-end state's factors G[n-1][t] w_t as three bf16 parts,
          // once per value (the products read them as operands).
          uint32_t hp[4], mp[4], lp[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) split3(GC[tb + u] * wacc[u], hp[u], mp[u], lp[u]);
          char* const wp = lds + L::WP + srow * L::kWpRow + 2 * tb;
          *reinterpret_cast<u32x2*>(wp) = u32x2{hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16)};
          *reinterpret_cast<u32x2*>(wp + kRows * L::kWpRow) = u32x2{mp[0] | (mp[1] << 16), mp[2] | (mp[3] << 16)};
          *reinterpret_cast<u32x2*>(wp + 2 * kRows * L::kWpRow) = u32x2{lp[0] | (lp[1] << 16), lp[2] | (lp[3] << 16)};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) o_pend[u] = qsg[u] + oacc[u];
        o_elem = out_h + static_cast<size_t>(c0 + tq) * Hv * kDK + srow;
        o_cnt = min(4, max(0, n - tq));
      }
    } else if constexpr (PC) {
      // ... its record, and the loads of the inputs of the chunk after it ...
      if (cl + 1 < n_seg)
        stage_rec_pc(reinterpret_cast<float*>(lds + ((cl + 1) & 1) * L::IN + L::REC), rr, ptid);
      if (cl + 2 < n_seg)
        fetch_chunk<TIn, true>(args, rg, r, h, g, row0, c0 + 2 * kC, min(kC, T - c0 - 2 * kC), ptid);
    }
    __syncthreads();
    if constexpr (PC) {
      // ... and the loads of its record.
      if (!compute && cl + 2 < n_seg) fetch_rec_pc(rec0 + static_cast<size_t>(cl + 2) * kRecFloats, rr, ptid);
    }
    if constexpr (CAPTURE) {
      if (compute) {
        // 4. States: S_t = a_t S_{t-1} + w_t k_t^T, each checkpointed; 8
        //    positions at a time so their LDS reads are issued together.
        for (int t0 = 0; t0 < n; t0 += 8) {
          float at[8], wt[8];
          f32x4 kk[8][kNCH];
          const f32x4 w0 = *reinterpret_cast<const f32x4*>(Wt + row_blk * kTS + t0);
          const f32x4 w1 = *reinterpret_cast<const f32x4*>(Wt + row_blk * kTS + t0 + 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            wt[u] = w0[u];
            wt[u + 4] = w1[u];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            at[u] = Av[t0 + u];
#pragma unroll
            for (int m = 0; m < kNCH; ++m) kk[u][m] = k4_at<BF>(inb, t0 + u, 4 * (li + kLPR * m));
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
      }
    } else {
      if (compute) {
        // 4. State at the chunk end only: S_C = g_{n-1} S_0 + sum_t G[n-1][t]
        //    w_t k_t^T on the matrix cores (wave w takes columns [32 w, 32 w +
        //    32)), every operand read before the first product. bf16 inputs:
        //    the f32 factors G[n-1][t] w_t as the three bf16 parts step 3
        //    wrote, against bf16 k (16x16x32 MFMA, exact products); f32
        //    inputs: 16x16x4 f32 MFMA.
        f32x4 d0 = {}, d1 = {};
        if constexpr (BF) {
          bf16x8 ah[2], am[2], al[2], b0[2], b1[2];
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const int t8 = 32 * c2 + 8 * kq;
            const char* const wp = lds + L::WP + srow * L::kWpRow + 2 * t8;
            ah[c2] = *reinterpret_cast<const bf16x8*>(wp);
            am[c2] = *reinterpret_cast<const bf16x8*>(wp + kRows * L::kWpRow);
            al[c2] = *reinterpret_cast<const bf16x8*>(wp + 2 * kRows * L::kWpRow);
            // k down its columns (positions t8 .. t8 + 7 of columns 32 w + i
            // and 32 w + 16 + i for lane i of the group) by the transposing
            // LDS read: in each group of 16 lanes, lane i of the result takes
            // element i % 4 of the 4 that lane 4 j + i / 4 addressed, as its
            // j-th value; lane s therefore addresses row t8 + s / 4 (+ 4),
            // columns from 32 w + 4 (s % 4) (+ 16).
            const char* const kc = inb + L::K + (t8 + (srow >> 2)) * L::kKRow + 2 * (32 * wave + 4 * (srow & 3));
            const u32x2 k0lo = ds_read_tr16(kc);
            const u32x2 k0hi = ds_read_tr16(kc + 4 * L::kKRow);
            const u32x2 k1lo = ds_read_tr16(kc + 32);
            const u32x2 k1hi = ds_read_tr16(kc + 4 * L::kKRow + 32);
            b0[c2] = __builtin_bit_cast(bf16x8, u32x4{k0lo.x, k0lo.y, k0hi.x, k0hi.y});
            b1[c2] = __builtin_bit_cast(bf16x8, u32x4{k1lo.x, k1lo.y, k1hi.x, k1hi.y});
          }
          f32x4 d0m = {}, d0l = {}, d1m = {}, d1l = {};
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[c2], ah[c2], d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[c2], ah[c2], d1, 0, 0, 0);
            d0m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[c2], am[c2], d0m, 0, 0, 0);
            d1m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[c2], am[c2], d1m, 0, 0, 0);
            d0l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b0[c2], al[c2], d0l, 0, 0, 0);
            d1l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b1[c2], al[c2], d1l, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            d0[u] = (d0l[u] + d0m[u]) + d0[u];
            d1[u] = (d1l[u] + d1m[u]) + d1[u];
          }
        } else {
          f32x4 wv[4];
          float k0[4][4], k1[4][4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int tq = 16 * q4 + 4 * kq;
            const f32x4 gc = *reinterpret_cast<const f32x4*>(GC + tq);
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(Wt + srow * kTS + tq);
            wv[q4] = f32x4{gc.x * w4.x, gc.y * w4.y, gc.z * w4.z, gc.w * w4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              k0[q4][u] = k_at<BF>(inb, tq + u, 32 * wave + srow);
              k1[q4][u] = k_at<BF>(inb, tq + u, 32 * wave + srow + 16);
            }
          }
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(k0[q4][u], wv[q4][u], d0, 0, 0, 0);
              d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(k1[q4][u], wv[q4][u], d1, 0, 0, 0);
            }
          }
        }
        // The products are taken with k as the first operand, so each lane
        // holds four consecutive columns of one row of the result (row srow,
        // columns 32 w + 4 kq .. + 3 and 16 further on): the new state goes
        // over S_0 in place and, for the bf16 products of the next chunk,
        // as its three bf16 parts, written here; the next chunk starts from
        // them without a trip through the lanes' registers.
        const float gn = Gv[n - 1];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const f32x4& d = hf ? d1 : d0;
          const int col = 32 * wave + 16 * hf + 4 * kq;
          float* const e = S0 + srow * kSS + col;
          const f32x4 old = *reinterpret_cast<const f32x4*>(e);
          f32x4 nv;
#pragma unroll
          for (int u = 0; u < 4; ++u) nv[u] = __builtin_fmaf(gn, old[u], d[u]);
          *reinterpret_cast<f32x4*>(e) = nv;
          if constexpr (BF) {
            uint32_t hp[4], mp[4], lp[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) split3(nv[u], hp[u], mp[u], lp[u]);
            char* const sp = lds + L::SPL + srow * L::kSplRow + 2 * col;
            *reinterpret_cast<u32x2*>(sp) = u32x2{hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16)};
            *reinterpret_cast<u32x2*>(sp + kRows * L::kSplRow) = u32x2{mp[0] | (mp[1] << 16), mp[2] | (mp[3] << 16)};
            *reinterpret_cast<u32x2*>(sp + 2 * kRows * L::kSplRow) =
                u32x2{lp[0] | (lp[1] << 16), lp[2] | (lp[3] << 16)};
          }
        }
      }
    }
  }
  if constexpr (!CAPTURE) {
    // The state after the segment, from S_0 into the lanes that own its rows.
    __syncthreads();
    if (compute) {
#pragma unroll
      for (int m = 0; m < kNCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(S0 + row_blk * kSS + 4 * (li + kLPR * m));
    }
  }
  if (compute) {
    store_pending();
    if (!CAPTURE) {
#pragma unroll
      for (int m = 0; m < kNCH; ++m) *reinterpret_cast<f32x4*>(state_row + 4 * (li + kLPR * m)) = s[m];
    }
  }
}

template <typename TIn, bool CAPTURE, bool LOGG, bool OUTBF, bool PC>
void launch_seq_kernel(const ChunkArgs& args, const float* ws, int chunk0, int n_seg, const float* init,
                       size_t init_rstride, hipStream_t s) {
  const int blocks = args.n_req * args.n_vheads * kRowBlocks;
  constexpr size_t lds = SeqLds<sizeof(TIn) == 2, PC>::BYTES;
  hipLaunchKernelGGL((gdn_chunked_kernel<TIn, CAPTURE, LOGG, OUTBF, PC>), dim3(blocks),
                     dim3(PC ? 2 * kThreads : kThreads), lds, s, args, ws, chunk0, n_seg, init, init_rstride);
}

// LDS bytes a block may use on the current device, queried once per device
// and thread (0 when the query fails).
int max_lds_per_block() {
  thread_local int cached_dev = -1;
  thread_local int cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) v = 0;
    cached = v;
    cached_dev = dev;
  }
  return cached;
}

// Segments of several chunks with bf16 inputs take the producer/consumer
// form where its LDS fits (151,552 bytes; gfx950 blocks may use 160 KiB); a
// single chunk has nothing to stage ahead (and the smaller form fits two
// blocks per CU), and two f32 input buffers would not fit in LDS.
template <typename TIn, bool CAPTURE, bool LOGG>
hipError_t launch_seq(const ChunkArgs& args, const float* ws, int chunk0, int n_seg, const float* init,
                      size_t init_rstride, bool out_bf16, hipStream_t s) {
  constexpr bool BF = sizeof(TIn) == 2;
  const bool pc = BF && n_seg > 1 && max_lds_per_block() >= static_cast<int>(SeqLds<true, true>::BYTES);
  if (out_bf16) {
    if (pc) launch_seq_kernel<TIn, CAPTURE, LOGG, true, BF>(args, ws, chunk0, n_seg, init, init_rstride, s);
    else launch_seq_kernel<TIn, CAPTURE, LOGG, true, false>(args, ws, chunk0, n_seg, init, init_rstride, s);
  } else {
    if (pc) launch_seq_kernel<TIn, CAPTURE, LOGG, false, BF>(args, ws, chunk0, n_seg, init, init_rstride, s);
    else launch_seq_kernel<TIn, CAPTURE, LOGG, false, false>(args, ws, chunk0, n_seg, init, init_rstride, s);
  }
  return launch_error();
}

// One segment: the pre-pass of its chunks, then the sequential pass.
template <typename TIn, bool LOGG>
hipError_t launch_segment(const ChunkArgs& args, float* ws, int chunk0, int n_seg, const float* init,
                          size_t init_rstride, bool capture, bool out_bf16, hipStream_t s) {
  const int pblocks = args.n_req * args.n_vheads * n_seg;
  hipLaunchKernelGGL((gdn_chunk_prep_kernel<TIn, LOGG>), dim3(pblocks), dim3(kThreads), kPLdsBytes, s, args, ws,
                     chunk0, n_seg);
  const hipError_t e = launch_error();
  if (e != hipSuccess) return e;
  return capture ? launch_seq<TIn, true, LOGG>(args, ws, chunk0, n_seg, init, init_rstride, out_bf16, s)
                 : launch_seq<TIn, false, LOGG>(args, ws, chunk0, n_seg, init, init_rstride, out_bf16, s);
}

template <typename TIn>
hipError_t launch_chunked(const ChunkArgs& args, float* ws, bool capture, bool log_gates, bool out_bf16,
                          hipStream_t s) {
  const int n_chunks = (args.n_pos + kC - 1) / kC;
  const size_t pos_stride = static_cast<size_t>(args.n_vheads) * kDK * kDK;
  for (int chunk0 = 0; chunk0 < n_chunks; chunk0 += kSegChunks) {
    const int n_seg = std::min(kSegChunks, n_chunks - chunk0);
    // The first segment starts from `state`; later ones from the state after
    // the previous segment: `state` itself without capture (updated in
    // place), the checkpoint of the position before the segment with.
    const float* init = args.state;
    size_t init_rstride = pos_stride;
    if (capture && chunk0 > 0) {
      init = args.ckpt + static_cast<size_t>(chunk0 * kC - 1) * pos_stride;
      init_rstride = static_cast<size_t>(args.n_pos) * pos_stride;
    }
    const hipError_t e =
        log_gates ? launch_segment<TIn, true>(args, ws, chunk0, n_seg, init, init_rstride, capture, out_bf16, s)
                  : launch_segment<TIn, false>(args, ws, chunk0, n_seg, init, init_rstride, capture, out_bf16, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t workspace_bytes(int n_req, int n_vheads, int n_pos) {
  const int n_chunks = (n_pos + kC - 1) / kC;
  return static_cast<size_t>(n_req) * n_vheads * std::min(n_chunks, kSegChunks) * kRecFloats * sizeof(float);
}

}  // namespace
}  // namespace hrs

using namespace hrs;

extern "C" size_t gdn_span_chunked_workspace_bytes(const hrs_chunked_desc* cd) {
  if (cd == nullptr) return 0;
  const hrs_gdn_desc* d = &cd->gdn;
  if (d->n_req < 1 || d->n_vheads < 1 || d->n_pos < 1 || d->n_pos > HRS_MAX_CHUNKED_POS) return 0;
  return workspace_bytes(d->n_req, d->n_vheads, d->n_pos);
}

extern "C" int gdn_span_chunked(const hrs_chunked_desc* cd, const void* q, const void* k, const void* v,
                                const void* a, const void* b, float* state, float* ckpt, void* out, void* workspace,
                                size_t workspace_bytes_given, void* stream) {
  if (cd == nullptr) return HRS_EINVAL;
  const hrs_gdn_desc* d = &cd->gdn;
  if (d->n_req < 1 || d->n_kheads < 1 || d->n_vheads < 1 || d->d_k < 1 || d->d_v < 1) return HRS_EINVAL;
  if (d->n_vheads % d->n_kheads != 0) return HRS_EINVAL;
  if (!dtype_ok(d->in_dtype) || !dtype_ok(cd->out_dtype)) return HRS_EINVAL;
  if (d->topo != HRS_CHAIN) return d->topo == HRS_TREE ? HRS_EUNSUPPORTED : HRS_EINVAL;
  if (d->n_pos < 1 || d->n_pos > HRS_MAX_CHUNKED_POS) return HRS_EINVAL;
  if (!q || !k || !v || !a || !b || !state || !out || !workspace) return HRS_EINVAL;
  if (static_cast<int64_t>(d->n_req) * d->n_vheads * kRowBlocks > (1 << 30)) return HRS_EINVAL;
  if (static_cast<int64_t>(d->n_req) * d->n_vheads * kSegChunks > (1 << 30)) return HRS_EINVAL;
  if (workspace_bytes_given < workspace_bytes(d->n_req, d->n_vheads, d->n_pos)) return HRS_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) || !aligned16(state) ||
      !aligned16(out) || (ckpt && !aligned16(ckpt)) || !aligned16(workspace))
    return HRS_EALIGN;
  if (d->d_k != kDK || d->d_v != kDK) return HRS_EUNSUPPORTED;

  ChunkArgs args;
  args.q = q; args.k = k; args.v = v; args.a = a; args.b = b;
  args.state = state; args.ckpt = ckpt; args.out = out;
  args.n_req = d->n_req; args.n_pos = d->n_pos; args.n_kheads = d->n_kheads; args.n_vheads = d->n_vheads;
  args.group = d->n_vheads / d->n_kheads; args.q_scale = d->q_scale;
  const bool logg = cd->log_gates != 0;
  const bool obf = cd->out_dtype == HRS_BF16;
  float* ws = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const hipError_t e = d->in_dtype == HRS_BF16 ? launch_chunked<uint16_t>(args, ws, ckpt != nullptr, logg, obf, s)
                                               : launch_chunked<float>(args, ws, ckpt != nullptr, logg, obf, s);
  return e == hipSuccess ? HRS_OK : HRS_EDEVICE;
}
