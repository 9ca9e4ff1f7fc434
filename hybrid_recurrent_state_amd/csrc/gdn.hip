// gdn_verify_span: the gated delta rule over a verify span with an F32
// state checkpoint after every position.
//
// Recurrence (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025):
//   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
// evaluated as u = S k, S' = a S + b (v - a u) k^T. Checkpoint capture at
// every verified position follows lucebox PR #506 ("perf(dflash):
// split-chain fast rollback with F32 SSM checkpoints"), Summary and
// Verification (every intermediate state written to a persist buffer);
// draft-tree verification follows lucebox PR #533 (DDTree).
//
// MI355X design
//  * The d_v rows of S evolve independently given (k, a, b, v_row), so one
//    head is split into row units: a wave owns 4 rows, 16 lanes per row, and
//    each lane keeps its DK/16 columns of S in VGPRs for the whole span. No
//    MFMA: the span is bound by checkpoint writes (about 1.6 flop per byte),
//    far below the fp32 ridge point.
//  * Lane l of a row owns float4 chunks l, l+16, ... of the row, so one store
//    instruction writes 16 consecutive 16-byte chunks per row: whole 128-byte
//    lines. Checkpoints are not read again until rollback: they are written
//    with streaming stores (normal stores measured ~12% slower), in chain
//    spans with the device-scope bit as well (2% faster again).
//  * Work order: units are numbered row block fastest, then head, then
//    request, and a block walks units W, W + n_blocks, ... When there are at
//    least as many 32-row units as compute units, the grid is one block per
//    CU with 8 row-owning waves: all CUs then advance through the positions
//    together and each position's checkpoint region (2 MiB per request) is
//    written as one contiguous sweep (5.1 TB/s for one block per unit on the
//    16-request Qwen shape, 5.9 TB/s this way: 73% of HBM peak and 85% of a
//    plain device store stream on the same GPU). Smaller problems use one
//    4-wave block per 16-row unit to spread over more CUs.
//  * The two row dot products (S k and S q) are butterfly sums over the 16
//    lanes with DPP moves; the association order is fixed, so the arithmetic
//    of a position never depends on span length, topology or launch shape.
//  * k, q (times q_scale), v rows, a and b of a window of positions are
//    staged into LDS as f32. In the capturing chain kernel 4 extra producer
//    waves stage the next window (and the next unit's initial state rows)
//    into a double buffer while the row-owning waves run the current one:
//    the vector-memory counter retires loads and stores in order, so a wave
//    that staged its own inputs would wait for all its outstanding
//    checkpoint stores first; split by role, the storing waves load nothing.
//  * Tree mode: the host turns each request's parent array into a stash
//    schedule. A position with a child that is not the next position saves
//    its state rows into an LDS slot (each lane its own 32 bytes, addressed
//    by the wave-uniform slot index, so there are no selects and no extra
//    registers); the child restores from the slot instead of re-reading the
//    parent's checkpoint. Up to 8 slots, as many as fit beside the staging
//    buffer. Trees that need more live slots use a kernel variant that
//    reloads the parent's checkpoint rows (this lane's own earlier writes);
//    only that variant has a vector-memory load inside the position loop.
//    The root starts from `state`.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.h"
#include "internal.h"

namespace hrs {
namespace {

constexpr int kLanesPerRow = 16; // lanes sharing one row of S
// s_waitcnt immediate for gfx9-family: vmcnt = 0, expcnt and lgkmcnt left at
// their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kWindow = 32;      // positions staged in LDS at a time

// LDS floats per staged position: k, q (scaled), the unit's v rows, a, b and,
// for trees, the tree code. Chain spans use the unpadded stride, so every
// other position's k and q rows are 8-byte aligned and are read with 16-byte
// LDS reads that the hardware splits; a 16-byte-aligned stride (and a layout
// with separate k, q and v arrays) measured 3% and 7% slower on the
// 16-request Qwen shape. Tree spans need the extra code word and pad to 16 bytes.
constexpr int pos_floats(int dk, int rows, bool tree) {
  return tree ? (2 * dk + rows + 3 + 3) / 4 * 4 : 2 * dk + rows + 2;
}

// LDS floats of one staging buffer (rounded to 16 bytes).
constexpr int staging_floats(int window, int pos_fl) { return (window * pos_fl + 3) / 4 * 4; }

constexpr size_t staging_bytes(int dk, int rows, int window, bool tree) {
  return static_cast<size_t>(staging_floats(window, pos_floats(dk, rows, tree))) * sizeof(float);
}

// Producer waves of the capturing chain kernel (one per SIMD).
constexpr int kProducerWaves = 4;

// LDS bytes of the producer/consumer kernel: two staging buffers, one unit's
// state rows and a flag word.
constexpr size_t pipelined_bytes(int dk, int rows, int window) {
  return 2 * staging_bytes(dk, rows, window, false) + (static_cast<size_t>(rows) * dk + 4) * sizeof(float);
}

// LDS bytes of one tree stash slot: every lane's dk / 16 floats of its row.
constexpr size_t slot_bytes(int dk, int waves) { return static_cast<size_t>(waves) * 64 * (dk / 16) * sizeof(float); }

// Kernel arguments of one launch. Every per-request pointer is offset to the
// launch's first request (req0), so the kernel indexes requests from 0.
struct GdnArgs {
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
  int32_t d_v;
  int32_t group;   // Hv / Hk
  int32_t req0;    // first request of this launch
  int32_t n_units; // row units of this launch: (d_v / rows per unit) * Hv * requests
  int32_t n_blocks; // blocks of this launch (block W walks units W, W + n_blocks, ...)
  int32_t window;  // positions staged in LDS at a time (min(n_pos, kWindow))
  float q_scale;
  // Zero-copy source of the initial state (gdn_verify_span_from): when
  // src_ckpt is set, request r starts from src_ckpt[r][src_node[r]].
  const float* src_ckpt;
  const int32_t* src_node;
  int32_t src_npos;
  int32_t n_req_total;
  const int32_t* src_node_all;  // src_node of the whole call (not offset), for the status count
  int32_t* status;  // optional: number of requests whose src_node is out of range
  // Fused layer (gdn_layer_verify_span): conv input, weights and state; q, k
  // and v are computed from them instead of read.
  const void* x;           // [R][T][C], C = 2*Hk*dk + Hv*dv, channels [q | k | v]
  const void* conv_w;      // [C][4]
  const void* conv_state;  // [R][3][C]
  int32_t conv_c;
  int32_t silu;
  float l2_eps;
  // Tree mode, for the n = geom_req requests of this launch, each array
  // [n][n_pos]: parent index at 0, restore code at n*T, save slot at 2*n*T
  // (gdn_tree_schedule); fused layers add the conv window sources
  // [n][n_pos][3] at 3*n*T (conv_window_sources).
  int32_t geom_req;
  int8_t geom[kGeomBytes];
};

// What the first loads of a launch need: the input pointers and the shape.
// They travel as leading scalar kernel arguments, which the hardware places
// in SGPRs before the first instruction (kernel-argument preloading, enabled
// for this file at build time), so the first data loads wait for no argument
// load; the rest of GdnArgs is loaded alongside them. Pointers as in GdnArgs
// (offset to the launch's first request).
struct Hot {
  const void* in0;     // q, or the conv input x (fused layer)
  const void* in1;     // k, or the conv weights
  const void* in2;     // v, or the conv state
  const void* a;
  const void* b;
  const float* state;  // initial state; nullptr when the span starts from a source checkpoint
  int n_pos;
  int n_kheads;
  int n_vheads;
  int d_v;
  int group;           // Hv / Hk
};

// The shape packed into two argument words: word A = n_pos | (d_v / 16) << 7 |
// n_vheads << 12 (n_pos <= 64, d_v <= 256, n_vheads < 2^20), word B = n_kheads.
inline uint32_t shape_word_a(int n_pos, int d_v, int n_vheads) {
  return static_cast<uint32_t>(n_pos) | (static_cast<uint32_t>(d_v / 16) << 7) | (static_cast<uint32_t>(n_vheads) << 12);
}

__device__ __forceinline__ Hot make_hot(const void* in0, const void* in1, const void* in2, const void* a,
                                        const void* b, const float* state, uint32_t wa, uint32_t wb) {
  Hot h;
  h.in0 = in0; h.in1 = in1; h.in2 = in2; h.a = a; h.b = b; h.state = state;
  h.n_pos = static_cast<int>(wa & 0x7Fu);
  h.d_v = static_cast<int>((wa >> 7) & 0x1Fu) * 16;
  h.n_vheads = static_cast<int>(wa >> 12);
  h.n_kheads = static_cast<int>(wb);
  h.group = h.n_vheads / h.n_kheads;
  return h;
}

// One row unit: rows [row0, row0 + RPB) of value head h of request r (the
// index within this launch, which every launch pointer is offset to).
struct Unit {
  int r;     // request within this launch (geometry tables are per launch too)
  int h;     // value head
  int g;     // key head
  int row0;  // first row
};

// Units are numbered row block fastest, then value head, then request.
__device__ __forceinline__ Unit unit_of(const Hot& hs, int W, int rpb) {
  const int nrb = hs.d_v / rpb;
  Unit u;
  u.row0 = (W % nrb) * rpb;
  u.h = (W / nrb) % hs.n_vheads;
  u.r = W / (nrb * hs.n_vheads);
  u.g = u.h / hs.group;
  return u;
}

// Staging, plain inputs: k and q (times q_scale) of key head g and the unit's
// v rows for positions [t0, t0 + tn), 8 elements per item, by the NTH staging
// threads (p is the thread's index among them). q/k and v items share one
// index space, so the staging takes as few rounds of loads as possible.
template <int DK, int NTH, int RPB, int POS_FLOATS, typename TIn>
__device__ __forceinline__ void stage_plain(const GdnArgs& args, const Hot& hs, float* buf, const Unit& u, int t0,
                                            int tn, int p) {
  const int T = hs.n_pos;
  const TIn* qg = static_cast<const TIn*>(hs.in0);
  const TIn* kg = static_cast<const TIn*>(hs.in1);
  const TIn* vg = static_cast<const TIn*>(hs.in2);
  constexpr int V8 = DK / 8;
  constexpr int R8 = RPB / 8;
  const int n_qk = tn * V8;
  const int total = n_qk + tn * R8;
  for (int e = p; e < total; e += NTH) {
    if (e < n_qk) {
      const int tt = e / V8;
      const int j = (e % V8) * 8;
      const size_t src = ((static_cast<size_t>(u.r) * T + t0 + tt) * hs.n_kheads + u.g) * DK + j;
      float kv[8], qv[8];
      load8<TIn>(kg + src, kv);
      load8<TIn>(qg + src, qv);
      float* lk = buf + tt * POS_FLOATS + j;
      float* lq = lk + DK;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lk[i] = kv[i];
        lq[i] = qv[i] * args.q_scale;
      }
    } else {
      const int ev = e - n_qk;
      const int tt = ev / R8;
      const int i0 = (ev % R8) * 8;
      const size_t src =
          ((static_cast<size_t>(u.r) * T + t0 + tt) * hs.n_vheads + u.h) * hs.d_v + u.row0 + i0;
      float vv[8];
      load8<TIn>(vg + src, vv);
      float* lv = buf + tt * POS_FLOATS + 2 * DK + i0;
#pragma unroll
      for (int i = 0; i < 8; ++i) lv[i] = vv[i];
    }
  }
}

// Sixteen consecutive elements as loaded (bf16 bits or f32; the source must
// be 16-byte aligned), widened one at a time where they are used: the raw
// form of bf16 takes half the registers of f32.
template <typename TIn> struct Raw16;
template <> struct Raw16<uint16_t> {
  u32x4 v[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    v[0] = reinterpret_cast<const u32x4*>(p)[0];
    v[1] = reinterpret_cast<const u32x4*>(p)[1];
  }
  __device__ __forceinline__ float at(int c) const {
    const uint32_t w = v[c >> 3][(c >> 1) & 3];
    return (c & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <> struct Raw16<float> {
  f32x4 v[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const f32x4*>(p)[i];
  }
  __device__ __forceinline__ float at(int c) const { return v[c >> 2][c & 3]; }
};

// Staging, fused layer: for every staged position, the conv (and SiLU) of
// the unit's channels, written where the plain staging puts q, k and v: q
// and k of key head g scaled to unit L2 norm (q also by q_scale), and the
// unit's v rows. One item is 16 channels of one position; the DK / 16 items
// of a q or k row sit in adjacent lanes, so the row's sum of squares is a DPP
// group sum and the normalisation needs no extra pass or barrier. Window rows
// come from x or the conv state: for a chain position t they are positions
// t-3..t-1 (conv-state row t+m when negative); for a tree the host table
// names them. Weight w[c][3] multiplies the current input.
template <int DK, int NTH, int RPB, int POS_FLOATS, typename TIn, bool TREE>
__device__ __forceinline__ void stage_fused(const GdnArgs& args, const Hot& hs, float* buf, const Unit& u, int t0,
                                            int tn, int p) {
  constexpr int CPI = 16;            // channels per item
  constexpr int QL = DK / CPI;       // items of one q or k row (4 or 8: a DPP group)
  constexpr int VI = RPB / CPI;      // items of the unit's v rows at one position
  static_assert(QL == 4 || QL == 8, "q/k row items form a DPP group");
  static_assert(NTH % QL == 0, "staging threads cover whole q/k rows");
  const int T = hs.n_pos;
  const int C = args.conv_c;
  const int Hk = hs.n_kheads;
  const TIn* x = static_cast<const TIn*>(hs.in0);
  const TIn* wc = static_cast<const TIn*>(hs.in1);
  const TIn* cs = static_cast<const TIn*>(hs.in2);
  const int n_qk = tn * 2 * QL;
  const int total = n_qk + tn * VI;
  for (int e = p; e < total; e += NTH) {
    int tt, ch, part;   // part: 0 q, 1 k, 2 v
    float* dst;
    if (e < n_qk) {
      const int row = e / QL;
      const int cg = e % QL;
      tt = row >> 1;
      part = row & 1;
      ch = part * Hk * DK + u.g * DK + cg * CPI;
      dst = buf + tt * POS_FLOATS + (part ? 0 : DK) + cg * CPI;   // k first, then q
    } else {
      const int i = e - n_qk;
      tt = i / VI;
      part = 2;
      ch = 2 * Hk * DK + u.h * hs.d_v + u.row0 + (i % VI) * CPI;
      dst = buf + tt * POS_FLOATS + 2 * DK + (i % VI) * CPI;
    }
    const int t = t0 + tt;
    Raw16<TIn> win[4];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      int src;
      if constexpr (TREE) {
        src = args.geom[3 * args.geom_req * T + (u.r * T + t) * 3 + m];
      } else {
        const int sq = t - 3 + m;
        src = sq >= 0 ? sq : -1 - (t + m);
      }
      const TIn* ptr = src >= 0 ? x + (static_cast<size_t>(u.r) * T + src) * C + ch
                                : cs + (static_cast<size_t>(u.r) * 3 + (-1 - src)) * C + ch;
      win[m].load(ptr);
    }
    win[3].load(x + (static_cast<size_t>(u.r) * T + t) * C + ch);
    Raw16<TIn> w[4];   // w[c][m] is element 4 c + m of the 64 weights
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i].load(wc + static_cast<size_t>(ch) * 4 + CPI * i);
    float y[CPI];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPI; ++c) {
      float acc = w[c >> 2].at(4 * (c & 3)) * win[0].at(c);
#pragma unroll
      for (int m = 1; m < 4; ++m) acc = __builtin_fmaf(w[c >> 2].at(4 * (c & 3) + m), win[m].at(c), acc);
      y[c] = args.silu ? silu_fast(acc) : acc;
      ss = __builtin_fmaf(y[c], y[c], ss);
    }
    if (part < 2) {
      // Every lane of a row's group takes this branch together (n_qk and the
      // loop stride are multiples of QL).
      ss = group_sum<QL>(ss);
      const float scale = (part ? 1.0f : args.q_scale) / sqrtf(ss + args.l2_eps);
#pragma unroll
      for (int c = 0; c < CPI; ++c) y[c] *= scale;
    }
#pragma unroll
    for (int c = 0; c < CPI; ++c) dst[c] = y[c];
  }
}

// Staging, per position: a, b and (trees) the position's tree code. The tree
// code travels through LDS: reading the kernel-argument bytes inside the
// position loop would be a vector load whose wait also drains every
// outstanding checkpoint store.
template <int DK, int NTH, int RPB, int POS_FLOATS, typename TIn, bool TREE>
__device__ __forceinline__ void stage_gates(const GdnArgs& args, const Hot& hs, float* buf, const Unit& u, int t0,
                                            int tn, int p) {
  const int T = hs.n_pos;
  const TIn* ag = static_cast<const TIn*>(hs.a);
  const TIn* bg = static_cast<const TIn*>(hs.b);
  for (int e = p; e < tn; e += NTH) {
    const size_t src = (static_cast<size_t>(u.r) * T + t0 + e) * hs.n_vheads + u.h;
    buf[e * POS_FLOATS + 2 * DK + RPB] = load_elem<TIn>(ag, src);
    buf[e * POS_FLOATS + 2 * DK + RPB + 1] = load_elem<TIn>(bg, src);
    if constexpr (TREE) {
      const int gi = u.r * T + t0 + e;
      const int nT = args.geom_req * T;
      const uint32_t code = static_cast<uint8_t>(args.geom[gi]) |
                            (static_cast<uint32_t>(static_cast<uint8_t>(args.geom[nT + gi])) << 8) |
                            (static_cast<uint32_t>(static_cast<uint8_t>(args.geom[2 * nT + gi])) << 16);
      buf[e * POS_FLOATS + 2 * DK + RPB + 2] = __uint_as_float(code);
    }
  }
}

template <int DK, int NTH, int RPB, int POS_FLOATS, typename TIn, bool TREE, bool FUSED>
__device__ __forceinline__ void stage_window(const GdnArgs& args, const Hot& hs, float* buf, const Unit& u, int t0,
                                             int tn, int p) {
  if constexpr (FUSED)
    stage_fused<DK, NTH, RPB, POS_FLOATS, TIn, TREE>(args, hs, buf, u, t0, tn, p);
  else
    stage_plain<DK, NTH, RPB, POS_FLOATS, TIn>(args, hs, buf, u, t0, tn, p);
  stage_gates<DK, NTH, RPB, POS_FLOATS, TIn, TREE>(args, hs, buf, u, t0, tn, p);
}

// The unit's initial state rows: `state`, or for a zero-copy span the
// previous span's checkpoint at the request's accepted position. nullptr when
// that index is out of range (the request then writes nothing).
template <int DK>
__device__ __forceinline__ const float* initial_rows(const GdnArgs& args, const Hot& hs, const Unit& u) {
  const size_t head_elems = static_cast<size_t>(hs.d_v) * DK;
  if (hs.state == nullptr) {
    const int node = args.src_node[u.r];
    if (node < 0 || node >= args.src_npos) return nullptr;
    return args.src_ckpt + ((static_cast<size_t>(u.r) * args.src_npos + node) * hs.n_vheads + u.h) * head_elems +
           static_cast<size_t>(u.row0) * DK;
  }
  return hs.state + (static_cast<size_t>(u.r) * hs.n_vheads + u.h) * head_elems +
         static_cast<size_t>(u.row0) * DK;
}

// Checkpoint rows of one position, from every lane of a wave (4 rows, LPR
// lanes per row; lane l of a row owns float4 chunks l, l + LPR, ... and
// `dst` is its row start). Stored through a raw buffer resource over the
// wave's 4 rows with the streaming and device-scope cache bits (nt sc1), so
// the lines are written through instead of waiting dirty in the XCD's L2;
// against plain nontemporal stores: 16 requests x 48 layers 101.8-102.2 vs
// 104.1-104.4 us per launch (same GPU, three alternating runs), the
// one-request chain unchanged; the tree loop keeps plain nontemporal stores
// (4% slower this way at one request). Offsets past the resource's 4 rows
// would be dropped by the hardware.
template <int DK, int NCH>
__device__ __forceinline__ void store_ckpt_rows(float* dst, const f32x4 (&s)[NCH], int lane) {
  constexpr int LPR = kLanesPerRow;
  constexpr int RPW = 64 / LPR;
  constexpr int kNtSc1 = 2 | 16;   // cache-policy bits of the store: nt (bit 1), sc1 (bit 4)
  const int rw = lane / LPR;
  const int li = lane % LPR;
  // The wave's first row: the same address in every lane.
  const uintptr_t base = reinterpret_cast<uintptr_t>(dst - rw * DK);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base >> 32));
  float* const wave_rows = reinterpret_cast<float*>((static_cast<uintptr_t>(hi) << 32) | lo);
  // Raw buffer (stride 0) of RPW rows; the third dword's data format is 32 bits.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(wave_rows, 0, RPW * DK * 4, 0x00020000);
#pragma unroll
  for (int m = 0; m < NCH; ++m)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), rsrc, (rw * DK + 4 * (li + LPR * m)) * 4,
                                           0, kNtSc1);
}

// An address that every lane of the wave holds alike, as a wave-uniform
// value (scalar registers), so that advancing it is scalar work.
__device__ __forceinline__ uintptr_t wave_uniform(uintptr_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uintptr_t>(hi) << 32) | lo;
}

// A raw-buffer offset past every resource here: an access there is dropped.
constexpr uint32_t kDroppedOffset = 0x80000000u;

// Pointers into global memory, for stores the compiler would otherwise emit
// as flat stores (which also count against the LDS wait counter).
typedef __attribute__((address_space(1))) char* GlobalBytes;
typedef __attribute__((address_space(1))) f32x4* GlobalF32x4;
typedef __attribute__((address_space(1))) float* GlobalFloat;

// The per-position stores of a wave, through raw buffer resources whose
// base is wave-uniform and advances by a scalar add per position (the lane
// offsets are loop invariant): the checkpoint rows of one position, with the
// cache-policy bits BITS (tree loops: the streaming bit alone, nt = 2, since
// the device-scope bit of the chain loops measured 4% slower on the
// one-request tree; the fused chain loop: nt and sc1), and the rows' outputs,
// stored by the first lane of each row (the other lanes' offset lies past the
// resource, where the hardware drops the write, so no lane mask is needed;
// in the 16-request chain loop, all 16 lanes of a row storing its value
// measured 6% slower).
template <int DK, int BITS>
struct WaveStores {
  static constexpr int LPR = kLanesPerRow;
  static constexpr int RPW = 64 / LPR;
  static constexpr int NCH = DK / (4 * LPR);
  float* ckpt;          // the wave's first checkpoint row at the current position
  float* out;           // the wave's first output at the current position
  size_t ckpt_step;     // floats between positions
  int out_step;
  uint32_t ckpt_off;    // this lane's byte offset in the wave's checkpoint rows
  uint32_t out_off;     // this lane's row's byte offset in the wave's outputs (first lane of a row)

  // ckpt_row0 and out_r: this lane's row at position 0 of the unit
  // (ckpt_row0 may be null: then store_ckpt is never called).
  __device__ __forceinline__ WaveStores(float* ckpt_row0, float* out_r, int t0, size_t pos_stride, int out_stride,
                                        int lane) {
    const int rw = lane / LPR;
    const int li = lane % LPR;
    ckpt = reinterpret_cast<float*>(
        wave_uniform(reinterpret_cast<uintptr_t>(ckpt_row0) - static_cast<uintptr_t>(rw) * DK * sizeof(float) +
                     static_cast<uintptr_t>(t0) * pos_stride * sizeof(float)));
    out = reinterpret_cast<float*>(
        wave_uniform(reinterpret_cast<uintptr_t>(out_r - rw + static_cast<size_t>(t0) * out_stride)));
    ckpt_step = pos_stride;
    out_step = out_stride;
    ckpt_off = static_cast<uint32_t>((rw * DK + 4 * li) * 4);
    out_off = li == 0 ? static_cast<uint32_t>(rw * 4) : kDroppedOffset;
  }
  __device__ __forceinline__ void store_ckpt(const f32x4 (&s)[NCH]) {
    // Raw buffer (stride 0) of RPW rows; the third dword's data format is 32 bits.
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(ckpt, 0, RPW * DK * 4, 0x00020000);
#pragma unroll
    for (int m = 0; m < NCH; ++m)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), rsrc, ckpt_off + m * LPR * 16, 0, BITS);
    ckpt += ckpt_step;
  }
  __device__ __forceinline__ void store_out(float o) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(out, 0, RPW * 4, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), rsrc, out_off, 0, 0);
    out += out_step;
  }
  // The same stores from the same bases as global streaming stores with
  // per-lane addresses, and the output from the first lane of each row only,
  // under a lane mask (the buffer form sends all 64 lanes and drops 60).
  // Used by tree blocks of 32 rows (many requests), where two row-owning
  // waves share each SIMD: 146 vs 157 us per 16-request launch. With one
  // row-owning wave per SIMD (one request) the buffer form's shorter
  // instruction stream is what counts (this form measured 16% slower there).
  __device__ __forceinline__ void store_ckpt_plain(const f32x4 (&s)[NCH]) {
    GlobalBytes p = (GlobalBytes)(ckpt) + ckpt_off;
#pragma unroll
    for (int m = 0; m < NCH; ++m) __builtin_nontemporal_store(s[m], reinterpret_cast<GlobalF32x4>(p + m * LPR * 16));
    ckpt += ckpt_step;
  }
  __device__ __forceinline__ void store_out_masked(float o, int lane) {
    if (lane % LPR == 0) ((GlobalFloat)(out))[lane / LPR] = o;
    out += out_step;
  }
};

// One row of S times x (k or q), in every lane of the row: each lane's
// float4 chunks in turn, then a butterfly over the row's 16 lanes.
template <int NCH>
__device__ __forceinline__ float row_dot(const f32x4 (&s)[NCH], const f32x4 (&x)[NCH]) {
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    acc = __builtin_fmaf(s[m].x, x[m].x, acc);
    acc = __builtin_fmaf(s[m].y, x[m].y, acc);
    acc = __builtin_fmaf(s[m].z, x[m].z, acc);
    acc = __builtin_fmaf(s[m].w, x[m].w, acc);
  }
  return group_sum<kLanesPerRow>(acc);
}

// S <- a S + c k^T on this lane's columns of its row.
template <int NCH>
__device__ __forceinline__ void update_row(f32x4 (&s)[NCH], const f32x4 (&k)[NCH], float a, float c) {
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    s[m].x = __builtin_fmaf(c, k[m].x, a * s[m].x);
    s[m].y = __builtin_fmaf(c, k[m].y, a * s[m].y);
    s[m].z = __builtin_fmaf(c, k[m].z, a * s[m].z);
    s[m].w = __builtin_fmaf(c, k[m].w, a * s[m].w);
  }
}

// Positions [t0, t0 + tn) of one unit, for the consumer threads: S rows in
// VGPRs, staged inputs from LDS, checkpoint and output stores. No barrier and
// (without RELOAD) no vector-memory load. LEAN selects the shorter loop for
// 32-row chain units (the fused layer's).
template <int DK, int NW, int RPB, int POS_FLOATS, bool TREE, bool RELOAD, bool CAPTURE, bool LEAN = false>
__device__ __forceinline__ void run_positions(const float* buf, f32x4* stash, f32x4 (&s)[DK / 64], int t0, int tn,
                                              float* ckpt_row0, float* out_r, size_t pos_stride, int out_stride) {
  constexpr int LPR = kLanesPerRow;
  constexpr int NCH = DK / (4 * LPR);
  constexpr int NTHREADS = NW * 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane % LPR;
  const int row_blk = (tid >> 6) * (64 / LPR) + lane / LPR;
  if constexpr (TREE) {
    // Tree spans (single-role blocks): each position's inputs are read from
    // LDS one position ahead (4% faster on 16 requests; the chain kernel,
    // whose producer waves share the SIMDs, measured 6% slower that way),
    // into the other of two register sets: the loop is unrolled by two, so
    // no copies between the sets. With one row-owning wave per SIMD (one
    // request) this loop was bound by its instruction stream (~8 cycles per
    // instruction, ~111 instructions and 0.37 us per position); without the
    // copies and with scalar store addresses, ~85 instructions: 48-layer
    // span-only stacks 11.6 -> 10.6 us per launch. Blocks of 32 rows (many
    // requests, two row-owning waves per SIMD) keep the copies and take
    // per-lane global stores instead (see WaveStores).
    struct In {
      f32x4 k[NCH], q[NCH];
      float a, b, v;
      int code;    // stash code
    };
    WaveStores<DK, 2> st(CAPTURE ? ckpt_row0 : nullptr, out_r, t0, pos_stride, out_stride, lane);
    auto fetch = [&](int tt, In& d) {
      const float* lp = buf + tt * POS_FLOATS;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        d.k[m] = *reinterpret_cast<const f32x4*>(lp + 4 * (li + LPR * m));
        d.q[m] = *reinterpret_cast<const f32x4*>(lp + DK + 4 * (li + LPR * m));
      }
      d.a = lp[2 * DK + RPB];
      d.b = lp[2 * DK + RPB + 1];
      d.v = lp[2 * DK + row_blk];
      d.code = __builtin_amdgcn_readfirstlane(__float_as_int(lp[2 * DK + RPB + 2]));
    };
    auto step = [&](const In& c) {
      const int rs = static_cast<int8_t>((c.code >> 8) & 0xFF);
      if (rs >= 0) {
#pragma unroll
        for (int m = 0; m < NCH; ++m) s[m] = stash[(rs * NCH + m) * NTHREADS + tid];
      } else if (RELOAD && rs == kFromGlobal) {
        const int p = static_cast<int8_t>(c.code & 0xFF);
        const float* src = ckpt_row0 + static_cast<size_t>(p) * pos_stride;
#pragma unroll
        for (int m = 0; m < NCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(src + 4 * (li + LPR * m));
        // Wait here, inside the rare reload branch: otherwise the compiler
        // waits at every later use of s on every position, and since the
        // vector-memory counter retires in order, each such wait would also
        // drain all outstanding checkpoint stores.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
      const float u = row_dot<NCH>(s, c.k);
      update_row<NCH>(s, c.k, c.a, c.b * __builtin_fmaf(-c.a, u, c.v));
      if constexpr (CAPTURE) {
        if constexpr (NW == 4)
          st.store_ckpt(s);
        else
          st.store_ckpt_plain(s);
      }
      const int sv = static_cast<int8_t>((c.code >> 16) & 0xFF);
      if (sv >= 0) {
#pragma unroll
        for (int m = 0; m < NCH; ++m) stash[(sv * NCH + m) * NTHREADS + tid] = s[m];
      }
      const float o = row_dot<NCH>(s, c.q);
      if constexpr (NW == 4)
        st.store_out(o);
      else
        st.store_out_masked(o, lane);
    };
    In A, B;
    if (tn > 0) fetch(0, A);
    if constexpr (NW == 4) {
      int tt = 0;
      for (; tt + 1 < tn; tt += 2) {
        fetch(tt + 1, B);
        step(A);
        fetch(min(tt + 2, tn - 1), A);   // the last pair re-reads its own last position
        step(B);
      }
      if (tt < tn) step(A);
    } else {
      // 32-row blocks: one register set copied per position. With these
      // stores it measured 146 vs 155 us per 16-request launch against the
      // two sets (the two sets with flat stores: 147).
      for (int tt = 0; tt < tn; ++tt) {
        B = A;
        if (tt + 1 < tn) fetch(tt + 1, A);
        step(B);
      }
    }
  } else if constexpr (NW == 4) {
    // Blocks of one 16-row unit (launches too small to give every CU more
    // than one unit): each SIMD runs one row-owning wave, so the position
    // loop is a dependent chain with nothing to hide its latency. It is
    // software-pipelined: position t+1's k, a, b and v and position t's q
    // are read from LDS during position t, and o_{t-1} = S_{t-1} q_{t-1} is
    // summed beside u_t = S_{t-1} k_t (the same state; two independent
    // sums whose butterflies interleave). Every sum keeps its association
    // order, so the results are bit-identical to the loop below.
    f32x4 kk[NCH], qp[NCH];
    float at = 0.0f, bt = 0.0f, vt = 0.0f;
    auto fetch_kabv = [&](int tt, f32x4 (&kd)[NCH], float& ad, float& bd, float& vd) {
      const float* lp = buf + tt * POS_FLOATS;
#pragma unroll
      for (int m = 0; m < NCH; ++m) kd[m] = *reinterpret_cast<const f32x4*>(lp + 4 * (li + LPR * m));
      ad = lp[2 * DK + RPB];
      bd = lp[2 * DK + RPB + 1];
      vd = lp[2 * DK + row_blk];
    };
#pragma unroll
    for (int m = 0; m < NCH; ++m) qp[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (tn > 0) fetch_kabv(0, kk, at, bt, vt);
    for (int tt = 0; tt < tn; ++tt) {
      const int t = t0 + tt;
      float u = 0.0f, o = 0.0f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        u = __builtin_fmaf(s[m].x, kk[m].x, u);
        o = __builtin_fmaf(s[m].x, qp[m].x, o);
        u = __builtin_fmaf(s[m].y, kk[m].y, u);
        o = __builtin_fmaf(s[m].y, qp[m].y, o);
        u = __builtin_fmaf(s[m].z, kk[m].z, u);
        o = __builtin_fmaf(s[m].z, qp[m].z, o);
        u = __builtin_fmaf(s[m].w, kk[m].w, u);
        o = __builtin_fmaf(s[m].w, qp[m].w, o);
      }
      u = group_sum<LPR>(u);
      o = group_sum<LPR>(o);
      // Next position's inputs (the last position re-reads its own: always
      // inside the staged window) and this position's q.
      f32x4 kn[NCH], qn[NCH];
      float an, bn, vn;
      fetch_kabv(min(tt + 1, tn - 1), kn, an, bn, vn);
      const float* lp = buf + tt * POS_FLOATS;
#pragma unroll
      for (int m = 0; m < NCH; ++m) qn[m] = *reinterpret_cast<const f32x4*>(lp + DK + 4 * (li + LPR * m));
      if (tt > 0 && li == 0) out_r[static_cast<size_t>(t - 1) * out_stride] = o;
      const float c = bt * __builtin_fmaf(-at, u, vt);
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        s[m].x = __builtin_fmaf(c, kk[m].x, at * s[m].x);
        s[m].y = __builtin_fmaf(c, kk[m].y, at * s[m].y);
        s[m].z = __builtin_fmaf(c, kk[m].z, at * s[m].z);
        s[m].w = __builtin_fmaf(c, kk[m].w, at * s[m].w);
      }
      if (CAPTURE) {
        store_ckpt_rows<DK, NCH>(ckpt_row0 + static_cast<size_t>(t) * pos_stride, s, lane);
      }
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        kk[m] = kn[m];
        qp[m] = qn[m];
      }
      at = an;
      bt = bn;
      vt = vn;
    }
    if (tn > 0) {
      float o = 0.0f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        o = __builtin_fmaf(s[m].x, qp[m].x, o);
        o = __builtin_fmaf(s[m].y, qp[m].y, o);
        o = __builtin_fmaf(s[m].z, qp[m].z, o);
        o = __builtin_fmaf(s[m].w, qp[m].w, o);
      }
      o = group_sum<LPR>(o);
      if (li == 0) out_r[static_cast<size_t>(t0 + tn - 1) * out_stride] = o;
    }
  } else if constexpr (LEAN) {
    // 32-row units of the fused layer: its producer waves compute the conv,
    // SiLU and norms on the same SIMDs, so the consumers' instruction count
    // matters there. The stores take wave-uniform bases advanced by scalar
    // adds, and the checkpoint stores are kept ahead of the output's sum (the
    // compiler would sink them to the end of the iteration): 72 instead of 87
    // instructions per position, 16-request fused step 5.27-5.28 vs
    // 5.36 ms. The plain kernel measured 0.5% slower this way and keeps the
    // loop below.
    WaveStores<DK, 2 | 16> st(CAPTURE ? ckpt_row0 : nullptr, out_r, t0, pos_stride, out_stride, lane);
    for (int tt = 0; tt < tn; ++tt) {
      const float* lp = buf + tt * POS_FLOATS;
      f32x4 kk[NCH], qq[NCH];
#pragma unroll
      for (int m = 0; m < NCH; ++m) kk[m] = *reinterpret_cast<const f32x4*>(lp + 4 * (li + LPR * m));
      const float u = row_dot<NCH>(s, kk);
      const float at = lp[2 * DK + RPB];
      update_row<NCH>(s, kk, at, lp[2 * DK + RPB + 1] * __builtin_fmaf(-at, u, lp[2 * DK + row_blk]));
      if (CAPTURE) st.store_ckpt(s);
      __builtin_amdgcn_sched_barrier(0);   // the stores stay here
#pragma unroll
      for (int m = 0; m < NCH; ++m) qq[m] = *reinterpret_cast<const f32x4*>(lp + DK + 4 * (li + LPR * m));
      st.store_out(row_dot<NCH>(s, qq));
    }
  } else {
    for (int tt = 0; tt < tn; ++tt) {
      const int t = t0 + tt;
      const float* lp = buf + tt * POS_FLOATS;
      f32x4 kk[NCH];
#pragma unroll
      for (int m = 0; m < NCH; ++m) kk[m] = *reinterpret_cast<const f32x4*>(lp + 4 * (li + LPR * m));
      float u = 0.0f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        u = __builtin_fmaf(s[m].x, kk[m].x, u);
        u = __builtin_fmaf(s[m].y, kk[m].y, u);
        u = __builtin_fmaf(s[m].z, kk[m].z, u);
        u = __builtin_fmaf(s[m].w, kk[m].w, u);
      }
      u = group_sum<LPR>(u);
      const float at = lp[2 * DK + RPB];
      const float bt = lp[2 * DK + RPB + 1];
      const float vt = lp[2 * DK + row_blk];
      const float c = bt * __builtin_fmaf(-at, u, vt);
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        s[m].x = __builtin_fmaf(c, kk[m].x, at * s[m].x);
        s[m].y = __builtin_fmaf(c, kk[m].y, at * s[m].y);
        s[m].z = __builtin_fmaf(c, kk[m].z, at * s[m].z);
        s[m].w = __builtin_fmaf(c, kk[m].w, at * s[m].w);
      }
      if (CAPTURE) {
        store_ckpt_rows<DK, NCH>(ckpt_row0 + static_cast<size_t>(t) * pos_stride, s, lane);
      }
      float o = 0.0f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const f32x4 qq = *reinterpret_cast<const f32x4*>(lp + DK + 4 * (li + LPR * m));
        o = __builtin_fmaf(s[m].x, qq.x, o);
        o = __builtin_fmaf(s[m].y, qq.y, o);
        o = __builtin_fmaf(s[m].z, qq.z, o);
        o = __builtin_fmaf(s[m].w, qq.w, o);
      }
      o = group_sum<LPR>(o);
      if (li == 0) out_r[static_cast<size_t>(t) * out_stride] = o;
    }
  }
}

// Producer staging of one item (a window of positions of one unit) into buf,
// by NTH threads (p = index among them); at a unit's first window also its
// initial state rows and the valid flag, unless STATE is false (the block's
// first item, whose rows the consumers load themselves). ONE_WAIT: the
// state-row and gate loads are issued before the input loads and all are
// written afterwards, so the thread waits for memory once; otherwise each
// part waits in turn.
template <int DK, int NTH, int RPB, int POS_FLOATS, typename TIn, bool FUSED, bool ONE_WAIT, bool STATE = true>
__device__ __forceinline__ void produce_item(const GdnArgs& args, const Hot& hs, float* buf, float* state_lds,
                                             int* flag_lds, const Unit& u, int t0, int tn, int p) {
  constexpr int N4 = RPB * DK / 4;   // float4 chunks of a unit's state rows
  constexpr int SPT = (N4 + NTH - 1) / NTH;
  static_assert(kWindow <= NTH, "one gate pair per staging thread");
  const int T = hs.n_pos;
  const float* init = (STATE && t0 == 0) ? initial_rows<DK>(args, hs, u) : nullptr;
  if constexpr (ONE_WAIT) {
    const TIn* ag = static_cast<const TIn*>(hs.a);
    const TIn* bg = static_cast<const TIn*>(hs.b);
    const size_t gsrc = (static_cast<size_t>(u.r) * T + t0 + min(p, tn - 1)) * hs.n_vheads + u.h;
    const float ga = load_elem<TIn>(ag, gsrc);
    const float gb = load_elem<TIn>(bg, gsrc);
    f32x4 sv[SPT];
    if (init != nullptr) {
#pragma unroll
      for (int k = 0; k < SPT; ++k) sv[k] = reinterpret_cast<const f32x4*>(init)[min(p + k * NTH, N4 - 1)];
    }
    if constexpr (FUSED)
      stage_fused<DK, NTH, RPB, POS_FLOATS, TIn, false>(args, hs, buf, u, t0, tn, p);
    else
      stage_plain<DK, NTH, RPB, POS_FLOATS, TIn>(args, hs, buf, u, t0, tn, p);
    if (p < tn) {
      buf[p * POS_FLOATS + 2 * DK + RPB] = ga;
      buf[p * POS_FLOATS + 2 * DK + RPB + 1] = gb;
    }
    if (init != nullptr) {
#pragma unroll
      for (int k = 0; k < SPT; ++k)
        if (p + k * NTH < N4) reinterpret_cast<f32x4*>(state_lds)[p + k * NTH] = sv[k];
    }
  } else {
    if (init != nullptr) {
      f32x4 sv[SPT];
#pragma unroll
      for (int k = 0; k < SPT; ++k) sv[k] = reinterpret_cast<const f32x4*>(init)[min(p + k * NTH, N4 - 1)];
#pragma unroll
      for (int k = 0; k < SPT; ++k)
        if (p + k * NTH < N4) reinterpret_cast<f32x4*>(state_lds)[p + k * NTH] = sv[k];
    }
    stage_window<DK, NTH, RPB, POS_FLOATS, TIn, false, FUSED>(args, hs, buf, u, t0, tn, p);
  }
  if (STATE && t0 == 0 && p == 0) flag_lds[0] = init != nullptr;
}

// NW waves own the unit's rows (the consumers). NP == 0: the same waves also
// stage every window before processing it. NP > 0: NP further waves (the
// producers) stage window i+1 (and, at a unit's start, its initial state
// rows) into the other half of a double buffer while the consumers process
// window i. Every wave has its own vector-memory counter, so the producers'
// loads never wait for the consumers' checkpoint stores, and the consumers
// issue no vector-memory load at all: the store stream does not stop between
// units.
// TREE: positions follow the launch's stash schedule; RELOAD: some position
// reloads its parent's checkpoint from memory (trees with more than
// kStashSlots live branch points). FUSED: one layer in its own order; the
// staging computes q, k and v from the conv input (conv, SiLU, split, q/k L2
// norm) instead of loading them.
template <int DK, int NW, int NP, typename TIn, bool TREE, bool RELOAD, bool CAPTURE, bool FUSED, int NX>
__global__ __launch_bounds__((NW + NP + NX) * 64) void gdn_span_kernel(const void* in0, const void* in1, const void* in2,
                                                                       const void* ga, const void* gb,
                                                                       const float* init_state, uint32_t shape_a,
                                                                       uint32_t shape_b, const GdnArgs args) {
  constexpr int LPR = kLanesPerRow;
  constexpr int RPW = 64 / LPR;          // rows per wave
  constexpr int RPB = RPW * NW;          // rows per unit
  constexpr int NCH = DK / (4 * LPR);    // float4 chunks per lane
  static_assert(NCH >= 1 && DK % (4 * LPR) == 0, "lane mapping");
  static_assert(NP == 0 || (!TREE && CAPTURE), "only the capturing chain kernel has producer waves");
  static_assert(NX == 0 || NP == 0, "staging helpers belong to the single-role kernel");
  constexpr int POS_FLOATS = pos_floats(DK, RPB, TREE);
  constexpr int NC = NW * 64;            // consumer threads

  extern __shared__ float lds[];
  const Hot hs = make_hot(in0, in1, in2, ga, gb, init_state, shape_a, shape_b);
  const int T = hs.n_pos;
  const int Hv = hs.n_vheads;
  const int dv = hs.d_v;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane % LPR;
  const int row_blk = (tid >> 6) * RPW + lane / LPR;
  const size_t head_elems = static_cast<size_t>(dv) * DK;
  const size_t pos_stride = static_cast<size_t>(Hv) * head_elems;   // one position of ckpt
  const int out_stride = Hv * dv;

  // Consumer pointers of the current unit.
  auto ckpt_of = [&](const Unit& u) -> float* {
    return CAPTURE ? args.ckpt + static_cast<size_t>(u.r) * T * pos_stride + static_cast<size_t>(u.h) * head_elems +
                         static_cast<size_t>(u.row0 + row_blk) * DK
                   : nullptr;
  };
  auto out_of = [&](const Unit& u) -> float* {
    return args.out + (static_cast<size_t>(u.r) * T * Hv + u.h) * dv + u.row0 + row_blk;
  };
  f32x4 s[NCH];

  if constexpr (NP == 0) {
    // One batch of argument loads before the unit loop's first test (the
    // producer/consumer kernel below gets this from the compiler unasked);
    // otherwise the bound, the shape and the pointers arrive one dependent
    // round trip after another before the first staging load.
    // (One asm statement takes every value, so that all loads are issued
    // before the single wait.)
    asm volatile("" : : "s"(args.state), "s"(args.ckpt), "s"(args.out), "s"(args.n_units), "s"(args.n_blocks),
                 "s"(args.window), "s"(args.q_scale), "s"(args.src_ckpt), "s"(args.src_node), "s"(args.src_npos),
                 "s"(args.geom_req));
    if constexpr (FUSED) asm volatile("" : : "s"(args.conv_c), "s"(args.silu), "s"(args.l2_eps));
    f32x4* const stash = reinterpret_cast<f32x4*>(lds + staging_floats(min(T, kWindow), POS_FLOATS));
    // NX further waves only help stage each window (they own no rows).
    const bool owner = NX == 0 || tid < NC;   // wave-uniform
    for (int W = blockIdx.x; W < args.n_units; W += args.n_blocks) {
      const Unit u = unit_of(hs, W, RPB);
      const float* init = initial_rows<DK>(args, hs, u);
      if (init == nullptr) continue;   // block-uniform: every thread has the same request
      if (owner) {
        init += static_cast<size_t>(row_blk) * DK;
#pragma unroll
        for (int m = 0; m < NCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(init + 4 * (li + LPR * m));
      }
      float* const ckpt_row0 = ckpt_of(u);
      float* const out_r = out_of(u);
      for (int t0 = 0; t0 < T; t0 += kWindow) {
        const int tn = min(kWindow, T - t0);
        __syncthreads();  // LDS reads of the previous window (or unit) are done
        stage_window<DK, NC + NX * 64, RPB, POS_FLOATS, TIn, TREE, FUSED>(args, hs, lds, u, t0, tn, tid);
        __syncthreads();
        if (owner)
          run_positions<DK, NW, RPB, POS_FLOATS, TREE, RELOAD, CAPTURE, FUSED>(lds, stash, s, t0, tn, ckpt_row0, out_r,
                                                                        pos_stride, out_stride);
      }
      if (!CAPTURE && owner) {
        float* state_row = args.state + (static_cast<size_t>(u.r) * Hv + u.h) * head_elems +
                           static_cast<size_t>(u.row0 + row_blk) * DK;
#pragma unroll
        for (int m = 0; m < NCH; ++m) *reinterpret_cast<f32x4*>(state_row + 4 * (li + LPR * m)) = s[m];
      }
    }
  } else {
    constexpr int NTH = NP * 64;           // producer threads
    // The window (args.window) is min(T, kWindow); computed here from the
    // preloaded shape so that the LDS layout needs no argument load.
    const int SB = staging_floats(min(T, kWindow), POS_FLOATS);
    float* const state_lds = lds + 2 * SB;
    int* const flag_lds = reinterpret_cast<int*>(state_lds + RPB * DK);
    const bool consumer = tid < NC;        // wave-uniform
    const int p = tid - NC;                // producer index
    const int nwin = (T + kWindow - 1) / kWindow;

    // Stage item i into buffer i % 2: all threads for item 0 (no checkpoint
    // store is in flight yet), the producers for every later item. Every
    // block of a launch holds at least one unit (the grid never has more
    // blocks than units), so item 0 is staged straight from the preloaded
    // arguments, before anything waits for the rest of the argument block.
    // The consumers load the first unit's state rows straight into their
    // registers in the same round of loads (no trip through LDS, and no
    // barrier for them before the first position).
    const Unit u0 = unit_of(hs, blockIdx.x, RPB);
    bool valid0 = false;
    if (consumer) {
      const float* init0 = initial_rows<DK>(args, hs, u0);
      valid0 = init0 != nullptr;
      if (valid0) {
#pragma unroll
        for (int m = 0; m < NCH; ++m)
          s[m] = *reinterpret_cast<const f32x4*>(init0 + static_cast<size_t>(row_blk) * DK + 4 * (li + LPR * m));
      }
    }
    produce_item<DK, (NW + NP) * 64, RPB, POS_FLOATS, TIn, FUSED, true, false>(args, hs, lds, state_lds, flag_lds,
                                                                               u0, 0, min(kWindow, T), tid);
    __syncthreads();
    auto item_unit = [&](int i) { return unit_of(hs, blockIdx.x + (i / nwin) * args.n_blocks, RPB); };
    const int n_my = (args.n_units - 1 - static_cast<int>(blockIdx.x)) / args.n_blocks + 1;
    const int n_items = n_my * nwin;       // (unit, window) pairs of this block, in order
    bool valid = false;
    float* ckpt_row0 = nullptr;
    float* out_r = nullptr;
    for (int i = 0; i < n_items; ++i) {
      const int j = i % nwin;
      if (consumer && j == 0) {
        const Unit u = unit_of(hs, blockIdx.x + (i / nwin) * args.n_blocks, RPB);
        valid = i == 0 ? valid0 : flag_lds[0] != 0;
        if (valid && i > 0) {
#pragma unroll
          for (int m = 0; m < NCH; ++m)
            s[m] = *reinterpret_cast<const f32x4*>(state_lds + row_blk * DK + 4 * (li + LPR * m));
        }
        ckpt_row0 = ckpt_of(u);
        out_r = out_of(u);
      }
      // The state rows and flag are read: producers may replace them (the
      // first item's rows came from memory, so it needs no barrier here).
      if (i > 0) __syncthreads();
      if (consumer) {
        if (valid) {
          const int t0 = j * kWindow;
          run_positions<DK, NW, RPB, POS_FLOATS, false, false, CAPTURE, FUSED>(
              lds + (i & 1) * SB, nullptr, s, t0, min(kWindow, T - t0), ckpt_row0, out_r, pos_stride, out_stride);
        }
      } else if (i + 1 < n_items) {
        const int t0 = ((i + 1) % nwin) * kWindow;
        // The fused staging issues all its loads before its first wait; the
        // plain staging measured faster with its loads spread over the item.
        produce_item<DK, NTH, RPB, POS_FLOATS, TIn, FUSED, FUSED>(args, hs, lds + ((i + 1) & 1) * SB, state_lds,
                                                                 flag_lds, item_unit(i + 1), t0, min(kWindow, T - t0),
                                                                 p);
      }
      __syncthreads();  // window i + 1 is staged; buffer i % 2 is free
    }
  }
  // The status word counts out-of-range source indices. It is taken last so
  // that no branch sits between the kernel's entry and its argument loads.
  if (args.status != nullptr && args.req0 == 0 && blockIdx.x == 0 && tid == (NP > 0 ? NC : 0)) {
    int32_t bad = 0;
    for (int i = 0; i < args.n_req_total; ++i) {
      const int32_t u = args.src_node_all[i];
      bad += (u < 0 || u >= args.src_npos) ? 1 : 0;
    }
    *args.status = bad;
  }
}

// Launch through hipExtLaunchKernelGGL so that optional timing events are
// recorded by the dispatch itself (no extra stream commands between kernels).
template <int DK, int NW, int NP, typename TIn, bool TREE, bool RELOAD, bool CAPTURE, bool FUSED, int NX = 0>
hipError_t launch_one(GdnArgs& args, int grid, int n_slots, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop) {
  constexpr int RPB = (64 / kLanesPerRow) * NW;
  args.n_blocks = grid;
  const size_t lds = NP > 0 ? pipelined_bytes(DK, RPB, args.window)
                            : staging_bytes(DK, RPB, args.window, TREE) + (TREE ? n_slots * slot_bytes(DK, NW) : 0);
  const void* in0 = FUSED ? args.x : args.q;
  const void* in1 = FUSED ? args.conv_w : args.k;
  const void* in2 = FUSED ? args.conv_state : args.v;
  const float* init_state = args.src_ckpt != nullptr ? nullptr : args.state;
  const uint32_t wa = shape_word_a(args.n_pos, args.d_v, args.n_vheads);
  const uint32_t wb = static_cast<uint32_t>(args.n_kheads);
  hipExtLaunchKernelGGL((gdn_span_kernel<DK, NW, NP, TIn, TREE, RELOAD, CAPTURE, FUSED, NX>), dim3(grid),
                        dim3((NW + NP + NX) * 64), lds, stream, start, stop, 0, in0, in1, in2, args.a, args.b,
                        init_state, wa, wb, args);
  return launch_error();
}

enum class Mode { kChainNoCapture, kChain, kTree, kTreeReload };

template <int DK, int NW, typename TIn, bool FUSED>
hipError_t launch_mode(GdnArgs& args, Mode mode, int grid, int n_slots, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  // f32 conv inputs need twice the registers of bf16 ones in the fused
  // staging; that variant keeps the single-role kernel (no spills). Fused
  // blocks of one 16-row unit (one request: one item per block, staged by
  // every wave) take 2 producer waves: 6-wave blocks measured 1% faster per
  // fused one-request step than 8-wave ones (0.520 vs 0.526 ms); the plain
  // span was 2% slower with fewer.
  constexpr int NP = (FUSED && sizeof(TIn) == 4) ? 0 : ((FUSED && NW == 4) ? 2 : kProducerWaves);
  // Trees in blocks of 16-row units (each block then usually holds one
  // unit, whose window its 4 waves would stage alone) take 4 staging-only
  // waves.
  constexpr int NXT = NW == 4 ? 4 : 0;
  switch (mode) {
    case Mode::kTreeReload:
      return launch_one<DK, NW, 0, TIn, true, true, true, FUSED, NXT>(args, grid, n_slots, s, e0, e1);
    case Mode::kTree:
      return launch_one<DK, NW, 0, TIn, true, false, true, FUSED, NXT>(args, grid, n_slots, s, e0, e1);
    case Mode::kChain: return launch_one<DK, NW, NP, TIn, false, false, true, FUSED>(args, grid, 0, s, e0, e1);
    default:
      // The fused layer always captures (checked by the entry point).
      if constexpr (FUSED) return hipErrorInvalidValue;
      else return launch_one<DK, NW, 0, TIn, false, false, false, false>(args, grid, 0, s, e0, e1);
  }
}

// Launch shape: 32-row units on a one-block-per-CU grid when there are at
// least as many such units as CUs, else one 4-wave block per 16-row unit.
int waves_for(int d_v, int n_vheads, int n_req_launch, int n_cu) {
  const int units32 = (d_v % 32 == 0) ? (d_v / 32) * n_vheads * n_req_launch : 0;
  return (units32 >= n_cu && n_cu > 0) ? 8 : 4;
}

template <int DK, typename TIn, bool FUSED>
hipError_t launch_dk(GdnArgs& args, int n_req_launch, int n_cu, int waves, Mode mode, int n_slots,
                     hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (waves == 8) {
    args.n_units = (args.d_v / 32) * args.n_vheads * n_req_launch;
    return launch_mode<DK, 8, TIn, FUSED>(args, mode, n_cu, n_slots, s, e0, e1);
  }
  args.n_units = (args.d_v / 16) * args.n_vheads * n_req_launch;
  return launch_mode<DK, 4, TIn, FUSED>(args, mode, args.n_units, n_slots, s, e0, e1);
}

template <bool FUSED>
hipError_t launch_any(const hrs_gdn_desc* d, GdnArgs& args, int n, int n_cu, int waves, Mode mode, int n_slots,
                      hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (d->d_k == 128)
    return d->in_dtype == HRS_BF16 ? launch_dk<128, uint16_t, FUSED>(args, n, n_cu, waves, mode, n_slots, s, e0, e1)
                                   : launch_dk<128, float, FUSED>(args, n, n_cu, waves, mode, n_slots, s, e0, e1);
  return d->in_dtype == HRS_BF16 ? launch_dk<64, uint16_t, FUSED>(args, n, n_cu, waves, mode, n_slots, s, e0, e1)
                                 : launch_dk<64, float, FUSED>(args, n, n_cu, waves, mode, n_slots, s, e0, e1);
}

// The two device attributes a launch shape depends on, queried once per
// device and thread (every layer of a step makes one call; the attribute
// queries cost more than the rest of the host work of a call).
struct DeviceLimits {
  int n_cu;      // compute units (0: unknown, one block per 16-row unit)
  int max_lds;   // LDS bytes a block may use
};

DeviceLimits device_limits() {
  thread_local int cached_dev = -1;
  thread_local DeviceLimits cached{0, 64 * 1024};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DeviceLimits{0, 64 * 1024};
  if (dev != cached_dev) {
    DeviceLimits lim{0, 64 * 1024};
    if (hipDeviceGetAttribute(&lim.n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) lim.n_cu = 0;
    if (hipDeviceGetAttribute(&lim.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      lim.max_lds = 64 * 1024;
    cached = lim;
    cached_dev = dev;
  }
  return cached;
}

// Inputs of the fused layer: the conv input and weights replace q, k and v.
struct FusedInputs {
  const void* x;
  const void* conv_w;
  const void* conv_state;
  int32_t silu;
  float l2_eps;
};

}  // namespace
}  // namespace hrs

using namespace hrs;

static int gdn_span_impl(const hrs_gdn_desc* d, const void* q, const void* k, const void* v, const void* a,
                         const void* b, float* state, float* ckpt, float* out, void* stream, void* start_event,
                         void* stop_event, const hrs_span_source* src = nullptr, int32_t* status = nullptr,
                         const FusedInputs* fused = nullptr) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_req < 1 || d->n_kheads < 1 || d->n_vheads < 1 || d->d_k < 1 || d->d_v < 1) return HRS_EINVAL;
  if (d->n_vheads % d->n_kheads != 0) return HRS_EINVAL;
  if (!dtype_ok(d->in_dtype)) return HRS_EINVAL;
  if (d->topo != HRS_CHAIN && d->topo != HRS_TREE) return HRS_EINVAL;
  if (fused != nullptr) {
    if (!fused->x || !fused->conv_w || !fused->conv_state || ckpt == nullptr) return HRS_EINVAL;
    if (!(fused->l2_eps >= 0.0f)) return HRS_EINVAL;
  } else if (!q || !k || !v) {
    return HRS_EINVAL;
  }
  if (!a || !b || !out) return HRS_EINVAL;
  if (src == nullptr && !state) return HRS_EINVAL;
  if (src != nullptr) {
    if (!src->ckpt || !src->node || ckpt == nullptr) return HRS_EINVAL;
    if (src->n_pos < 1 || src->n_pos > HRS_MAX_POS) return HRS_EINVAL;
    // The new checkpoints must not overwrite the ones the span starts from.
    const size_t elems = static_cast<size_t>(d->n_vheads) * d->d_v * d->d_k * sizeof(float) * d->n_req;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(ckpt), a1 = a0 + elems * d->n_pos;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(src->ckpt), b1 = b0 + elems * src->n_pos;
    if (a0 < b1 && b0 < a1) return HRS_EINVAL;
    if (!aligned16(src->ckpt) || !aligned16(src->node) || (status && !aligned16(status))) return HRS_EALIGN;
  }
  if (d->topo == HRS_TREE && ckpt == nullptr) return HRS_EINVAL;
  if (static_cast<int64_t>(d->d_v) * d->n_vheads > (1 << 20) || d->n_req > (1 << 20)) return HRS_EINVAL;
  const int geo = check_topology(d->topo, d->parent, d->n_req, d->n_pos);
  if (geo != HRS_OK) return geo;
  if ((fused == nullptr && (!aligned16(q) || !aligned16(k) || !aligned16(v))) || !aligned16(a) || !aligned16(b) ||
      (state && !aligned16(state)) || !aligned16(out) || (ckpt && !aligned16(ckpt)))
    return HRS_EALIGN;
  if (fused != nullptr &&
      (!aligned16(fused->x) || !aligned16(fused->conv_w) || !aligned16(fused->conv_state)))
    return HRS_EALIGN;
  if (d->d_k != 64 && d->d_k != 128) return HRS_EUNSUPPORTED;
  if (d->d_v % 16 != 0 || d->d_v > 256) return HRS_EUNSUPPORTED;

  GdnArgs args;
  args.q = q; args.k = k; args.v = v; args.a = a; args.b = b;
  args.state = state; args.ckpt = ckpt; args.out = out;
  args.n_pos = d->n_pos; args.n_kheads = d->n_kheads; args.n_vheads = d->n_vheads;
  args.d_v = d->d_v; args.group = d->n_vheads / d->n_kheads; args.q_scale = d->q_scale;
  args.src_ckpt = src ? src->ckpt : nullptr;
  args.src_node = src ? src->node : nullptr;
  args.src_npos = src ? src->n_pos : 0;
  args.n_req_total = d->n_req;
  args.src_node_all = args.src_node;
  args.status = src ? status : nullptr;
  args.x = fused ? fused->x : nullptr;
  args.conv_w = fused ? fused->conv_w : nullptr;
  args.conv_state = fused ? fused->conv_state : nullptr;
  args.conv_c = 2 * d->n_kheads * d->d_k + d->n_vheads * d->d_v;
  args.silu = fused ? fused->silu : 0;
  args.l2_eps = fused ? fused->l2_eps : 0.0f;
  args.geom_req = 0;

  const bool tree = d->topo == HRS_TREE;
  const bool capture = ckpt != nullptr;
  // Tree geometry bytes per (request, position): parent, restore, save, and
  // for the fused layer three conv window sources.
  const int geom_per_pos = fused ? 6 : 3;
  const int per_launch = tree ? std::max(1, (kGeomBytes / geom_per_pos) / d->n_pos) : 4096;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const DeviceLimits lim = device_limits();
  const int n_cu = lim.n_cu, max_lds = lim.max_lds;
  args.window = std::min(kWindow, static_cast<int>(d->n_pos));
  // Per-request strides of every per-request buffer; each launch gets its
  // pointers offset to its first request.
  const size_t es = dtype_size(d->in_dtype);
  const size_t T_ = static_cast<size_t>(d->n_pos);
  const size_t head = static_cast<size_t>(d->d_v) * d->d_k;
  const size_t st_q = T_ * d->n_kheads * d->d_k * es, st_v = T_ * d->n_vheads * d->d_v * es;
  const size_t st_g = T_ * d->n_vheads * es, st_state = static_cast<size_t>(d->n_vheads) * head;
  const size_t st_x = T_ * static_cast<size_t>(args.conv_c) * es, st_cs = 3 * static_cast<size_t>(args.conv_c) * es;
  const GdnArgs base = {q, k, v, a, b, state, ckpt, out};
  const void* base_x = args.x;
  const void* base_cs = args.conv_state;
  const float* base_src = args.src_ckpt;
  const int32_t* base_node = args.src_node;
  auto at = [](const void* p, size_t bytes) -> const void* {
    return p == nullptr ? nullptr : static_cast<const char*>(p) + bytes;
  };
  auto atf = [](float* p, size_t elems) -> float* { return p == nullptr ? nullptr : p + elems; };
  for (int r0 = 0; r0 < d->n_req; r0 += per_launch) {
    const int n = std::min(per_launch, d->n_req - r0);
    const size_t r = static_cast<size_t>(r0);
    args.req0 = r0;
    args.q = at(base.q, r * st_q);
    args.k = at(base.k, r * st_q);
    args.v = at(base.v, r * st_v);
    args.a = at(base.a, r * st_g);
    args.b = at(base.b, r * st_g);
    args.state = atf(base.state, r * st_state);
    args.ckpt = atf(base.ckpt, r * T_ * st_state);
    args.out = atf(base.out, r * T_ * d->n_vheads * d->d_v);
    args.x = at(base_x, r * st_x);
    args.conv_state = at(base_cs, r * st_cs);
    args.src_ckpt = base_src == nullptr ? nullptr : base_src + r * static_cast<size_t>(args.src_npos) * st_state;
    args.src_node = base_node == nullptr ? nullptr : base_node + r;
    // The first launch records the start event, the last one the stop event.
    hipEvent_t e0 = r0 == 0 ? static_cast<hipEvent_t>(start_event) : nullptr;
    hipEvent_t e1 = r0 + n >= d->n_req ? static_cast<hipEvent_t>(stop_event) : nullptr;
    Mode mode = capture ? Mode::kChain : Mode::kChainNoCapture;
    const int waves = waves_for(d->d_v, d->n_vheads, n, n_cu);
    int n_slots = 0;
    if (tree) {
      const int T_ = d->n_pos;
      const int nT = n * T_;
      int8_t* g_parent = args.geom;
      int8_t* g_restore = args.geom + nT;
      int8_t* g_save = args.geom + 2 * nT;
      int8_t* g_window = args.geom + 3 * nT;
      args.geom_req = n;
      // Stash slots that fit in LDS beside the staging buffer.
      const size_t stage = staging_bytes(d->d_k, 4 * waves, args.window, true);
      const size_t per_slot = slot_bytes(d->d_k, waves);
      const size_t room = static_cast<size_t>(max_lds) > stage ? static_cast<size_t>(max_lds) - stage : 0;
      const int fit = static_cast<int>(std::min<size_t>(kStashSlots, room / per_slot));
      for (int i = 0; i < nT; ++i) g_parent[i] = static_cast<int8_t>(d->parent[static_cast<size_t>(r0) * T_ + i]);
      for (int j = 0; j < n; ++j) {
        const int32_t* par = d->parent + static_cast<size_t>(r0 + j) * T_;
        gdn_tree_schedule(par, T_, fit, g_restore + j * T_, g_save + j * T_);
        if (fused) conv_window_sources(par, T_, 4, g_window + j * T_ * 3);
      }
      mode = Mode::kTree;
      for (int i = 0; i < nT; ++i) {
        if (g_restore[i] == kFromGlobal) mode = Mode::kTreeReload;
        if (g_save[i] >= n_slots) n_slots = g_save[i] + 1;
      }
    }
    const hipError_t e = fused ? launch_any<true>(d, args, n, n_cu, waves, mode, n_slots, s, e0, e1)
                               : launch_any<false>(d, args, n, n_cu, waves, mode, n_slots, s, e0, e1);
    if (e != hipSuccess) return HRS_EDEVICE;
  }
  return HRS_OK;
}

extern "C" int gdn_verify_span(const hrs_gdn_desc* d, const void* q, const void* k, const void* v,
                               const void* a, const void* b, float* state, float* ckpt, float* out,
                               void* stream) {
  return gdn_span_impl(d, q, k, v, a, b, state, ckpt, out, stream, nullptr, nullptr);
}

extern "C" int gdn_verify_span_from(const hrs_gdn_desc* d, const hrs_span_source* src, const void* q, const void* k,
                                    const void* v, const void* a, const void* b, float* ckpt, float* out,
                                    int32_t* status, void* stream) {
  if (src == nullptr) return HRS_EINVAL;
  return gdn_span_impl(d, q, k, v, a, b, nullptr, ckpt, out, stream, nullptr, nullptr, src, status);
}

extern "C" int gdn_verify_span_timed(const hrs_gdn_desc* d, const void* q, const void* k, const void* v,
                                     const void* a, const void* b, float* state, float* ckpt, float* out,
                                     void* stream, void* start_event, void* stop_event) {
  return gdn_span_impl(d, q, k, v, a, b, state, ckpt, out, stream, start_event, stop_event);
}

extern "C" int gdn_layer_verify_span(const hrs_gdn_layer_desc* d, const void* x, const void* conv_w,
                                     const void* conv_state, const void* a, const void* b, const float* state,
                                     const hrs_span_source* src, float* ckpt, float* out, int32_t* status,
                                     void* stream) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->conv_width != 4) return HRS_EUNSUPPORTED;
  if ((state == nullptr) == (src == nullptr)) return HRS_EINVAL;   // exactly one initial state
  if (ckpt == nullptr) return HRS_EINVAL;
  FusedInputs f{x, conv_w, conv_state, d->silu != 0 ? 1 : 0, d->l2_eps};
  return gdn_span_impl(&d->gdn, nullptr, nullptr, nullptr, a, b, const_cast<float*>(state), ckpt, out, stream,
                       nullptr, nullptr, src, status, &f);
}

extern "C" const char* hrs_last_hip_error_string(void) {
  return hipGetErrorString(static_cast<hipError_t>(hrs_last_hip_error()));
}
