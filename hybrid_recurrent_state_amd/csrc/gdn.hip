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
//    lines. Checkpoints are written with nontemporal stores; they are not
//    read again until rollback (normal stores measured ~12% slower).
//  * Work order: units are numbered row block fastest, then head, then
//    request, and a block walks units W, W + gridDim.x, ... When there are at
//    least as many 32-row units as compute units, the grid is one 8-wave block
//    per CU: all CUs then advance through the positions together and each
//    position's checkpoint region (2 MiB per request) is written as one
//    contiguous sweep. Measured on the 16-request Qwen shape: 6.0 TB/s versus
//    5.1 TB/s for one block per unit, and 75% of HBM peak, at the plain
//    store-stream ceiling. Smaller problems use one 4-wave block per 16-row
//    unit to spread over more CUs.
//  * The two row dot products (S k and S q) are butterfly sums over the 16
//    lanes with DPP moves; the association order is fixed, so the arithmetic
//    of a position never depends on span length, topology or launch shape.
//  * k, q (times q_scale), v rows, a and b of a window of positions are
//    staged once per unit into LDS as f32.
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

constexpr size_t staging_bytes(int dk, int rows, int window, bool tree) {
  return static_cast<size_t>(window) * pos_floats(dk, rows, tree) * sizeof(float);
}

// LDS bytes of one tree stash slot: every lane's dk / 16 floats of its row.
constexpr size_t slot_bytes(int dk, int waves) { return static_cast<size_t>(waves) * 64 * (dk / 16) * sizeof(float); }

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
  int32_t window;  // positions staged in LDS at a time (min(n_pos, kWindow))
  float q_scale;
  // Zero-copy source of the initial state (gdn_verify_span_from): when
  // src_ckpt is set, request r starts from src_ckpt[r][src_node[r]].
  const float* src_ckpt;
  const int32_t* src_node;
  int32_t src_npos;
  int32_t n_req_total;
  int32_t* status;  // optional: number of requests whose src_node is out of range
  // Tree mode, each [requests of this launch][n_pos]: parent index, restore
  // code and save slot (gdn_tree_schedule).
  int8_t parent[kGeomBytes / 3];
  int8_t restore[kGeomBytes / 3];
  int8_t save[kGeomBytes / 3];
};

// TREE: positions follow the launch's stash schedule; RELOAD: some position
// reloads its parent's checkpoint from memory (trees with more than
// kStashSlots live branch points). Without RELOAD the position loop holds no
// vector-memory load at all, so the compiler never has to wait on the
// in-order vector-memory counter (which the checkpoint stores also occupy).
template <int DK, int NW, typename TIn, bool TREE, bool RELOAD, bool CAPTURE>
__global__ __launch_bounds__(NW * 64) void gdn_span_kernel(const GdnArgs args) {
  constexpr int LPR = kLanesPerRow;
  constexpr int RPW = 64 / LPR;          // rows per wave
  constexpr int RPB = RPW * NW;          // rows per unit
  constexpr int NCH = DK / (4 * LPR);    // float4 chunks per lane
  static_assert(NCH >= 1 && DK % (4 * LPR) == 0, "lane mapping");
  constexpr int POS_FLOATS = pos_floats(DK, RPB, TREE);

  extern __shared__ float lds[];
  // Tree stash: [slot][chunk][thread] float4, after the staged positions.
  f32x4* const stash = reinterpret_cast<f32x4*>(lds + args.window * POS_FLOATS);
  constexpr int NTHREADS = NW * 64;

  const int T = args.n_pos;
  const int Hv = args.n_vheads;
  const int Hk = args.n_kheads;
  const int dv = args.d_v;
  const int nrb = dv / RPB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane % LPR;
  const int row_blk = wave * RPW + lane / LPR;
  const size_t head_elems = static_cast<size_t>(dv) * DK;
  const size_t pos_stride = static_cast<size_t>(Hv) * head_elems;   // one position of ckpt
  const TIn* qg = static_cast<const TIn*>(args.q);
  const TIn* kg = static_cast<const TIn*>(args.k);
  const TIn* vg = static_cast<const TIn*>(args.v);
  const TIn* ag = static_cast<const TIn*>(args.a);
  const TIn* bg = static_cast<const TIn*>(args.b);

  if (args.status != nullptr && args.req0 == 0 && blockIdx.x == 0 && threadIdx.x == 0) {
    int32_t bad = 0;
    for (int i = 0; i < args.n_req_total; ++i) {
      const int32_t u = args.src_node[i];
      bad += (u < 0 || u >= args.src_npos) ? 1 : 0;
    }
    *args.status = bad;
  }
  for (int W = blockIdx.x; W < args.n_units; W += gridDim.x) {
    const int rb = W % nrb;
    const int h = (W / nrb) % Hv;
    const int rl = W / (nrb * Hv);           // request within the launch
    const int r = args.req0 + rl;
    const int g = h / args.group;
    const int row0 = rb * RPB;
    const int row = row0 + row_blk;

    float* state_row =
        args.state ? args.state + (static_cast<size_t>(r) * Hv + h) * head_elems + static_cast<size_t>(row) * DK
                   : nullptr;
    const float* init_row = state_row;
    if (args.src_ckpt != nullptr) {
      // Zero-copy rollback: start from the previous span's checkpoint of its
      // accepted position. A request with an index outside the previous span
      // writes nothing (reported through the status word).
      const int node = args.src_node[r];
      if (node < 0 || node >= args.src_npos) continue;
      init_row = args.src_ckpt + ((static_cast<size_t>(r) * args.src_npos + node) * Hv + h) * head_elems +
                 static_cast<size_t>(row) * DK;
    }
    float* ckpt_row0 = nullptr;
    if (CAPTURE)
      ckpt_row0 = args.ckpt + static_cast<size_t>(r) * T * pos_stride + static_cast<size_t>(h) * head_elems +
                  static_cast<size_t>(row) * DK;
    float* out_r = args.out + (static_cast<size_t>(r) * T * Hv + h) * dv + row;

    // This lane's columns: chunk m covers [4 (li + LPR m), +4).
    f32x4 s[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(init_row + 4 * (li + LPR * m));

    for (int t0 = 0; t0 < T; t0 += kWindow) {
      const int tn = min(kWindow, T - t0);
      __syncthreads();  // LDS reads of the previous window (or unit) are done
      // Stage k and q (scaled) of key head g, 8 elements per thread-step.
      {
        constexpr int V8 = DK / 8;
        for (int e = tid; e < tn * V8; e += NW * 64) {
          const int tt = e / V8;
          const int j = (e % V8) * 8;
          const size_t src = ((static_cast<size_t>(r) * T + t0 + tt) * Hk + g) * DK + j;
          float kv[8], qv[8];
          load8<TIn>(kg + src, kv);
          load8<TIn>(qg + src, qv);
          float* lk = lds + tt * POS_FLOATS + j;
          float* lq = lk + DK;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            lk[i] = kv[i];
            lq[i] = qv[i] * args.q_scale;
          }
        }
        for (int e = tid; e < tn * RPB; e += NW * 64) {
          const int tt = e / RPB;
          const int i = e % RPB;
          const size_t src = ((static_cast<size_t>(r) * T + t0 + tt) * Hv + h) * dv + row0 + i;
          lds[tt * POS_FLOATS + 2 * DK + i] = load_elem<TIn>(vg, src);
        }
        for (int e = tid; e < tn; e += NW * 64) {
          const size_t src = (static_cast<size_t>(r) * T + t0 + e) * Hv + h;
          lds[e * POS_FLOATS + 2 * DK + RPB] = load_elem<TIn>(ag, src);
          lds[e * POS_FLOATS + 2 * DK + RPB + 1] = load_elem<TIn>(bg, src);
          if constexpr (TREE) {
            // The tree code travels through LDS: reading the kernel-argument
            // bytes inside the position loop would be a vector load whose wait
            // also drains every outstanding checkpoint store.
            const int gi = rl * T + t0 + e;
            const uint32_t code = static_cast<uint8_t>(args.parent[gi]) |
                                  (static_cast<uint32_t>(static_cast<uint8_t>(args.restore[gi])) << 8) |
                                  (static_cast<uint32_t>(static_cast<uint8_t>(args.save[gi])) << 16);
            lds[e * POS_FLOATS + 2 * DK + RPB + 2] = __uint_as_float(code);
          }
        }
      }
      __syncthreads();

      for (int tt = 0; tt < tn; ++tt) {
        const int t = t0 + tt;
        const float* lp = lds + tt * POS_FLOATS;
        int tree_code = 0;
        if constexpr (TREE) {
          tree_code = __builtin_amdgcn_readfirstlane(__float_as_int(lp[2 * DK + RPB + 2]));
          const int rs = static_cast<int8_t>((tree_code >> 8) & 0xFF);
          if (rs >= 0) {
#pragma unroll
            for (int m = 0; m < NCH; ++m) s[m] = stash[(rs * NCH + m) * NTHREADS + tid];
          } else if (RELOAD && rs == kFromGlobal) {
            const int p = static_cast<int8_t>(tree_code & 0xFF);
            const float* src = ckpt_row0 + static_cast<size_t>(p) * pos_stride;
#pragma unroll
            for (int m = 0; m < NCH; ++m) s[m] = *reinterpret_cast<const f32x4*>(src + 4 * (li + LPR * m));
            // Wait here, inside the rare reload branch: otherwise the compiler
            // waits at every later use of s on every position, and since the
            // vector-memory counter retires in order, each such wait would also
            // drain all outstanding checkpoint stores.
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
          }
        }
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
          float* dst = ckpt_row0 + static_cast<size_t>(t) * pos_stride;
#pragma unroll
          for (int m = 0; m < NCH; ++m)
            __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(dst + 4 * (li + LPR * m)));
        }
        if constexpr (TREE) {
          const int sv = static_cast<int8_t>((tree_code >> 16) & 0xFF);
          if (sv >= 0) {
#pragma unroll
            for (int m = 0; m < NCH; ++m) stash[(sv * NCH + m) * NTHREADS + tid] = s[m];
          }
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
        if (li == 0) out_r[static_cast<size_t>(t) * Hv * dv] = o;
      }
    }
    if (!CAPTURE) {
#pragma unroll
      for (int m = 0; m < NCH; ++m) *reinterpret_cast<f32x4*>(state_row + 4 * (li + LPR * m)) = s[m];
    }
  }
}

// Launch through hipExtLaunchKernelGGL so that optional timing events are
// recorded by the dispatch itself (no extra stream commands between kernels).
template <int DK, int NW, typename TIn, bool TREE, bool RELOAD, bool CAPTURE>
hipError_t launch_one(GdnArgs& args, int grid, int n_slots, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop) {
  constexpr int RPB = (64 / kLanesPerRow) * NW;
  const size_t lds = staging_bytes(DK, RPB, args.window, TREE) + (TREE ? n_slots * slot_bytes(DK, NW) : 0);
  hipExtLaunchKernelGGL((gdn_span_kernel<DK, NW, TIn, TREE, RELOAD, CAPTURE>), dim3(grid), dim3(NW * 64), lds,
                        stream, start, stop, 0, args);
  return launch_error();
}

enum class Mode { kChainNoCapture, kChain, kTree, kTreeReload };

template <int DK, int NW, typename TIn>
hipError_t launch_mode(GdnArgs& args, Mode mode, int grid, int n_slots, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  switch (mode) {
    case Mode::kTreeReload: return launch_one<DK, NW, TIn, true, true, true>(args, grid, n_slots, s, e0, e1);
    case Mode::kTree: return launch_one<DK, NW, TIn, true, false, true>(args, grid, n_slots, s, e0, e1);
    case Mode::kChain: return launch_one<DK, NW, TIn, false, false, true>(args, grid, 0, s, e0, e1);
    default: return launch_one<DK, NW, TIn, false, false, false>(args, grid, 0, s, e0, e1);
  }
}

// Launch shape: 32-row units on a one-block-per-CU grid when there are at
// least as many such units as CUs, else one 4-wave block per 16-row unit.
// Launch shape: 32-row units on a one-block-per-CU grid when there are at
// least as many such units as CUs, else one 4-wave block per 16-row unit.
int waves_for(int d_v, int n_vheads, int n_req_launch, int n_cu) {
  const int units32 = (d_v % 32 == 0) ? (d_v / 32) * n_vheads * n_req_launch : 0;
  return (units32 >= n_cu && n_cu > 0) ? 8 : 4;
}

template <int DK, typename TIn>
hipError_t launch_dk(GdnArgs& args, int n_req_launch, int n_cu, int waves, Mode mode, int n_slots,
                     hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (waves == 8) {
    args.n_units = (args.d_v / 32) * args.n_vheads * n_req_launch;
    return launch_mode<DK, 8, TIn>(args, mode, n_cu, n_slots, s, e0, e1);
  }
  args.n_units = (args.d_v / 16) * args.n_vheads * n_req_launch;
  return launch_mode<DK, 4, TIn>(args, mode, args.n_units, n_slots, s, e0, e1);
}

}  // namespace
}  // namespace hrs

using namespace hrs;

static int gdn_span_impl(const hrs_gdn_desc* d, const void* q, const void* k, const void* v, const void* a,
                         const void* b, float* state, float* ckpt, float* out, void* stream, void* start_event,
                         void* stop_event, const hrs_span_source* src = nullptr, int32_t* status = nullptr) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_req < 1 || d->n_kheads < 1 || d->n_vheads < 1 || d->d_k < 1 || d->d_v < 1) return HRS_EINVAL;
  if (d->n_vheads % d->n_kheads != 0) return HRS_EINVAL;
  if (!dtype_ok(d->in_dtype)) return HRS_EINVAL;
  if (d->topo != HRS_CHAIN && d->topo != HRS_TREE) return HRS_EINVAL;
  if (!q || !k || !v || !a || !b || !out) return HRS_EINVAL;
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
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) ||
      (state && !aligned16(state)) || !aligned16(out) || (ckpt && !aligned16(ckpt)))
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
  args.status = src ? status : nullptr;

  const bool tree = d->topo == HRS_TREE;
  const bool capture = ckpt != nullptr;
  const int per_launch = tree ? std::max(1, (kGeomBytes / 3) / d->n_pos) : 4096;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int dev = 0, n_cu = 0, max_lds = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 0;  // falls back to one block per 16-row unit
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    max_lds = 64 * 1024;
  args.window = std::min(kWindow, static_cast<int>(d->n_pos));
  for (int r0 = 0; r0 < d->n_req; r0 += per_launch) {
    const int n = std::min(per_launch, d->n_req - r0);
    args.req0 = r0;
    // The first launch records the start event, the last one the stop event.
    hipEvent_t e0 = r0 == 0 ? static_cast<hipEvent_t>(start_event) : nullptr;
    hipEvent_t e1 = r0 + n >= d->n_req ? static_cast<hipEvent_t>(stop_event) : nullptr;
    Mode mode = capture ? Mode::kChain : Mode::kChainNoCapture;
    const int waves = waves_for(d->d_v, d->n_vheads, n, n_cu);
    int n_slots = 0;
    if (tree) {
      const int T_ = d->n_pos;
      // Stash slots that fit in LDS beside the staging buffer.
      const size_t stage = staging_bytes(d->d_k, 4 * waves, args.window, true);
      const size_t per_slot = slot_bytes(d->d_k, waves);
      const size_t room = static_cast<size_t>(max_lds) > stage ? static_cast<size_t>(max_lds) - stage : 0;
      const int fit = static_cast<int>(std::min<size_t>(kStashSlots, room / per_slot));
      for (int i = 0; i < n * T_; ++i)
        args.parent[i] = static_cast<int8_t>(d->parent[static_cast<size_t>(r0) * T_ + i]);
      for (int j = 0; j < n; ++j)
        gdn_tree_schedule(d->parent + static_cast<size_t>(r0 + j) * T_, T_, fit, args.restore + j * T_,
                          args.save + j * T_);
      mode = Mode::kTree;
      for (int i = 0; i < n * T_; ++i) {
        if (args.restore[i] == kFromGlobal) mode = Mode::kTreeReload;
        if (args.save[i] >= n_slots) n_slots = args.save[i] + 1;
      }
    }
    hipError_t e;
    if (d->d_k == 128)
      e = d->in_dtype == HRS_BF16 ? launch_dk<128, uint16_t>(args, n, n_cu, waves, mode, n_slots, s, e0, e1)
                                  : launch_dk<128, float>(args, n, n_cu, waves, mode, n_slots, s, e0, e1);
    else
      e = d->in_dtype == HRS_BF16 ? launch_dk<64, uint16_t>(args, n, n_cu, waves, mode, n_slots, s, e0, e1)
                                  : launch_dk<64, float>(args, n, n_cu, waves, mode, n_slots, s, e0, e1);
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

extern "C" const char* hrs_last_hip_error_string(void) {
  return hipGetErrorString(static_cast<hipError_t>(hrs_last_hip_error()));
}
