// conv1d_verify_span: causal depthwise conv over the verify span with the
// conv state (last W-1 inputs) captured after every position.
//
// The hybrid layer's state is the recurrent state plus a short conv state
// (openinfer PR #626, "feat(qwen35): add opt-in DFlash speculative
// decoding", What Changed); restoring it after rollback is on-device
// (lucebox PR #533, "feat: DFlash support for tensor-parallel Qwen3.6
// targets", Changes).
//
// MI355X design: in capture mode for a chain, one thread takes 8 channels of
// two consecutive positions and slides the window over five loaded rows
// (measured 8.5 us versus 10.4 us for one position per thread on 16
// requests x 8192 channels). Every thread loads once and then stores, so a
// launch is one load phase and one store phase; a variant in which each
// thread walked several rows with the next row's loads issued before the
// current row's stores was not faster at these sizes (27.6 MB per launch on
// 16 requests, where the launch's fixed latency is a large part of the
// time). Captured states are written with nontemporal stores (not read
// again by this span); 128-thread blocks measured faster than 256. For a tree every (position, 8-channel group) is
// an independent thread: the host turns the parent array into a table that
// names, for each position and window slot, the x row or conv-state row to
// read (x rows are re-read from L2 by up to W threads). Loads and stores
// are 16 bytes per lane, coalesced along channels. Captured states are raw
// copies of input bits, so they are exact in any dtype. Without capture
// (decode, chain only) one thread walks its channels through the positions
// in order and writes the advanced state at the end, so no thread reads a
// state row another thread has already overwritten.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.h"
#include "internal.h"

namespace hrs {
namespace {

constexpr int kThreads = 128;
constexpr int kWidth = 4;
constexpr int kBack = kWidth - 1;

struct ConvArgs {
  const void* x;
  const void* w;
  void* conv_state;
  void* conv_ckpt;
  float* y;
  int32_t n_pos;
  int32_t channels;
  int32_t req0;
  int32_t per_request_table;  // 0: one table shared by all requests (chain)
  int32_t silu;
  int8_t src[kGeomBytes];     // [requests of this launch or 1][n_pos][W-1]
};

// Eight consecutive elements of a row, kept as raw bits and as f32.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<u32x4*>(p) = v; }
  __device__ __forceinline__ void store_nt(uint16_t* p) const {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  }
  __device__ __forceinline__ float f(int i) const {
    const uint32_t w = v[i >> 1];
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <> struct Raw8<float> {
  f32x4 v0, v1;
  __device__ __forceinline__ void load(const float* p) {
    v0 = *reinterpret_cast<const f32x4*>(p);
    v1 = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<f32x4*>(p) = v0;
    *reinterpret_cast<f32x4*>(p + 4) = v1;
  }
  __device__ __forceinline__ void store_nt(float* p) const {
    __builtin_nontemporal_store(v0, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(v1, reinterpret_cast<f32x4*>(p + 4));
  }
  __device__ __forceinline__ float f(int i) const { return i < 4 ? v0[i] : v1[i - 4]; }
};

// Weights of 8 channels: w[c][m], c in [c0, c0+8), m in [0, W).
template <typename T>
__device__ __forceinline__ void load_weights(const T* w, int c0, float (&wt)[8][kWidth]) {
  float buf[8 * kWidth];
#pragma unroll
  for (int i = 0; i < kWidth; ++i) load8<T>(w + static_cast<size_t>(c0) * kWidth + 8 * i, buf + 8 * i);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int m = 0; m < kWidth; ++m) wt[c][m] = buf[c * kWidth + m];
}

template <typename T>
__device__ __forceinline__ void conv_out(const float (&wt)[8][kWidth], const Raw8<T> (&win)[kWidth], int silu_on,
                                         float* y) {
  float o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float acc = wt[c][0] * win[0].f(c);
#pragma unroll
    for (int m = 1; m < kWidth; ++m) acc = __builtin_fmaf(wt[c][m], win[m].f(c), acc);
    o[c] = acc;
  }
  if (silu_on) {   // one uniform branch for the 8 channels
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = silu_fast(o[c]);
  }
  *reinterpret_cast<f32x4*>(y) = f32x4{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<f32x4*>(y + 4) = f32x4{o[4], o[5], o[6], o[7]};
}

// Capture mode: one thread per (position, 8-channel group).
template <typename T, bool STORE>
__global__ __launch_bounds__(kThreads) void conv_capture_kernel(const ConvArgs args) {
  args_in_registers(args.x, args.w, args.conv_state, args.conv_ckpt, args.y, args.n_pos, args.channels,
                    args.req0, args.per_request_table, args.silu);
  const int C = args.channels;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (c0 >= C) return;
  const int T_ = args.n_pos;
  const int t = blockIdx.y;
  const int rl = blockIdx.z;
  const int r = args.req0 + rl;
  const T* x = static_cast<const T*>(args.x);
  const T* cs = static_cast<const T*>(args.conv_state);
  T* ck = static_cast<T*>(args.conv_ckpt);
  const int8_t* src = args.src + (args.per_request_table ? rl * T_ * kBack : 0) + t * kBack;

  Raw8<T> win[kWidth];
#pragma unroll
  for (int m = 0; m < kBack; ++m) {
    const int s = src[m];
    if (s >= 0)
      win[m].load(x + (static_cast<size_t>(r) * T_ + s) * C + c0);
    else
      win[m].load(cs + (static_cast<size_t>(r) * kBack + (-1 - s)) * C + c0);
  }
  win[kBack].load(x + (static_cast<size_t>(r) * T_ + t) * C + c0);
  float wt[8][kWidth];
  load_weights<T>(static_cast<const T*>(args.w), c0, wt);

  conv_out<T>(wt, win, args.silu, args.y + (static_cast<size_t>(r) * T_ + t) * C + c0);
  if (STORE) {
    T* dst = ck + (static_cast<size_t>(r) * T_ + t) * kBack * C + c0;
#pragma unroll
    for (int m = 0; m < kBack; ++m) win[m + 1].store_nt(dst + static_cast<size_t>(m) * C);
  }
}

// Capture mode, chain: one thread per (kChainPos consecutive positions,
// 8-channel group); the window slides over kChainPos + W - 1 loaded rows.
constexpr int kChainPos = 2;
template <typename T, bool STORE>
__global__ __launch_bounds__(kThreads) void conv_chain_kernel(const ConvArgs args) {
  args_in_registers(args.x, args.w, args.conv_state, args.conv_ckpt, args.y, args.n_pos, args.channels,
                    args.req0, args.per_request_table, args.silu);
  const int C = args.channels;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (c0 >= C) return;
  const int T_ = args.n_pos;
  const int t0 = blockIdx.y * kChainPos;
  const int tn = min(kChainPos, T_ - t0);
  const int r = args.req0 + blockIdx.z;
  const T* x = static_cast<const T*>(args.x);
  const T* cs = static_cast<const T*>(args.conv_state);
  T* ck = static_cast<T*>(args.conv_ckpt);
  // rows[i] is sequence element t0 - kBack + i of [conv_state rows, x rows].
  Raw8<T> rows[kChainPos + kBack];
#pragma unroll
  for (int i = 0; i < kChainPos + kBack; ++i) {
    const int s = t0 - kBack + i;
    if (s < 0)
      rows[i].load(cs + (static_cast<size_t>(r) * kBack + (s + kBack)) * C + c0);
    else if (s < t0 + tn)
      rows[i].load(x + (static_cast<size_t>(r) * T_ + s) * C + c0);
  }
  float wt[8][kWidth];
  load_weights<T>(static_cast<const T*>(args.w), c0, wt);
#pragma unroll
  for (int j = 0; j < kChainPos; ++j) {
    if (j < tn) {
      const int t = t0 + j;
      const Raw8<T> win[kWidth] = {rows[j], rows[j + 1], rows[j + 2], rows[j + 3]};
      conv_out<T>(wt, win, args.silu, args.y + (static_cast<size_t>(r) * T_ + t) * C + c0);
      if (STORE) {
        T* dst = ck + (static_cast<size_t>(r) * T_ + t) * kBack * C + c0;
#pragma unroll
        for (int m = 0; m < kBack; ++m) win[m + 1].store_nt(dst + static_cast<size_t>(m) * C);
      }
    }
  }
}

// No capture (chain): one thread per 8-channel group walks the positions.
template <typename T>
__global__ __launch_bounds__(kThreads) void conv_inplace_kernel(const ConvArgs args) {
  args_in_registers(args.x, args.w, args.conv_state, args.conv_ckpt, args.y, args.n_pos, args.channels,
                    args.req0, args.per_request_table, args.silu);
  const int C = args.channels;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (c0 >= C) return;
  const int T_ = args.n_pos;
  const int r = args.req0 + blockIdx.z;
  const T* x = static_cast<const T*>(args.x);
  T* cs = static_cast<T*>(args.conv_state);
  Raw8<T> win[kWidth];
#pragma unroll
  for (int m = 0; m < kBack; ++m) win[m].load(cs + (static_cast<size_t>(r) * kBack + m) * C + c0);
  float wt[8][kWidth];
  load_weights<T>(static_cast<const T*>(args.w), c0, wt);
  for (int t = 0; t < T_; ++t) {
    win[kBack].load(x + (static_cast<size_t>(r) * T_ + t) * C + c0);
    conv_out<T>(wt, win, args.silu, args.y + (static_cast<size_t>(r) * T_ + t) * C + c0);
#pragma unroll
    for (int m = 0; m < kBack; ++m) win[m] = win[m + 1];
  }
#pragma unroll
  for (int m = 0; m < kBack; ++m) win[m].store(cs + (static_cast<size_t>(r) * kBack + m) * C + c0);
}

// Modes: capture (y and conv checkpoints), y only with a read-only conv
// state, or in-place decode (chain, conv_state advanced).
enum class ConvMode { kCapture, kOutputOnly, kInPlace };

template <typename T>
hipError_t launch(ConvArgs& args, ConvMode mode, bool tree, int n, hipStream_t s) {
  const int groups = args.channels / 8;
  dim3 block(kThreads);
  const unsigned gx = (groups + kThreads - 1) / kThreads;
  if (mode == ConvMode::kInPlace) {
    hipLaunchKernelGGL(conv_inplace_kernel<T>, dim3(gx, 1, n), block, 0, s, args);
  } else if (!tree) {
    dim3 grid(gx, (args.n_pos + kChainPos - 1) / kChainPos, n);
    if (mode == ConvMode::kCapture)
      hipLaunchKernelGGL((conv_chain_kernel<T, true>), grid, block, 0, s, args);
    else
      hipLaunchKernelGGL((conv_chain_kernel<T, false>), grid, block, 0, s, args);
  } else {
    dim3 grid(gx, args.n_pos, n);
    if (mode == ConvMode::kCapture)
      hipLaunchKernelGGL((conv_capture_kernel<T, true>), grid, block, 0, s, args);
    else
      hipLaunchKernelGGL((conv_capture_kernel<T, false>), grid, block, 0, s, args);
  }
  return launch_error();
}

struct AdvanceArgs {
  const void* x;
  void* conv_state;
  const int32_t* path;
  const int32_t* accept_len;
  int32_t* status;
  int32_t n_req;
  int32_t n_pos;
  int32_t channels;
};

// conv_state[l][r] <- last W-1 rows of [conv_state[l][r], x[l][r][path...]].
// Grid (channel groups / kThreads, R, L). Each thread loads the rows it needs
// for its 8 channels before storing any, so the in-place shift of old state
// rows is safe.
template <typename T>
__global__ __launch_bounds__(kThreads) void conv_advance_kernel(const AdvanceArgs args) {
  const int C = args.channels;
  const int T_ = args.n_pos;
  const int r = blockIdx.y;
  const int l = blockIdx.z;
  if (args.status != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
    int32_t bad = 0;
    for (int i = 0; i < args.n_req; ++i) {
      const int32_t len = args.accept_len[i];
      bool ok = len >= 0 && len < T_;
      for (int j = 0; ok && j <= len; ++j) {
        const int32_t p = args.path[static_cast<size_t>(i) * T_ + j];
        ok = p >= 0 && p < T_;
      }
      bad += ok ? 0 : 1;
    }
    *args.status = bad;
  }
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (c0 >= C) return;
  const int len = args.accept_len[r];
  if (len < 0 || len >= T_) return;
  const int n = len + 1;  // positions on the accepted path
  const int32_t* path = args.path + static_cast<size_t>(r) * T_;
  const size_t lr = static_cast<size_t>(l) * args.n_req + r;
  const T* x = static_cast<const T*>(args.x) + lr * T_ * C;
  T* cs = static_cast<T*>(args.conv_state) + lr * kBack * C;
  int src[kBack];
#pragma unroll
  for (int m = 0; m < kBack; ++m) {
    const int j = n + m;  // index into [state rows 0..W-2, x rows of the path]
    if (j < kBack) {
      src[m] = -1 - j;
    } else {
      const int p = path[j - kBack];
      if (p < 0 || p >= T_) return;
      src[m] = p;
    }
  }
  Raw8<T> rows[kBack];
#pragma unroll
  for (int m = 0; m < kBack; ++m) {
    if (src[m] >= 0)
      rows[m].load(x + static_cast<size_t>(src[m]) * C + c0);
    else
      rows[m].load(cs + static_cast<size_t>(-1 - src[m]) * C + c0);
  }
#pragma unroll
  for (int m = 0; m < kBack; ++m) rows[m].store(cs + static_cast<size_t>(m) * C + c0);
}

}  // namespace
}  // namespace hrs

using namespace hrs;

static int conv_span_impl(const hrs_conv_desc* d, const void* x, const void* w, void* conv_state,
                          void* conv_ckpt, float* y, void* stream, bool output_only) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_req < 1 || d->channels < 8 || d->channels % 8 != 0 || d->width < 2) return HRS_EINVAL;
  if (!dtype_ok(d->dtype)) return HRS_EINVAL;
  if (d->topo != HRS_CHAIN && d->topo != HRS_TREE) return HRS_EINVAL;
  if (!x || !w || !conv_state || !y) return HRS_EINVAL;
  if (d->topo == HRS_TREE && conv_ckpt == nullptr && !output_only) return HRS_EINVAL;
  if (d->n_req > 65535 * 64) return HRS_EINVAL;
  const int geo = check_topology(d->topo, d->parent, d->n_req, d->n_pos);
  if (geo != HRS_OK) return geo;
  if (!aligned16(x) || !aligned16(w) || !aligned16(conv_state) || !aligned16(y) ||
      (conv_ckpt && !aligned16(conv_ckpt)))
    return HRS_EALIGN;
  if (d->width != kWidth) return HRS_EUNSUPPORTED;

  ConvArgs args;
  args.x = x; args.w = w; args.conv_state = conv_state; args.conv_ckpt = conv_ckpt; args.y = y;
  args.n_pos = d->n_pos; args.channels = d->channels; args.silu = d->silu != 0;
  const bool tree = d->topo == HRS_TREE;
  const ConvMode mode = output_only ? ConvMode::kOutputOnly
                                    : (conv_ckpt != nullptr ? ConvMode::kCapture : ConvMode::kInPlace);
  const int T_ = d->n_pos;
  const int table = T_ * kBack;
  int per_launch = 65535;
  args.per_request_table = tree ? 1 : 0;
  if (tree) per_launch = std::max(1, kGeomBytes / table);
  else conv_window_sources(nullptr, T_, kWidth, args.src);

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (int r0 = 0; r0 < d->n_req; r0 += per_launch) {
    const int n = std::min(per_launch, d->n_req - r0);
    args.req0 = r0;
    if (tree)
      for (int i = 0; i < n; ++i)
        conv_window_sources(d->parent + static_cast<size_t>(r0 + i) * T_, T_, kWidth, args.src + i * table);
    const hipError_t e = d->dtype == HRS_BF16 ? launch<uint16_t>(args, mode, tree, n, s)
                                              : launch<float>(args, mode, tree, n, s);
    if (e != hipSuccess) return HRS_EDEVICE;
  }
  return HRS_OK;
}

extern "C" int conv1d_verify_span(const hrs_conv_desc* d, const void* x, const void* w, void* conv_state,
                                  void* conv_ckpt, float* y, void* stream) {
  return conv_span_impl(d, x, w, conv_state, conv_ckpt, y, stream, false);
}

extern "C" int conv1d_verify_span_nocapture(const hrs_conv_desc* d, const void* x, const void* w,
                                            const void* conv_state, float* y, void* stream) {
  return conv_span_impl(d, x, w, const_cast<void*>(conv_state), nullptr, y, stream, true);
}

extern "C" int conv_state_advance(const hrs_conv_advance_desc* d, const void* x, void* conv_state,
                                  const int32_t* path, const int32_t* accept_len, int32_t* status, void* stream) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_layers < 1 || d->n_req < 1 || d->n_pos < 1 || d->n_pos > HRS_MAX_POS || d->channels < 8 ||
      d->channels % 8 != 0 || d->width < 2 || !dtype_ok(d->dtype))
    return HRS_EINVAL;
  if (!x || !conv_state || !path || !accept_len) return HRS_EINVAL;
  if (d->n_req > 65535 || d->n_layers > 65535) return HRS_EINVAL;
  if (!aligned16(x) || !aligned16(conv_state) || !aligned16(path) || !aligned16(accept_len) ||
      (status && !aligned16(status)))
    return HRS_EALIGN;
  if (d->width != kWidth) return HRS_EUNSUPPORTED;
  AdvanceArgs args;
  args.x = x; args.conv_state = conv_state; args.path = path; args.accept_len = accept_len; args.status = status;
  args.n_req = d->n_req; args.n_pos = d->n_pos; args.channels = d->channels;
  const dim3 grid((d->channels / 8 + kThreads - 1) / kThreads, d->n_req, d->n_layers);
  (void)hipGetLastError();
  if (d->dtype == HRS_BF16)
    hipLaunchKernelGGL(conv_advance_kernel<uint16_t>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), args);
  else
    hipLaunchKernelGGL(conv_advance_kernel<float>, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), args);
  return launch_error() == hipSuccess ? HRS_OK : HRS_EDEVICE;
}
