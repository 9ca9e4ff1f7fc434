// rollback_restore: fast rollback of every layer's recurrent and conv state
// to the accepted position's checkpoint, in one launch, with the accepted
// index read from device memory.
//
// lucebox PR #533 ("feat: DFlash support for tensor-parallel Qwen3.6
// targets"), Changes: both states go back to the accepted position without
// leaving the device, with a single wait once the rollback is done. lucebox
// PR #506 ("perf(dflash): split-chain fast rollback with F32 SSM
// checkpoints"), Summary: the state comes from the float32 checkpoint that
// verification stored at that position, so no accepted token is re-run.
//
// MI355X design: a plain HBM-bound copy. The grid is (64 KiB chunk, layer x
// request) of 1024-thread blocks; each thread issues four 16-byte
// nontemporal loads before its four streaming stores, so every wave keeps
// 4 KiB in flight (on 16 requests x 48 layers, 3.3 GB: 542 us, 6.1 TB/s,
// against 580 us for 256-thread blocks; eight loads per thread were slower;
// 522-531 us, 6.3 TB/s, since the stores also carry the device-scope bit). A block whose request carries an index
// outside [0, T) copies nothing; block (0, 0) alone writes the status word
// (the count of such requests), so the word needs no clearing and no atomics.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace hrs {
namespace {

constexpr int kThreads = 1024;
constexpr int kVecPerThread = 4;
constexpr size_t kChunkBytes = static_cast<size_t>(kThreads) * kVecPerThread * 16;

struct RollbackArgs {
  const u32x4* ckpt;
  u32x4* state;
  const u32x4* conv_ckpt;
  u32x4* conv_state;
  const int32_t* accept_node;
  int32_t* status;
  int64_t state_vecs;   // 16-byte vectors of one (layer, request) state
  int64_t conv_vecs;    // 16-byte vectors of one (layer, request) conv state
  int32_t state_chunks;
  int32_t n_req;
  int32_t n_pos;
};

__device__ __forceinline__ void copy_chunk(const u32x4* src, u32x4* dst, int64_t n_vecs, int64_t chunk) {
  const int64_t base = chunk * (kThreads * kVecPerThread) + threadIdx.x;
  u32x4 v[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t e = base + static_cast<int64_t>(i) * kThreads;
    if (e < n_vecs) v[i] = __builtin_nontemporal_load(src + e);
  }
  // Stores through a buffer resource over the destination with the
  // streaming and device-scope cache bits (nt sc1): 16 requests x 48 layers
  // 525-531 vs 542-545 us with plain nontemporal stores (same GPU, three
  // alternating runs).
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(dst, 0, static_cast<int>(n_vecs * 16), 0x00020000);
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t e = base + static_cast<int64_t>(i) * kThreads;
    if (e < n_vecs) __builtin_amdgcn_raw_buffer_store_b128(v[i], rsrc, static_cast<int>(e * 16), 0, 2 | 16);
  }
}

__global__ __launch_bounds__(kThreads) void rollback_kernel(const RollbackArgs args) {
  const int lr = blockIdx.y;              // layer * R + request
  const int r = lr % args.n_req;
  const int T_ = args.n_pos;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    int32_t bad = 0;
    for (int i = 0; i < args.n_req; ++i) {
      const int32_t u = args.accept_node[i];
      bad += (u < 0 || u >= T_) ? 1 : 0;
    }
    *args.status = bad;
  }
  const int32_t u = args.accept_node[r];
  if (u < 0 || u >= T_) return;
  const int chunk = blockIdx.x;
  if (chunk < args.state_chunks) {
    const u32x4* src = args.ckpt + (static_cast<int64_t>(lr) * T_ + u) * args.state_vecs;
    u32x4* dst = args.state + static_cast<int64_t>(lr) * args.state_vecs;
    copy_chunk(src, dst, args.state_vecs, chunk);
  } else {
    const u32x4* src = args.conv_ckpt + (static_cast<int64_t>(lr) * T_ + u) * args.conv_vecs;
    u32x4* dst = args.conv_state + static_cast<int64_t>(lr) * args.conv_vecs;
    copy_chunk(src, dst, args.conv_vecs, chunk - args.state_chunks);
  }
}

}  // namespace
}  // namespace hrs

using namespace hrs;

extern "C" int rollback_restore(const hrs_rollback_desc* d, const float* ckpt, float* state, const void* conv_ckpt,
                                void* conv_state, const int32_t* accept_node, int32_t* status, void* stream) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_layers < 1 || d->n_req < 1 || d->n_pos < 1 || d->n_pos > HRS_MAX_POS || d->n_vheads < 1 ||
      d->d_k < 1 || d->d_v < 1)
    return HRS_EINVAL;
  if (!ckpt || !state || !accept_node || !status) return HRS_EINVAL;
  const bool conv = conv_ckpt != nullptr || conv_state != nullptr;
  if (conv) {
    if (!conv_ckpt || !conv_state || d->conv_channels < 1 || d->conv_width < 2 || !dtype_ok(d->conv_dtype))
      return HRS_EINVAL;
  }
  if (static_cast<int64_t>(d->n_layers) * d->n_req > 65535) return HRS_EINVAL;
  if (!aligned16(ckpt) || !aligned16(state) || !aligned16(accept_node) || !aligned16(status) ||
      (conv && (!aligned16(conv_ckpt) || !aligned16(conv_state))))
    return HRS_EALIGN;
  const int64_t state_bytes = static_cast<int64_t>(d->n_vheads) * d->d_v * d->d_k * 4;
  const int64_t conv_bytes =
      conv ? static_cast<int64_t>(d->conv_width - 1) * d->conv_channels * static_cast<int64_t>(dtype_size(d->conv_dtype))
           : 0;
  if (state_bytes % 16 != 0 || conv_bytes % 16 != 0) return HRS_EINVAL;
  // The copy addresses one state (or conv state) through a buffer resource
  // whose size is a signed 32-bit byte count.
  if (state_bytes > INT32_MAX || conv_bytes > INT32_MAX) return HRS_EINVAL;

  RollbackArgs args;
  args.ckpt = reinterpret_cast<const u32x4*>(ckpt);
  args.state = reinterpret_cast<u32x4*>(state);
  args.conv_ckpt = static_cast<const u32x4*>(conv_ckpt);
  args.conv_state = static_cast<u32x4*>(conv_state);
  args.accept_node = accept_node;
  args.status = status;
  args.state_vecs = state_bytes / 16;
  args.conv_vecs = conv_bytes / 16;
  args.state_chunks = static_cast<int32_t>((state_bytes + kChunkBytes - 1) / kChunkBytes);
  const int conv_chunks = static_cast<int>((conv_bytes + kChunkBytes - 1) / kChunkBytes);
  args.n_req = d->n_req;
  args.n_pos = d->n_pos;
  const dim3 grid(args.state_chunks + conv_chunks, d->n_layers * d->n_req);
  (void)hipGetLastError();
  hipLaunchKernelGGL(rollback_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), args);
  return launch_error() == hipSuccess ? HRS_OK : HRS_EDEVICE;
}
