// accept_greedy: target argmax per verified position and greedy acceptance of
// the longest matching prefix (chain) or root path (draft tree).
//
// Greedy verification of one draft block (openinfer PR #626, "feat(qwen35):
// add opt-in DFlash speculative decoding", Summary: the output must match
// plain greedy decoding); chain and DDTree verification (lucebox PR #533,
// "feat: DFlash support for tensor-parallel Qwen3.6 targets", Verification).
//
// MI355X design: the argmax rows are long (151,936 entries) and few (T per
// request), so pass 1 splits every row into 16384-entry chunks, one block
// each, streaming 16-byte nontemporal loads (each thread issues its eight
// loads before its first compare; chunks of 8192 measured 2% slower, of
// 32768 7% slower). A chunk is reduced in two passes over the registers: the
// largest value by a chain of IEEE maximum operations over quieted values
// (NaN never wins; three operands fold into one instruction), then the
// lowest index holding that value (float equality, so -0 and +0 tie and the
// lower index wins). Only the per-thread result becomes a 64-bit key (ordered
// value bits above the complemented index); the block's maximum key goes to
// the caller's workspace. Taking the maximum key realises "largest value,
// lowest index on ties, NaN never wins" in any reduction order, so the result
// is deterministic. (A 64-bit key per element cost ~14 vector instructions
// per logit and made pass 1 compute-bound; this form costs ~5.) Pass 2 is one
// wave per request: the lanes issue the loads of the row keys, the draft
// tokens and the parents in one round (64-bit maximum per row in LDS), then
// a chain is accepted by one ballot (position t matches when its draft token
// equals the argmax at t - 1; the accepted length is the run of matches from
// position 1) and a tree by one lane walking its T <= 64 positions in LDS.
// The kernel boundary orders the two passes. (Finishing each request in pass
// 1 instead, in the block that counts itself last in a per-request arrival
// counter, was slower: with 323 blocks per request counting on one address
// the device-scope atomics serialise, 72 us against 27 us for the two passes
// at the time, 16 requests x 17 rows of 151,936 logits.)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "device.h"
#include "internal.h"

namespace hrs {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16384;  // logits per pass-1 block
static_assert(kChunk % (kThreads * 8) == 0, "whole 8-logit slices per thread");

struct AcceptArgs {
  const int32_t* tokens;
  const uint64_t* keys;   // workspace [rows][n_chunks]
  int32_t* argmax;
  int32_t* accept_node;
  int32_t* accept_len;
  int32_t* path;
  int32_t* bonus;
  int32_t n_pos;
  int32_t n_chunks;
  int32_t req0;
  int32_t tree;
  int8_t parent[kGeomBytes];  // tree: [requests of this launch][n_pos]
};

// Order-preserving map of a float to u32: NaN -> 0 (below everything),
// -0 -> +0, otherwise larger floats map to larger integers.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  if (x != x) return 0u;
  if (x == 0.0f) x = 0.0f;
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float x, uint32_t idx) {
  return (static_cast<uint64_t>(ordered_bits(x)) << 32) | static_cast<uint64_t>(~idx);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

constexpr int kIter = kChunk / (kThreads * 8);   // 16-byte slices per thread

// The key of this thread's slices. Values are quieted first: in IEEE mode a
// signalling NaN operand makes the hardware maximum return NaN (a bf16 NaN
// whose top mantissa bit is clear widens to one), while a quiet NaN operand
// is skipped. Slices it >= n_valid (past the row's end) take no part.
__device__ __forceinline__ uint64_t thread_key(float (&v)[kIter][8], const int (&e)[kIter], int n_valid) {
  float m = -__builtin_inff();
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[it][i] = __builtin_canonicalizef(v[it][i]);
    if (it < n_valid) {
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, v[it][i]);
    }
  }
  uint32_t idx = 0xFFFFFFFFu;
#pragma unroll
  for (int it = kIter - 1; it >= 0; --it) {
    if (it < n_valid) {
#pragma unroll
      for (int i = 7; i >= 0; --i) idx = v[it][i] == m ? static_cast<uint32_t>(e[it] + i) : idx;
    }
  }
  if (idx != 0xFFFFFFFFu) return make_key(m, idx);
  // No element equals m: every valid element is NaN (the key of the lowest
  // index, below every number), or the thread has no valid slice.
  return n_valid > 0 ? make_key(__builtin_nanf(""), static_cast<uint32_t>(e[0])) : 0;
}

// The logits are read once: nontemporal loads (16 requests x 17 rows x
// 151,936 bf16 logits: 18.2 vs 19.7 us per call with plain loads).
template <typename T> __device__ __forceinline__ void load8_nt(const T* p, float* o);
template <> __device__ __forceinline__ void load8_nt<uint16_t>(const uint16_t* p, float* o) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x);
  o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
  o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z);
  o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
}
template <> __device__ __forceinline__ void load8_nt<float>(const float* p, float* o) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
  o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void argmax_partial_kernel(const T* logits, uint64_t* keys, int32_t vocab,
                                                                  int32_t n_chunks) {
  const int row = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x % n_chunks;
  const T* base = logits + static_cast<size_t>(row) * vocab;
  const int begin = chunk * kChunk;
  const int end = min(vocab, begin + kChunk);
  // All of the thread's loads are issued before the first use; slices past
  // the row's end re-read the chunk's last eight logits (end - 8 >= begin
  // since vocab is a multiple of 8) and are left out. Slice it starts at
  // begin + (it * kThreads + tid) * 8, so the valid slices are a prefix.
  float v[kIter][8];
  int e[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    e[it] = begin + (it * kThreads + threadIdx.x) * 8;
    load8_nt<T>(base + min(e[it], end - 8), v[it]);
  }
  int n_valid = 0;
#pragma unroll
  for (int it = 0; it < kIter; ++it) n_valid += e[it] < end ? 1 : 0;
  uint64_t best = thread_key(v, e, n_valid);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(best, m);
    best = o > best ? o : best;
  }
  __shared__ uint64_t wave_best[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t b = wave_best[0];
    for (int i = 1; i < kThreads / 64; ++i) b = wave_best[i] > b ? wave_best[i] : b;
    keys[blockIdx.x] = b;
  }
}

__global__ __launch_bounds__(64) void accept_walk_kernel(const AcceptArgs args) {
  const int T_ = args.n_pos;
  const int rl = blockIdx.x;
  const int r = args.req0 + rl;
  const int lane = threadIdx.x;
  __shared__ unsigned long long row_key[HRS_MAX_POS];
  __shared__ int32_t am[HRS_MAX_POS];
  __shared__ int32_t tok[HRS_MAX_POS];
  __shared__ int32_t par[HRS_MAX_POS];
  __shared__ int32_t path_s[HRS_MAX_POS];
  __shared__ int32_t depth[HRS_MAX_POS];
  __shared__ int32_t matched[HRS_MAX_POS];
  __shared__ int32_t len_s;
  // Everything the walk reads is loaded first, by all lanes at once and in
  // one round trip to memory: the row's chunk keys (eight per lane, from
  // clamped indices), the draft tokens and the parents; the walk itself then
  // touches LDS only.
  const int n_keys = T_ * args.n_chunks;
  const uint64_t* k = args.keys + static_cast<size_t>(r) * n_keys;
  const int tl = min(lane, T_ - 1);
  const int32_t tk = args.tokens[static_cast<size_t>(r) * T_ + tl];
  const int32_t pr = args.tree ? args.parent[rl * T_ + tl] : tl - 1;
  for (int i0 = 0; i0 < n_keys; i0 += 64 * 8) {
    uint64_t kv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kv[j] = k[min(i0 + lane + 64 * j, n_keys - 1)];
    if (i0 == 0) {
      if (lane < T_) {
        row_key[lane] = 0;
        tok[lane] = tk;
        par[lane] = pr;
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + lane + 64 * j;
      if (i < n_keys) atomicMax(&row_key[i / args.n_chunks], static_cast<unsigned long long>(kv[j]));
    }
  }
  __syncthreads();
  if (lane < T_) {
    const int32_t idx = static_cast<int32_t>(~static_cast<uint32_t>(row_key[lane]));
    am[lane] = idx;
    args.argmax[static_cast<size_t>(r) * T_ + lane] = idx;
  }
  __syncthreads();
  if (!args.tree) {
    // Chain: position t is accepted when every position 1..t matches, i.e.
    // draft token t equals the argmax at t - 1; the accepted length is the
    // run of matches from position 1 (one ballot), the path 0..len.
    const bool m = lane >= 1 && lane < T_ && tok[lane] == am[lane - 1];
    const uint64_t mask = __ballot(m);
    const int len = __builtin_ctzll(~(mask >> 1));
    if (lane == 0) {
      args.accept_node[r] = len;
      args.accept_len[r] = len;
      args.bonus[r] = am[len];
    }
    if (lane < T_) args.path[static_cast<size_t>(r) * T_ + lane] = lane <= len ? lane : -1;
    return;
  }
  if (lane == 0) {
    matched[0] = 1;
    depth[0] = 0;
    int32_t best = 0;
    for (int t = 1; t < T_; ++t) {
      const int p = par[t];
      depth[t] = depth[p] + 1;
      matched[t] = (matched[p] && tok[t] == am[p]) ? 1 : 0;
      if (matched[t] && depth[t] > depth[best]) best = t;
    }
    const int len = depth[best];
    int node = best;
    for (int d = len; d >= 0; --d) {
      path_s[d] = node;
      node = par[node];
    }
    len_s = len;
    args.accept_node[r] = best;
    args.accept_len[r] = len;
    args.bonus[r] = am[best];
  }
  __syncthreads();
  if (lane < T_) args.path[static_cast<size_t>(r) * T_ + lane] = lane <= len_s ? path_s[lane] : -1;
}

}  // namespace
}  // namespace hrs

using namespace hrs;

// Pass 1 runs one block per (row, 16384-logit chunk): at most 2^24 blocks.
constexpr int64_t kMaxChunkBlocks = int64_t{1} << 24;

static bool accept_desc_ok(const hrs_accept_desc* d) {
  return d && d->n_req >= 1 && d->vocab >= 8 && d->vocab % 8 == 0 && dtype_ok(d->logit_dtype) &&
         (d->topo == HRS_CHAIN || d->topo == HRS_TREE) && d->n_pos >= 1 && d->n_pos <= HRS_MAX_POS &&
         static_cast<int64_t>(d->n_req) * d->n_pos <= 65535 * 64 &&
         static_cast<int64_t>(d->n_req) * d->n_pos * ((d->vocab + kChunk - 1) / kChunk) <= kMaxChunkBlocks;
}

static int accept_chunks(const hrs_accept_desc* d) { return (d->vocab + kChunk - 1) / kChunk; }

extern "C" size_t accept_greedy_workspace_bytes(const hrs_accept_desc* d) {
  if (!accept_desc_ok(d)) return 0;
  return static_cast<size_t>(d->n_req) * d->n_pos * accept_chunks(d) * sizeof(uint64_t);
}

// Checks shared by both entry points; HRS_OK or the status to return.
static int accept_check(const hrs_accept_desc* d, const void* logits, const int32_t* tokens, const int32_t* argmax,
                        const int32_t* accept_node, const int32_t* accept_len, const int32_t* path,
                        const int32_t* bonus) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->topo == HRS_TREE || d->topo == HRS_CHAIN) {
    const int geo = check_topology(d->topo, d->parent, d->n_req < 1 ? 0 : d->n_req, d->n_pos);
    if (geo != HRS_OK) return geo;
  }
  if (!accept_desc_ok(d)) return HRS_EINVAL;
  if (!logits || !tokens || !argmax || !accept_node || !accept_len || !path || !bonus) return HRS_EINVAL;
  if (!aligned16(logits) || !aligned16(tokens) || !aligned16(argmax) || !aligned16(accept_node) ||
      !aligned16(accept_len) || !aligned16(path) || !aligned16(bonus))
    return HRS_EALIGN;
  return HRS_OK;
}

// Both passes of a checked call, with the pass-1 keys at `keys` (device
// memory of accept_greedy_workspace_bytes(d) bytes).
static int accept_launch(const hrs_accept_desc* d, const void* logits, const int32_t* tokens, int32_t* argmax,
                         int32_t* accept_node, int32_t* accept_len, int32_t* path, int32_t* bonus, uint64_t* keys,
                         hipStream_t s) {
  const int n_chunks = accept_chunks(d);
  const int rows = d->n_req * d->n_pos;
  (void)hipGetLastError();
  const dim3 grid1(rows * n_chunks);
  if (d->logit_dtype == HRS_BF16)
    hipLaunchKernelGGL(argmax_partial_kernel<uint16_t>, grid1, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(logits), keys, d->vocab, n_chunks);
  else
    hipLaunchKernelGGL(argmax_partial_kernel<float>, grid1, dim3(kThreads), 0, s,
                       static_cast<const float*>(logits), keys, d->vocab, n_chunks);
  if (launch_error() != hipSuccess) return HRS_EDEVICE;

  AcceptArgs args;
  args.tokens = tokens; args.keys = keys; args.argmax = argmax; args.accept_node = accept_node;
  args.accept_len = accept_len; args.path = path; args.bonus = bonus;
  args.n_pos = d->n_pos; args.n_chunks = n_chunks;
  args.tree = d->topo == HRS_TREE;
  const int per_launch = args.tree ? std::max(1, kGeomBytes / d->n_pos) : 65535;
  for (int r0 = 0; r0 < d->n_req; r0 += per_launch) {
    const int n = std::min(per_launch, d->n_req - r0);
    args.req0 = r0;
    if (args.tree)
      for (int i = 0; i < n * d->n_pos; ++i)
        args.parent[i] = static_cast<int8_t>(d->parent[static_cast<size_t>(r0) * d->n_pos + i]);
    hipLaunchKernelGGL(accept_walk_kernel, dim3(n), dim3(64), 0, s, args);
    if (launch_error() != hipSuccess) return HRS_EDEVICE;
  }
  return HRS_OK;
}

extern "C" int accept_greedy(const hrs_accept_desc* d, const void* logits, const int32_t* tokens, int32_t* argmax,
                             int32_t* accept_node, int32_t* accept_len, int32_t* path, int32_t* bonus,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const int st = accept_check(d, logits, tokens, argmax, accept_node, accept_len, path, bonus);
  if (st != HRS_OK) return st;
  if (workspace == nullptr || workspace_bytes < accept_greedy_workspace_bytes(d)) return HRS_EINVAL;
  if (!aligned16(workspace)) return HRS_EALIGN;
  return accept_launch(d, logits, tokens, argmax, accept_node, accept_len, path, bonus,
                       static_cast<uint64_t*>(workspace), static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// accept_greedy_noalloc: the pass-1 keys in a fixed device array instead of a
// caller's workspace, for callers that cannot allocate.

static_assert(HRS_ACCEPT_NOALLOC_MAX_BYTES % 256 == 0, "whole 256-byte lines");

// One copy per GPU the library runs on, held until the process ends. In host
// code this name is only a stand-in for the symbol: the device address of
// each GPU's copy comes from hipGetSymbolAddress on that GPU.
static __device__ __align__(256) unsigned char scratch[HRS_ACCEPT_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with it current) and kept.
static int scratch_address(void** out) {
  int dev = 0;
  const hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) {
    set_last_hip_error(static_cast<int>(e0));
    return HRS_EDEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return HRS_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_address[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    set_last_hip_error(static_cast<int>(e));
    if (e != hipSuccess || p == nullptr) return HRS_EDEVICE;
    g_scratch_address[dev] = p;
  }
  *out = g_scratch_address[dev];
  return HRS_OK;
}

extern "C" int accept_greedy_noalloc(const hrs_accept_desc* d, const void* logits, const int32_t* tokens,
                                     int32_t* argmax, int32_t* accept_node, int32_t* accept_len, int32_t* path,
                                     int32_t* bonus, void* stream) {
  const int st = accept_check(d, logits, tokens, argmax, accept_node, accept_len, path, bonus);
  if (st != HRS_OK) return st;
  if (accept_greedy_workspace_bytes(d) > HRS_ACCEPT_NOALLOC_MAX_BYTES) return HRS_EINVAL;
  void* keys = nullptr;
  const int sa = scratch_address(&keys);
  if (sa != HRS_OK) return sa;
  return accept_launch(d, logits, tokens, argmax, accept_node, accept_len, path, bonus, static_cast<uint64_t*>(keys),
                       static_cast<hipStream_t>(stream));
}
