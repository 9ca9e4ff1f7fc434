// ring_set_2d / ring_get_2d: batched feature-ring row copies with wraparound.
//
// lucebox PR #533 ("feat: DFlash support for tensor-parallel Qwen3.6
// targets"), Changes: the draft's feature ring is kept in step on the device
// by 2-D row copies (a set and a get per stretch of rows that does not wrap),
// so no per-token host round trip or stream wait is left.
//
// MI355X design: the host splits wrapping runs into non-wrapping segments and
// passes them in the kernel arguments, so one launch copies every row of
// every run. Grid = (4 KiB column chunk, segment, row within the segment):
// a block reads its segment's fields at an index it knows at entry, so the
// copy waits for one round of argument loads (a binary search over the
// segments' row prefix sums took one dependent round per step; 16 requests
// of 17 rows: 24 segments); blocks past their segment's length return at
// once. 16 bytes per lane.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "device.h"
#include "internal.h"

namespace hrs {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSeg = 120;

struct RingArgs {
  u32x4* dst_ring;         // set: ring written; get: nullptr
  const u32x4* src_ring;   // get: ring read; set: nullptr
  u32x4* dst_packed;
  const u32x4* src_packed;
  int64_t row_vecs;        // 16-byte vectors per row
  int32_t n_slots;
  int32_t n_seg;
  int32_t seg_ring[kMaxSeg];
  int32_t seg_slot[kMaxSeg];
  int32_t seg_row[kMaxSeg];     // first packed row of the segment
  int32_t seg_n[kMaxSeg];       // rows of the segment
};

__global__ __launch_bounds__(kThreads) void ring_copy_kernel(const RingArgs args) {
  const int sg = blockIdx.y;    // < n_seg (the grid's y extent)
  const int i = blockIdx.z;     // row within the segment
  args_in_registers(args.dst_ring, args.src_ring, args.dst_packed, args.src_packed, args.row_vecs, args.n_slots,
                    args.seg_ring[sg], args.seg_slot[sg], args.seg_row[sg], args.seg_n[sg]);
  if (i >= args.seg_n[sg]) return;
  const int64_t slot = static_cast<int64_t>(args.seg_ring[sg]) * args.n_slots + args.seg_slot[sg] + i;
  const int64_t prow = static_cast<int64_t>(args.seg_row[sg]) + i;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= args.row_vecs) return;
  if (args.dst_ring) {
    args.dst_ring[slot * args.row_vecs + e] = args.src_packed[prow * args.row_vecs + e];
  } else {
    args.dst_packed[prow * args.row_vecs + e] = args.src_ring[slot * args.row_vecs + e];
  }
}

struct Seg {
  int32_t ring, slot, n, row;
};

int check_and_split(const hrs_ring_desc* d, bool set, std::vector<Seg>& segs) {
  if (d == nullptr) return HRS_EINVAL;
  if (d->n_rings < 1 || d->n_slots < 1 || d->width < 1 || d->n_packed_rows < 0 || d->n_runs < 0)
    return HRS_EINVAL;
  if (!dtype_ok(d->dtype)) return HRS_EINVAL;
  if ((static_cast<int64_t>(d->width) * dtype_size(d->dtype)) % 16 != 0) return HRS_EINVAL;
  if (d->n_runs > 0 && d->runs == nullptr) return HRS_EINVAL;
  for (int i = 0; i < d->n_runs; ++i) {
    const hrs_ring_run& r = d->runs[i];
    if (r.ring_id < 0 || r.ring_id >= d->n_rings) return HRS_EINVAL;
    if (r.start_pos < 0 || r.start_pos >= d->n_slots) return HRS_EINVAL;
    if (r.n_rows < 0 || r.n_rows > d->n_slots) return HRS_EINVAL;
    if (r.packed_row < 0 || static_cast<int64_t>(r.packed_row) + r.n_rows > d->n_packed_rows) return HRS_EINVAL;
    if (r.n_rows == 0) continue;
    const int32_t first = std::min(r.n_rows, d->n_slots - r.start_pos);
    segs.push_back({r.ring_id, r.start_pos, first, r.packed_row});
    if (r.n_rows > first) segs.push_back({r.ring_id, 0, r.n_rows - first, r.packed_row + first});
  }
  // Destinations must not overlap: the result would depend on copy order.
  std::vector<std::pair<int64_t, int64_t>> iv;
  iv.reserve(segs.size());
  for (const Seg& s : segs) {
    const int64_t b = set ? static_cast<int64_t>(s.ring) * d->n_slots + s.slot : s.row;
    iv.push_back({b, b + s.n});
  }
  std::sort(iv.begin(), iv.end());
  for (size_t i = 1; i < iv.size(); ++i)
    if (iv[i].first < iv[i - 1].second) return HRS_EINVAL;
  return HRS_OK;
}

int ring_copy(const hrs_ring_desc* d, bool set, void* ring_w, const void* ring_r, void* packed_w,
              const void* packed_r, void* stream) {
  std::vector<Seg> segs;
  const int st = check_and_split(d, set, segs);
  if (st != HRS_OK) return st;
  const void* ring = set ? ring_w : ring_r;
  const void* packed = set ? packed_r : packed_w;
  if (!ring || (!packed && d->n_packed_rows > 0)) return HRS_EINVAL;
  if (!aligned16(ring) || !aligned16(packed)) return HRS_EALIGN;
  if (segs.empty()) return HRS_OK;
  // A segment is one grid z extent: split any longer than the z limit.
  constexpr int32_t kMaxRows = 65535;
  std::vector<Seg> parts;
  parts.reserve(segs.size());
  for (const Seg& g : segs)
    for (int32_t o = 0; o < g.n; o += kMaxRows)
      parts.push_back({g.ring, g.slot + o, std::min(kMaxRows, g.n - o), g.row + o});
  segs.swap(parts);

  RingArgs args;
  args.dst_ring = set ? static_cast<u32x4*>(ring_w) : nullptr;
  args.src_ring = set ? nullptr : static_cast<const u32x4*>(ring_r);
  args.dst_packed = set ? nullptr : static_cast<u32x4*>(packed_w);
  args.src_packed = set ? static_cast<const u32x4*>(packed_r) : nullptr;
  args.row_vecs = static_cast<int64_t>(d->width) * dtype_size(d->dtype) / 16;
  args.n_slots = d->n_slots;
  const dim3 block(kThreads);
  const unsigned gx = static_cast<unsigned>((args.row_vecs + kThreads - 1) / kThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  size_t i = 0;
  while (i < segs.size()) {
    int n = 0;
    int longest = 0;   // grid z extent: the longest segment of this launch (<= n_slots)
    while (i < segs.size() && n < kMaxSeg) {
      args.seg_ring[n] = segs[i].ring;
      args.seg_slot[n] = segs[i].slot;
      args.seg_row[n] = segs[i].row;
      args.seg_n[n] = segs[i].n;
      longest = std::max(longest, static_cast<int>(segs[i].n));
      ++n;
      ++i;
    }
    args.n_seg = n;
    hipLaunchKernelGGL(ring_copy_kernel, dim3(gx, n, longest), block, 0, s, args);
    if (launch_error() != hipSuccess) return HRS_EDEVICE;
  }
  return HRS_OK;
}

}  // namespace
}  // namespace hrs

extern "C" int ring_set_2d(const hrs_ring_desc* d, void* ring, const void* packed, void* stream) {
  return hrs::ring_copy(d, true, ring, nullptr, nullptr, packed, stream);
}

extern "C" int ring_get_2d(const hrs_ring_desc* d, const void* ring, void* packed, void* stream) {
  return hrs::ring_copy(d, false, nullptr, ring, packed, nullptr, stream);
}
