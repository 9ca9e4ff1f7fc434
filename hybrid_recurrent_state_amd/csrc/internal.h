// Internal declarations shared by the library's translation units.
// Host-side checks live in validate.cpp (plain C++, no HIP calls); device
// helpers are only visible when compiling HIP sources.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/hrs.h"

namespace hrs {

// Bytes of per-request geometry a kernel argument block carries. A launch
// covers as many requests as fit; larger batches are split into several
// launches on the same stream.
constexpr int kGeomBytes = 3072;

// Tree schedule of the GDN span: for every position, where its starting
// state comes from and whether its result must be kept for later children.
constexpr int8_t kFromPrevious = -1;  // restore: continue from position t-1
constexpr int8_t kFromGlobal = -2;    // restore: reload checkpoint of parent[t]
constexpr int kStashSlots = 8;        // most stash slots a schedule uses

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_size(hrs_dtype d) { return d == HRS_F32 ? 4 : 2; }

inline bool dtype_ok(int d) { return d == HRS_F32 || d == HRS_BF16; }

// Geometry guard shared by every entry point that takes a topology. Checks
// n_req parent rows of n_pos entries each (tree mode), or n_pos alone
// (chain mode). Returns HRS_OK or HRS_EGEOMETRY.
int check_topology(int topo, const int32_t* parent, int32_t n_req, int32_t n_pos);

// Per-thread record of the last HIP error seen by an entry point (0 = none).
void set_last_hip_error(int err);

// Stash schedule of one request's tree (parent[0] == -1, parent[t] < t).
// restore[t]: kFromPrevious, kFromGlobal, or a slot in [0, n_slots) that
// holds parent[t]'s state (n_slots <= kStashSlots). save[t]: a slot to store position t's state in
// after computing it, or -1. A position's state is stashed when one of its
// children is not the next position; slots are assigned greedily (lowest free
// slot, freed after the last child reads it); when no slot is free the
// children reload the parent's checkpoint from memory.
void gdn_tree_schedule(const int32_t* parent, int32_t n_pos, int n_slots, int8_t* restore, int8_t* save);

// Conv window sources of every position of one request: for window slot m
// (0 = oldest, W-2 = the slot before the current input) the x row to read
// (>= 0) or the conv-state row encoded as -1 - row. parent == nullptr means
// a chain. out has n_pos * (width - 1) entries.
void conv_window_sources(const int32_t* parent, int32_t n_pos, int32_t width, int8_t* out);

}  // namespace hrs
