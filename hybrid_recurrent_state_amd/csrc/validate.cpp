// Host-only checks of the C ABI: the draft geometry guard, status strings and
// the conv window-source table. No HIP calls, so every rejection path can be
// exercised on a machine without a GPU.
//
// The guard follows lucebox PR #506 ("perf(dflash): split-chain fast rollback
// with F32 SSM checkpoints"), Safety boundary: malformed geometry is rejected
// before anything executes. Chain mode accepts only the root-inclusive pure
// chain; tree mode (draft trees, lucebox PR #533 Verification: DDTree)
// accepts any parent array in topological order.
#include <vector>

#include "internal.h"

extern "C" int hrs_validate_tree(const int32_t* parent, int32_t n_pos, int32_t require_chain,
                                 int32_t* geometry_class) {
  int32_t cls = HRS_GEOM_OK;
  if (parent == nullptr) {
    cls = HRS_GEOM_NULL;
  } else if (n_pos < 1 || n_pos > HRS_MAX_POS) {
    cls = HRS_GEOM_TRUNCATED;
  } else {
    for (int32_t i = 0; i < n_pos && cls == HRS_GEOM_OK; ++i) {
      const int32_t p = parent[i];
      if (i == 0) {
        if (p != -1) cls = HRS_GEOM_ROOT;
      } else if (p == -1) {
        cls = HRS_GEOM_ROOT;
      } else if (p < -1 || p >= n_pos) {
        cls = HRS_GEOM_RANGE;
      } else if (p >= i) {
        cls = HRS_GEOM_FORWARD;
      } else if (require_chain && p != i - 1) {
        cls = HRS_GEOM_NOT_CHAIN;
      }
    }
  }
  if (geometry_class) *geometry_class = cls;
  return cls == HRS_GEOM_OK ? HRS_OK : HRS_EGEOMETRY;
}

extern "C" const char* hrs_strerror(int status) {
  switch (status) {
    case HRS_OK: return "ok";
    case HRS_EINVAL: return "invalid argument (size, null pointer or dtype)";
    case HRS_EGEOMETRY: return "draft geometry rejected";
    case HRS_EALIGN: return "device pointer not 16-byte aligned";
    case HRS_EDEVICE: return "HIP launch failed";
    case HRS_EUNSUPPORTED: return "shape outside the built kernel set";
    default: return "unknown status";
  }
}

extern "C" int hrs_abi_version(void) { return HRS_ABI_VERSION; }

namespace {
thread_local int g_last_hip_error = 0;
}

extern "C" int hrs_last_hip_error(void) { return g_last_hip_error; }

namespace hrs {

void set_last_hip_error(int err) { g_last_hip_error = err; }

int check_topology(int topo, const int32_t* parent, int32_t n_req, int32_t n_pos) {
  if (topo == HRS_CHAIN) {
    return (n_pos >= 1 && n_pos <= HRS_MAX_POS) ? HRS_OK : HRS_EGEOMETRY;
  }
  if (topo != HRS_TREE) return HRS_EINVAL;
  if (parent == nullptr) return HRS_EGEOMETRY;
  for (int32_t r = 0; r < n_req; ++r) {
    if (hrs_validate_tree(parent + static_cast<size_t>(r) * n_pos, n_pos, 0, nullptr) != HRS_OK)
      return HRS_EGEOMETRY;
  }
  return HRS_OK;
}

void gdn_tree_schedule(const int32_t* parent, int32_t n_pos, int n_slots, int8_t* restore, int8_t* save) {
  if (n_slots > kStashSlots) n_slots = kStashSlots;
  std::vector<int32_t> last_child(n_pos, -1);   // last child that is not the next position
  for (int32_t c = 1; c < n_pos; ++c) {
    const int32_t p = parent[c];
    if (c != p + 1) last_child[p] = c;
  }
  std::vector<int32_t> slot_of(n_pos, -1);
  bool busy[kStashSlots] = {false};
  for (int32_t t = 0; t < n_pos; ++t) {
    const int32_t p = parent[t];
    if (t == 0 || p == t - 1) {
      restore[t] = kFromPrevious;
    } else if (slot_of[p] >= 0) {
      restore[t] = static_cast<int8_t>(slot_of[p]);
      if (last_child[p] == t) busy[slot_of[p]] = false;   // last reader frees the slot
    } else {
      restore[t] = kFromGlobal;
    }
    save[t] = -1;
    if (last_child[t] >= 0) {
      for (int i = 0; i < n_slots; ++i) {
        if (!busy[i]) {
          busy[i] = true;
          slot_of[t] = i;
          save[t] = static_cast<int8_t>(i);
          break;
        }
      }
    }
  }
}

void conv_window_sources(const int32_t* parent, int32_t n_pos, int32_t width, int8_t* out) {
  // The window of position t is the last `width` entries of the sequence
  // [conv_state rows..., x along t's root path]; slot m < width-1 is
  // (width-1-m) steps up t's root path, or a conv-state row once the path
  // runs out.
  const int32_t back = width - 1;
  std::vector<int32_t> depth(n_pos, 0);
  for (int32_t t = 0; t < n_pos; ++t) {
    const int32_t p = parent ? parent[t] : t - 1;
    depth[t] = p < 0 ? 0 : depth[p] + 1;
    for (int32_t m = 0; m < back; ++m) {
      const int32_t up = back - m;  // steps above t
      int32_t node = t;
      int32_t steps = 0;
      while (steps < up && node >= 0) {
        node = parent ? parent[node] : node - 1;
        ++steps;
      }
      int8_t src;
      if (node >= 0) {
        src = static_cast<int8_t>(node);
      } else {
        // Ran past the root: position in the padded sequence is depth + m,
        // which indexes the conv state (rows 0..back-1).
        const int32_t row = depth[t] + m;
        src = static_cast<int8_t>(-1 - row);
      }
      out[t * back + m] = src;
    }
  }
}

}  // namespace hrs
