// Host-logic check of the tree stash schedule and the conv window-source
// table (built with g++ against csrc/validate.cpp by tests/test_host_schedule.py).
//
// Schedule: replay it symbolically. "cur" holds the index of the position whose
// state the registers hold (-1 = the pre-span state); every restore must hand
// position t the state of parent[t], and a stash slot must never be overwritten
// while a later reader still needs it.
// Window sources: compare with the root path walked explicitly.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "internal.h"

using namespace hrs;

static int check_schedule(const std::vector<int32_t>& parent, int n_slots, int* used_global) {
  const int T = static_cast<int>(parent.size());
  std::vector<int8_t> restore(T), save(T);
  gdn_tree_schedule(parent.data(), T, n_slots, restore.data(), save.data());
  int cur = -1;
  int slot[kStashSlots];
  for (int i = 0; i < kStashSlots; ++i) slot[i] = -100;
  for (int t = 0; t < T; ++t) {
    int src;
    if (restore[t] == kFromPrevious) src = cur;
    else if (restore[t] == kFromGlobal) { src = parent[t]; ++*used_global; }
    else if (restore[t] >= 0 && restore[t] < n_slots) src = slot[restore[t]];
    else { std::printf("bad restore code %d at %d\n", restore[t], t); return 1; }
    const int want = t == 0 ? -1 : parent[t];
    if (src != want) { std::printf("position %d starts from %d, parent is %d\n", t, src, want); return 1; }
    cur = t;
    if (save[t] >= 0) {
      if (save[t] >= n_slots) { std::printf("bad save slot\n"); return 1; }
      slot[save[t]] = t;
    }
  }
  return 0;
}

static int check_window(const std::vector<int32_t>& parent, bool chain) {
  const int T = static_cast<int>(parent.size());
  std::vector<int8_t> src(T * 3);
  conv_window_sources(chain ? nullptr : parent.data(), T, 4, src.data());
  for (int t = 0; t < T; ++t) {
    std::vector<int> path;  // root .. t
    for (int n = t; n >= 0; n = parent[n]) path.insert(path.begin(), n);
    // sequence = [cs0, cs1, cs2, x[path...]]; window slots m = last 4 entries minus the current
    const int len = 3 + static_cast<int>(path.size());
    for (int m = 0; m < 3; ++m) {
      const int j = len - 4 + m;
      const int want = j < 3 ? -1 - j : path[j - 3];
      if (src[t * 3 + m] != want) { std::printf("window t=%d m=%d got %d want %d\n", t, m, src[t * 3 + m], want); return 1; }
    }
  }
  return 0;
}

int main() {
  std::vector<std::vector<int32_t>> cases = {
    {-1},
    {-1, 0, 1, 2, 3, 4},                          // chain
    {-1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0},        // root with 11 children: one slot reused
    {-1, 0, 0, 1, 1, 2, 3, 3},
    {-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9},  // 10 live branch points > 8 slots
  };
  std::mt19937 rng(7);
  for (int trial = 0; trial < 20000; ++trial) {
    const int T = 1 + static_cast<int>(rng() % 64);
    std::vector<int32_t> p(T, -1);
    const int mode = trial % 3;
    for (int i = 1; i < T; ++i) {
      if (mode == 0) p[i] = static_cast<int32_t>(rng() % i);
      else if (mode == 1) p[i] = (rng() % 4 == 0) ? static_cast<int32_t>(rng() % i) : i - 1;
      else p[i] = std::max(0, i - 1 - static_cast<int>(rng() % 3));
    }
    cases.push_back(p);
  }
  int global = 0, overflow_case = 0;
  for (size_t c = 0; c < cases.size(); ++c) {
    int g = 0;
    for (int ns = 0; ns <= kStashSlots; ++ns) {
      int g0 = 0;
      if (check_schedule(cases[c], ns, &g0)) { std::printf("schedule case %zu slots %d failed\n", c, ns); return 1; }
      if (ns == kStashSlots) g = g0;
    }
    if (check_window(cases[c], false)) { std::printf("window case %zu failed\n", c); return 1; }
    if (c == 4) overflow_case = g;
    global += g;
  }
  std::vector<int32_t> chain(17);
  for (int i = 0; i < 17; ++i) chain[i] = i - 1;
  if (check_window(chain, true)) return 1;
  if (overflow_case != 2) { std::printf("expected 2 global reloads in the 10-branch case, got %d\n", overflow_case); return 1; }
  std::printf("OK %zu trees, %d global reloads\n", cases.size(), global);
  return 0;
}
