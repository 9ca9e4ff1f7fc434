"""Draft-tree geometry guard: the oracle (test infrastructure only).

lucebox PR #506 (Safety boundary) keeps verification fail-closed: sibling,
malformed-root, skipped-parent, cyclic/forward-parent, out-of-range,
truncated and null geometry are rejected before anything executes; only a
root-inclusive pure chain is accepted there. This library also verifies
trees, so the guard has two modes: ``require_chain`` (the page's rule) and a
tree mode in which siblings and non-adjacent parents are legal.

Geometry is a parent array over T positions: position 0 is the committed
root (parent -1), every other position names an earlier position.

Verdict codes (lowest-index offending position decides; per position the
checks run in the order listed):
  0 OK
  1 NULL       no parent array where one is required
  2 TRUNCATED  T outside [1, max_pos]
  3 ROOT       parent[0] != -1, or a second root (parent[i] == -1, i > 0)
  4 RANGE      parent[i] < -1 or parent[i] >= T
  5 FORWARD    i <= parent[i] < T (self, cyclic or forward parent)
  6 NOT_CHAIN  chain mode only: parent[i] != i - 1 (covers the page's
               "sibling" and "skipped-parent" classes)

Pins (tests/test_oracle_geometry.py): the hand-built cases of
tests/golden/tree_geometry.txt, one or more per class named on the page, and
acyclicity of every accepted array checked by walking to the root. Parity
pinned.
"""
from __future__ import annotations

OK, NULL, TRUNCATED, ROOT, RANGE, FORWARD, NOT_CHAIN = range(7)
NAMES = {OK: "OK", NULL: "NULL", TRUNCATED: "TRUNCATED", ROOT: "ROOT",
         RANGE: "RANGE", FORWARD: "FORWARD", NOT_CHAIN: "NOT_CHAIN"}
MAX_POS = 64


def check_tree(parent, n_pos: int, require_chain: bool, max_pos: int = MAX_POS) -> int:
    if parent is None:
        return NULL
    if n_pos < 1 or n_pos > max_pos:
        return TRUNCATED
    for i in range(n_pos):
        p = int(parent[i])
        if i == 0:
            if p != -1:
                return ROOT
            continue
        if p == -1:
            return ROOT
        if p < -1 or p >= n_pos:
            return RANGE
        if p >= i:
            return FORWARD
        if require_chain and p != i - 1:
            return NOT_CHAIN
    return OK
