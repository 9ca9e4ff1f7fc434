"""CPU oracle for the speculative verify-span hot path. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The GPU library never calls it, and it shares no code with the
GPU library: no kernels, headers, helpers, tables or pre/post-processing.

Everything here is plain, slow and written to be checked by eye against its
definition. Floating point is float64, except where the pages fix a
precision: the recurrent state is stored as float32 after every position
("F32 SSM checkpoints", lucebox PR #506, Summary and Memory trade-off), so the
oracle carries a float32-rounded state from one position to the next, and
outputs are rounded to float32 once.

What each module computes and where it comes from:
  gdn       - the gated delta rule over a chain or parent-indexed tree of
              positions, state checkpoint after every position
              (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025,
              recurrence of the gated delta rule; checkpoint capture from
              lucebox PR #506, Summary).
  conv      - causal depthwise conv1d of width W over the same positions,
              conv state (last W-1 inputs) captured after every position
              (openinfer PR #626, What Changed: hybrid state includes the
              conv state; lucebox PR #533, Changes: conv state restored on
              device).
  accept    - row argmax and greedy acceptance for a chain or a tree
              (openinfer PR #626, Summary: one active greedy request;
              lucebox PR #533, Verification: chain speculative generation
              and DDTree).
  rollback  - the rolled-back state defined by replaying the accepted path
              from the pre-span state (openinfer PR #626, What Changed:
              conservative commit that restores the canonical state and
              replays the accepted span), which the checkpoint restore of
              lucebox PR #506 must reproduce without replay.
  ring      - feature-ring row placement with wraparound (lucebox PR #533,
              Changes: one get_2d and one set_2d per non-wrapping run).
  geometry  - the draft-tree geometry guard (lucebox PR #506, Safety
              boundary).
  fused     - one layer in its own order: conv with SiLU, split into q/k/v
              heads, q/k L2 norm, gated delta rule (composition of the above).

Parity status of each function is stated in its module header.
"""
from . import accept, conv, fused, gdn, geometry, ring, rollback  # noqa: F401
from .common import widen  # noqa: F401
