"""Seeded synthetic inputs for the verify-span hot path.

This module only draws numbers and arranges them into the shapes the path
consumes. It holds none of the method's arithmetic: no recurrence, no
convolution, no argmax and no acceptance rule. Both the CPU oracle (through
the tests and the bench) and the GPU library receive exactly the arrays made
here.

The pages (lucebox PR #533 "feat: DFlash support for tensor-parallel Qwen3.6
targets", lucebox PR #506 "perf(dflash): split-chain fast rollback with F32
SSM checkpoints", openinfer PR #626 "feat(qwen35): add opt-in DFlash
speculative decoding") measure whole models on real prompts; no weights or
prompts are available here, so every workload is synthetic with the shapes
of a Qwen3.6-27B-style Gated DeltaNet layer.

Representation:
  * f32 data is ``np.float32``;
  * bf16 data is carried as its bit pattern in ``np.uint16`` (rounded from
    f32 with round-to-nearest-even);
  * integer data is ``np.int32``.

Seeding: every (layer, request) unit draws from its own
``SeedSequence([seed, layer, request])``, so one unit of a large workload can
be regenerated on its own for sampled checks.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Entropy tags that keep the per-purpose streams apart.
_TAG_CONV_W = 0x7FFF0001
_TAG_LOGITS = 0x7FFF0002
_TAG_RING = 0x7FFF0003
_TAG_TREE = 0x7FFF0004
_TAG_ACCEPT = 0x7FFF0005


def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``np.uint16``. Inputs here are finite.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = x.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for building inputs)."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (bits.astype(np.uint32) << 16).view(np.float32)


def cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits(x32)
    raise ValueError(dtype)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes and input recipe of one synthetic workload."""

    name: str
    seed: int
    n_req: int
    n_layers: int
    n_kheads: int
    n_vheads: int
    d_k: int
    d_v: int
    n_pos: int          # T = K + 1: the committed root plus K draft positions
    dtype: str          # q/k/v/a/b and conv x/w/state dtype
    conv_channels: int
    conv_width: int
    vocab: int          # 0 = no logits (accepted index written directly)
    tree: bool = False
    tree_max_depth: int = 8      # depth of every node is < 8 before a child is added
    tree_max_children: int = 3
    ring_slots: int = 0
    ring_width: int = 0
    logits_distinct: bool = False  # every value of a row distinct (f32 rows only)

    @property
    def n_draft(self) -> int:
        return self.n_pos - 1


# The five workloads. Names say what they are.
WORKLOADS: Dict[str, Workload] = {}


def _reg(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


TINY_CHAIN = _reg(Workload(
    name="tiny-chain-h4-d64-k8", seed=0, n_req=1, n_layers=1, n_kheads=4,
    n_vheads=4, d_k=64, d_v=64, n_pos=9, dtype=F32, conv_channels=768,
    conv_width=4, vocab=1024, logits_distinct=True))
QWEN_LAYER_CHAIN = _reg(Workload(
    name="qwen27b-gdn-layer-chain-k16", seed=1, n_req=1, n_layers=1,
    n_kheads=16, n_vheads=32, d_k=128, d_v=128, n_pos=17, dtype=BF16,
    conv_channels=8192, conv_width=4, vocab=0))
QWEN_STACK_CHAIN = _reg(Workload(
    name="qwen27b-gdn-48layer-chain-k16", seed=2, n_req=1, n_layers=48,
    n_kheads=16, n_vheads=32, d_k=128, d_v=128, n_pos=17, dtype=BF16,
    conv_channels=8192, conv_width=4, vocab=151936))
QWEN_STACK_R16 = _reg(Workload(
    name="qwen27b-gdn-48layer-chain-k16-r16-ring4096", seed=3, n_req=16,
    n_layers=48, n_kheads=16, n_vheads=32, d_k=128, d_v=128, n_pos=17,
    dtype=BF16, conv_channels=8192, conv_width=4, vocab=151936,
    ring_slots=4096, ring_width=5120))
QWEN_STACK_TREE = _reg(Workload(
    name="qwen27b-gdn-48layer-ddtree22", seed=4, n_req=1, n_layers=48,
    n_kheads=16, n_vheads=32, d_k=128, d_v=128, n_pos=23, dtype=BF16,
    conv_channels=8192, conv_width=4, vocab=151936, tree=True))

# Order matches the published list of configurations (small to batched/tree).
WORKLOAD_ORDER: List[str] = [TINY_CHAIN.name, QWEN_LAYER_CHAIN.name,
                             QWEN_STACK_CHAIN.name, QWEN_STACK_R16.name,
                             QWEN_STACK_TREE.name]


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (for reduced test sizes)."""
    return dataclasses.replace(w, **kw)


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(e) for e in entropy]))


def _unit_norm(x: np.ndarray) -> np.ndarray:
    """Scale each last-axis vector to unit L2 norm (an input-distribution step)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


@dataclasses.dataclass
class UnitInputs:
    """Inputs of one (layer, request) unit, in the kernel layouts."""

    q: np.ndarray           # [T, Hk, d_k]
    k: np.ndarray           # [T, Hk, d_k]
    v: np.ndarray           # [T, Hv, d_v]
    a: np.ndarray           # [T, Hv]  decay gate in (0, 1)
    b: np.ndarray           # [T, Hv]  write strength in (0, 1)
    state: np.ndarray       # [Hv, d_v, d_k] float32
    x: np.ndarray           # [T, C] conv input
    conv_state: np.ndarray  # [W-1, C], oldest row first


def gen_unit(w: Workload, layer: int, req: int) -> UnitInputs:
    """Draw the GDN and conv inputs of one (layer, request) unit.

    q, k ~ N(0,1) scaled to unit norm per head; v ~ N(0,1);
    a = exp(-softplus(z)) = 1 / (1 + e^z), b = sigmoid(z'), z, z' ~ N(0,1);
    initial state ~ N(0, 0.02^2) in float32; conv x ~ N(0,1) and conv
    state ~ N(0,1). All values are rounded to the workload dtype (the
    state stays float32).
    """
    T, Hk, Hv, dk, dv, C = w.n_pos, w.n_kheads, w.n_vheads, w.d_k, w.d_v, w.conv_channels
    rng = _rng(w.seed, layer, req)
    q = _unit_norm(rng.standard_normal((T, Hk, dk)))
    k = _unit_norm(rng.standard_normal((T, Hk, dk)))
    v = rng.standard_normal((T, Hv, dv))
    za = rng.standard_normal((T, Hv))
    zb = rng.standard_normal((T, Hv))
    a = 1.0 / (1.0 + np.exp(za))
    b = _sigmoid(zb)
    state = (rng.standard_normal((Hv, dv, dk), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    x = rng.standard_normal((T, C), dtype=np.float32)
    cs = rng.standard_normal((w.conv_width - 1, C), dtype=np.float32)
    d = w.dtype
    return UnitInputs(
        q=cast(q.astype(np.float32), d), k=cast(k.astype(np.float32), d),
        v=cast(v.astype(np.float32), d), a=cast(a.astype(np.float32), d),
        b=cast(b.astype(np.float32), d), state=state,
        x=cast(x, d), conv_state=cast(cs, d))


def gen_conv_weight(w: Workload, layer: int) -> np.ndarray:
    """Depthwise conv weights [C, W] ~ N(0,1)*0.5, one set per layer."""
    rng = _rng(w.seed, layer, _TAG_CONV_W)
    wt = rng.standard_normal((w.conv_channels, w.conv_width), dtype=np.float32) * np.float32(0.5)
    return cast(wt.astype(np.float32), w.dtype)


def chain_parent(n_pos: int) -> np.ndarray:
    """Parent array of a root-inclusive chain: node t's parent is t-1."""
    return np.arange(-1, n_pos - 1, dtype=np.int32)


def gen_tree_parent(w: Workload, req: int) -> np.ndarray:
    """Random draft tree: node 0 is the root; node i (1..T-1) picks its parent
    uniformly among earlier nodes whose depth is below ``tree_max_depth`` and
    that have fewer than ``tree_max_children`` children."""
    if not w.tree:
        return chain_parent(w.n_pos)
    rng = _rng(w.seed, _TAG_TREE, req)
    parent = np.full(w.n_pos, -1, dtype=np.int32)
    depth = np.zeros(w.n_pos, dtype=np.int64)
    nchild = np.zeros(w.n_pos, dtype=np.int64)
    for i in range(1, w.n_pos):
        ok = [j for j in range(i)
              if depth[j] < w.tree_max_depth and nchild[j] < w.tree_max_children]
        p = ok[int(rng.integers(len(ok)))]
        parent[i] = p
        depth[i] = depth[p] + 1
        nchild[p] += 1
    return parent


@dataclasses.dataclass
class AcceptInputs:
    """Per-request draft tokens, planted argmax indices and (optionally) logits."""

    parent: np.ndarray        # [T] int32
    tokens: np.ndarray        # [T] int32 (tokens[0] is the committed root token)
    planted_argmax: np.ndarray  # [T] int32, the index planted as each row's unique max
    planted_node: int         # the node the plant was built to be accepted
    logits: Optional[np.ndarray]  # [T, V] in the workload dtype, or None


def _path_to(parent: np.ndarray, u: int) -> List[int]:
    out = []
    while u >= 0:
        out.append(u)
        u = int(parent[u])
    return out[::-1]


def gen_accept(w: Workload, req: int, with_logits: bool = True) -> AcceptInputs:
    """Plant a target node and build draft tokens and logits around it.

    Chain: the planted accepted count j ~ U{0..K}; drafts 1..j copy the
    planted argmax of their predecessor and draft j+1 (if any) differs.
    Tree: the planted node is uniform over all nodes; on the root path to it
    each child's token equals its parent's planted argmax; at the planted node
    and at every node off that path the planted argmax equals no child's
    token. Sibling tokens are distinct.

    Logits rows are N(0,1)*2 with the planted index raised to a unique
    maximum (2*max|row| + 1). For rows that must have all-distinct values
    (f32 tiny workload) the row is a shuffled set of distinct values whose
    largest value is moved to the planted index.
    """
    T, V = w.n_pos, max(w.vocab, 2)
    parent = gen_tree_parent(w, req)
    rng = _rng(w.seed, _TAG_ACCEPT, req)
    if w.tree:
        target = int(rng.integers(T))
    else:
        target = int(rng.integers(T))  # j ~ U{0..K}; the accepted node is j
    on_path = _path_to(parent, target)
    next_on_path = {on_path[i]: on_path[i + 1] for i in range(len(on_path) - 1)}
    children: List[List[int]] = [[] for _ in range(T)]
    for i in range(1, T):
        children[int(parent[i])].append(i)

    tokens = np.zeros(T, dtype=np.int32)
    tokens[0] = int(rng.integers(V))
    argmax = np.zeros(T, dtype=np.int32)
    # Visit nodes in index order (parents first) choosing tokens, then argmax.
    for n in range(T):
        kids = children[n]
        if kids:
            toks = rng.choice(V, size=len(kids), replace=False)
            for c, tk in zip(kids, toks):
                tokens[c] = int(tk)
        if n in next_on_path:
            argmax[n] = tokens[next_on_path[n]]
        else:
            taken = {int(tokens[c]) for c in kids}
            while True:
                cand = int(rng.integers(V))
                if cand not in taken:
                    break
            argmax[n] = cand

    logits = None
    if with_logits and w.vocab > 0:
        lr = _rng(w.seed, _TAG_LOGITS, req)
        if w.logits_distinct:
            rows = np.empty((T, w.vocab), dtype=np.float32)
            for t in range(T):
                while True:
                    vals = (lr.standard_normal(w.vocab) * 2.0).astype(np.float32)
                    if np.unique(vals).size == w.vocab:
                        break
                top = int(np.argmax(vals))
                vals[[top, argmax[t]]] = vals[[argmax[t], top]]
                rows[t] = vals
        else:
            rows = (lr.standard_normal((T, w.vocab), dtype=np.float32) * np.float32(2.0))
            big = 2.0 * np.max(np.abs(rows), axis=1) + 1.0
            rows[np.arange(T), argmax] = big.astype(np.float32)
        logits = cast(rows, w.dtype)
    return AcceptInputs(parent=parent, tokens=tokens, planted_argmax=argmax,
                        planted_node=target, logits=logits)


@dataclasses.dataclass
class RingInputs:
    ring: np.ndarray        # [n_rings, S, D] bf16 bits (initial contents)
    packed: np.ndarray      # [n_rings * T, D] bf16 bits (rows to write)
    runs: List[tuple]       # (ring_id, start_pos, n_rows, packed_row)


def gen_ring(w: Workload, with_ring: bool = True) -> RingInputs:
    """Feature ring of ``n_req`` rings x ``ring_slots`` slots x ``ring_width``.

    Request r writes its T rows at slots (p_r + i) mod S; even r start in
    the last 16 slots (so the run wraps), odd r anywhere a run fits.
    """
    S, D, R, T = w.ring_slots, w.ring_width, w.n_req, w.n_pos
    rng = _rng(w.seed, _TAG_RING, 0)
    runs = []
    for r in range(R):
        if r % 2 == 0:
            p = int(rng.integers(S - 16, S))
        else:
            p = int(rng.integers(0, S - T + 1))
        runs.append((r, p, T, r * T))
    packed = bf16_bits(rng.standard_normal((R * T, D), dtype=np.float32))
    ring = None
    if with_ring:
        ring = bf16_bits(rng.standard_normal((R, S, D), dtype=np.float32))
    return RingInputs(ring=ring, packed=packed, runs=runs)
