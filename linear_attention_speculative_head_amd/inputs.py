"""Seeded synthetic inputs for the TreeWY verify/commit path.

This module only draws numbers and builds draft-tree topologies; it holds none of
the method's arithmetic, and both the GPU path and the CPU oracle are fed from it.

Shapes follow the Gated DeltaNet layers of the Qwen3.5 hybrids the TreeWY paper
evaluates (arXiv 2608.20961, §2 "The memory problem": dk = dv = 128, 32 value heads
per GDN layer at 35B-A3B, 64 at 397B-A17B, 30 GDN layers at 35B-A3B).

Layouts (all C-contiguous):
    S0     [B, H, dv, dk]  float32   committed state, row v contiguous over dk
    q, k   [B, N, H, dk]   float32   token-major; values are bf16-exact when dtype == "bf16"
    v      [B, N, H, dv]   float32   (same)
    alpha  [B, N, H]       float32   decay gate in (0, 1)
    beta   [B, N, H]       float32   write strength in (0, 1)
    parent [B, N]          int32     -1 = child of the committed state S0, else a smaller index
    accepted [B]           int32     accepted node, -1 = nothing accepted

Value laws: S0 ~ N(0, 0.05^2); q, k ~ N(0, 1) then L2-normalised per vector; v ~ N(0, 1);
alpha ~ U(0.90, 0.999); beta = sigmoid(N(0, 1)).  For dtype "bf16", q, k and v are
rounded to bfloat16 (round-to-nearest-even) after normalisation, so both sides see the
same bf16 values.
"""

from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

D = 128  # dk = dv on every GDN layer of the modelled family

# name -> shape description; the random-tree tuple is (max_depth, max_branching)
CONFIGS = {
    0: dict(B=1, H=1, N=4, layers=1, dtype="f32", tree="chain", accept="uniform",
            desc="B1 x H1, chain N=4, fp32 q/k/v"),
    1: dict(B=32, H=32, N=4, layers=1, dtype="bf16", tree="chain", accept="prefix",
            desc="B32 x H32, chain N=4, bf16 q/k/v, accepted prefix ~U{0..4}"),
    2: dict(B=64, H=32, N=16, layers=1, dtype="bf16", tree=(5, 4), accept="uniform",
            desc="B64 x H32, random tree N=16 (depth<=5, branching<=4), bf16 q/k/v"),
    3: dict(B=128, H=32, N=64, layers=30, dtype="bf16", tree=(6, 8), accept="uniform",
            desc="B128 x H32, random tree N=64 (depth<=6, branching<=8), 30 layers, bf16 q/k/v"),
    4: dict(B=256, H=64, N=32, layers=1, dtype="bf16", tree=(6, 4), accept="skew34",
            desc="B256 x H64, random tree N=32 (depth<=6, branching<=4), accepted skewed to depth 3-4"),
}


# ----------------------------------------------------------------------------- trees

def chain_tree(n: int) -> np.ndarray:
    """A chain of n draft tokens: node i hangs off node i-1, node 0 off S0."""
    return np.arange(-1, n - 1, dtype=np.int32)


def full_tree(widths: Sequence[int]) -> np.ndarray:
    """Complete tree with per-level branching (w1, w2, ...), laid out in DFS pre-order.

    The committed state has w1 children, each of those w2, and so on (the
    ``draft_tree_widths`` shape of the paper's §4 and Table 2).
    """
    parent: List[int] = []

    def grow(p: int, level: int) -> None:
        if level == len(widths):
            return
        for _ in range(widths[level]):
            me = len(parent)
            parent.append(p)
            grow(me, level + 1)

    grow(-1, 0)
    return np.asarray(parent, dtype=np.int32)


def random_tree(rng: np.random.Generator, n: int, max_depth: int, max_branch: int) -> np.ndarray:
    """Random draft tree of n nodes in DFS pre-order.

    Node 0 hangs off S0.  Node t >= 1 attaches uniformly to one of the open slots on
    the current root-to-(t-1) path (S0 itself included): a slot is open when its
    node has fewer than ``max_branch`` children and depth below ``max_depth``.  The
    path is then cut back to the chosen node, which keeps the order a DFS pre-order.
    If no slot is open the whole tree is drawn again from the same generator (at most
    1000 times; a shape that cannot hold n nodes raises ValueError).
    """
    cap = sum(max_branch ** d for d in range(1, max_depth + 1))
    if n < 1 or n > cap:
        raise ValueError(f"a tree of depth <= {max_depth}, branching <= {max_branch} "
                         f"holds at most {cap} nodes, not {n}")
    for _attempt in range(1000):
        parent = np.empty(n, dtype=np.int32)
        nchild = np.zeros(n + 1, dtype=np.int64)  # index 0 counts S0's children
        depth = np.zeros(n, dtype=np.int64)
        parent[0] = -1
        nchild[0] = 1
        depth[0] = 1
        path = [-1, 0]  # S0 then node 0
        ok = True
        for t in range(1, n):
            cands = [p for p in path
                     if nchild[p + 1] < max_branch and (p < 0 or depth[p] < max_depth)]
            if not cands:
                ok = False
                break
            p = cands[int(rng.integers(len(cands)))]
            parent[t] = p
            nchild[p + 1] += 1
            depth[t] = 1 if p < 0 else depth[p] + 1
            path = path[: path.index(p) + 1] + [t]
        if ok:
            return parent
    raise ValueError(f"could not draw a tree of {n} nodes (depth <= {max_depth}, "
                     f"branching <= {max_branch})")


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """depth(t) = 1 + depth(parent(t)); a child of S0 has depth 1."""
    d = np.zeros(len(parent), dtype=np.int32)
    for t, p in enumerate(parent):
        d[t] = 1 if p < 0 else d[p] + 1
    return d


# ----------------------------------------------------------------------------- values

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return x


@dataclass
class Layer:
    S0: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray


@dataclass
class Problem:
    """One verify+commit workload: a batch of draft trees and one or more GDN layers."""
    cfg: int
    B: int
    H: int
    N: int
    dtype: str                 # "f32" or "bf16": the element type of q, k, v on the device
    parent: np.ndarray         # [B, N] int32
    accepted: np.ndarray       # [B] int32
    layers: List[Layer] = field(default_factory=list)
    dk: int = D
    dv: int = D


def draw_layer(rng: np.random.Generator, B: int, H: int, N: int, dtype: str,
               dk: int = D, dv: int = D) -> Layer:
    S0 = (np.float32(0.05) * rng.standard_normal((B, H, dv, dk), dtype=np.float32))
    q = _unit_rows(rng, (B, N, H, dk))
    k = _unit_rows(rng, (B, N, H, dk))
    v = rng.standard_normal((B, N, H, dv), dtype=np.float32)
    alpha = (np.float32(0.90) + np.float32(0.099) * rng.random((B, N, H), dtype=np.float32))
    alpha = np.minimum(alpha, np.float32(0.999))
    z = rng.standard_normal((B, N, H), dtype=np.float32)
    beta = (np.float32(1.0) / (np.float32(1.0) + np.exp(-z))).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return Layer(S0=S0, q=q, k=k, v=v, alpha=alpha, beta=beta)


def draw_trees(rng: np.random.Generator, B: int, N: int, tree, accept: str):
    parent = np.empty((B, N), dtype=np.int32)
    accepted = np.empty(B, dtype=np.int32)
    for b in range(B):
        if tree == "chain":
            par = chain_tree(N)
        else:
            max_depth, max_branch = tree
            par = random_tree(rng, N, max_depth, max_branch)
        parent[b] = par
        if accept == "uniform":
            a = int(rng.integers(N))
        elif accept == "prefix":      # accepted prefix length L ~ U{0..N}; a = L - 1
            a = int(rng.integers(N + 1)) - 1
        elif accept == "skew34":      # 80%: uniform over depth-3/4 nodes when there are any
            d = tree_depths(par)
            mid = np.flatnonzero((d == 3) | (d == 4))
            if len(mid) and rng.random() < 0.8:
                a = int(mid[rng.integers(len(mid))])
            else:
                a = int(rng.integers(N))
        else:
            raise ValueError(accept)
        accepted[b] = a
    return parent, accepted


def make_problem(cfg: int, instance: int = 0, layers: Optional[int] = None,
                 B: Optional[int] = None) -> Problem:
    """Draw configuration ``cfg`` (0..4).  ``instance`` selects an independent draw.

    ``layers`` limits how many of the configuration's layers are drawn (each layer has
    its own spawned seed, so layer l is the same whatever the limit); ``B`` keeps only
    the first B sequences' trees (the per-layer tensors are then drawn at that B).
    """
    c = CONFIGS[cfg]
    nl = c["layers"] if layers is None else min(layers, c["layers"])
    Bx = c["B"] if B is None else B
    seeds = np.random.SeedSequence([1000 + cfg, instance]).spawn(1 + c["layers"])
    tr = np.random.default_rng(seeds[0])
    parent, accepted = draw_trees(tr, c["B"], c["N"], c["tree"], c["accept"])
    parent, accepted = parent[:Bx].copy(), accepted[:Bx].copy()
    P = Problem(cfg=cfg, B=Bx, H=c["H"], N=c["N"], dtype=c["dtype"],
                parent=parent, accepted=accepted)
    draw = lambda l: draw_layer(np.random.default_rng(seeds[1 + l]), Bx, c["H"], c["N"], c["dtype"])
    if nl > 1:
        # every layer has a generator of its own, so drawing them on several threads (numpy
        # releases the interpreter lock while it fills arrays) gives the same numbers
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(nl, _host_threads())) as ex:
            P.layers.extend(ex.map(draw, range(nl)))
    else:
        P.layers.extend(draw(l) for l in range(nl))
    return P


def _host_threads() -> int:
    """Host threads for drawing: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# the full-tree shapes of the paper's Table 2 and of Table 4 in Appendix B (w1, w2, w3 per
# level, from a chain up to width 3 on every level)
PAPER_TREE_SHAPES = [(1, 1, 1), (2, 1, 1), (2, 2, 1), (2, 2, 2), (3, 2, 2), (3, 3, 2), (3, 3, 3)]


def make_tree_shape(widths: Sequence[int], instance: int = 0, B: int = 32, H: int = 32,
                    dtype: str = "bf16") -> Problem:
    """Every sequence drafts the same full tree (w1, w2, ...); the accepted node is uniform
    over its nodes.  One layer, the configuration-1 batch (B x H) by default."""
    par = full_tree(widths)
    N = len(par)
    key = [2000, instance] + [int(w) for w in widths]
    seeds = np.random.SeedSequence(key).spawn(2)
    tr = np.random.default_rng(seeds[0])
    parent = np.stack([par] * B).astype(np.int32)
    accepted = tr.integers(0, N, size=B).astype(np.int32)
    P = Problem(cfg=-1, B=B, H=H, N=N, dtype=dtype, parent=parent, accepted=accepted)
    P.layers.append(draw_layer(np.random.default_rng(seeds[1]), B, H, N, dtype))
    return P


# ----------------------------------------------------------------------------- softmax layers

# Softmax-attention layers of the modelled hybrids: head dimension 256, 2 key/value heads
# (paper §2).  The pages do not give the query-head count; 8 query heads per key/value head
# is this package's reading (grouped-query attention, query head hq reads key/value head
# hq // G).
ATTN_D = 256
ATTN_HKV = 2
ATTN_G = 8


@dataclass
class AttnProblem:
    """One tree-verify pass of a softmax-attention layer: the committed cache, the draft
    tokens' queries/keys/values and the tree.  Cache rows at or past a sequence's committed
    length hold a large constant, so that reading them would show."""
    B: int
    Hkv: int
    G: int
    N: int
    d: int
    T_max: int
    Kc: np.ndarray        # [B, Hkv, T_max, d] float32 (bf16-exact)
    Vc: np.ndarray
    ctx: np.ndarray       # [B] int32 committed length
    Qd: np.ndarray        # [B, N, Hq, d]
    Kd: np.ndarray        # [B, N, Hkv, d]
    Vd: np.ndarray
    parent: np.ndarray    # [B, N] int32
    accepted: np.ndarray  # [B] int32

    @property
    def Hq(self) -> int:
        return self.Hkv * self.G


def make_attention_problem(seed: int, B: int, Hkv: int = ATTN_HKV, G: int = ATTN_G, N: int = 4,
                           T_max: int = 256, ctx=None, tree="chain", d: int = ATTN_D,
                           parent: Optional[np.ndarray] = None,
                           accepted: Optional[np.ndarray] = None) -> AttnProblem:
    """Entries ~ N(0, 1) rounded to bf16 (scores q.k / sqrt(d) then have unit spread)."""
    rng = np.random.default_rng(np.random.SeedSequence([88, seed]))
    if parent is None:
        if tree == "chain":
            parent = np.stack([chain_tree(N)] * B)
        else:
            parent = np.stack([random_tree(rng, N, tree[0], tree[1]) for _ in range(B)])
    parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, N)
    if ctx is None:
        ctx = rng.integers(0, T_max - N + 1, size=B)
    ctx = np.ascontiguousarray(ctx, dtype=np.int32).reshape(B)
    assert (ctx >= 0).all() and (ctx + N <= T_max).all()
    if accepted is None:
        accepted = rng.integers(-1, N, size=B)
    accepted = np.ascontiguousarray(accepted, dtype=np.int32).reshape(B)
    Hq = Hkv * G
    f = lambda *s: round_bf16(rng.standard_normal(s, dtype=np.float32))
    Kc, Vc = f(B, Hkv, T_max, d), f(B, Hkv, T_max, d)
    for b in range(B):                   # rows past the committed prefix: a loud constant
        Kc[b, :, ctx[b]:] = 64.0
        Vc[b, :, ctx[b]:] = 4096.0
    return AttnProblem(B=B, Hkv=Hkv, G=G, N=N, d=d, T_max=T_max, Kc=Kc, Vc=Vc, ctx=ctx,
                       Qd=f(B, N, Hq, d), Kd=f(B, N, Hkv, d), Vd=f(B, N, Hkv, d),
                       parent=parent, accepted=accepted)


def make_custom(seed: int, B: int, H: int, N: int, dtype: str = "bf16",
                parent: Optional[np.ndarray] = None, tree=(6, 4),
                accepted: Optional[np.ndarray] = None, dk: int = D, dv: int = D) -> Problem:
    """A one-layer problem with explicit sizes, for edge cases and small parity runs."""
    rng = np.random.default_rng(np.random.SeedSequence([77, seed]))
    if parent is None:
        if tree == "chain":
            parent = np.stack([chain_tree(N)] * B)
        else:
            parent = np.stack([random_tree(rng, N, tree[0], tree[1]) for _ in range(B)])
    parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, N)
    if accepted is None:
        accepted = rng.integers(-1, N, size=B).astype(np.int32)
    accepted = np.ascontiguousarray(accepted, dtype=np.int32).reshape(B)
    P = Problem(cfg=-1, B=B, H=H, N=N, dtype=dtype, parent=parent, accepted=accepted, dk=dk, dv=dv)
    P.layers.append(draw_layer(rng, B, H, N, dtype, dk=dk, dv=dv))
    return P
