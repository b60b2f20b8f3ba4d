"""Algorithmic byte counts for the verify/commit path (host-side bookkeeping only).

"Algorithmic" bytes are what the method itself must move through HBM, each tensor
once: the committed state read once per head by verify, every per-node input read once
and every output written once, and the commit's read-modify-write of the accepted
head's state plus the path rows it folds in.  Re-reads that a kernel happens to make
through L2 are not counted.  These are the figures the roofline fraction divides by.

Memory arithmetic of the TreeWY paper (arXiv 2608.20961, §2 "The memory problem" and
§3 "Reconstruct on commit") is reproduced by ``gdn_state_bytes`` and friends and pinned
by ``tests/golden/memory_arithmetic.json``.
"""

from __future__ import annotations

import numpy as np

from .inputs import tree_depths

D = 128


def gdn_state_bytes(layers: int, heads: int, dv: int = D, dk: int = D, elem: int = 2) -> int:
    """Recurrent state held per sequence by the GDN layers: layers x heads x dv x dk."""
    return layers * heads * dv * dk * elem


def kv_bytes_per_token(softmax_layers: int, kv_heads: int, head_dim: int, elem: int = 2) -> int:
    """Softmax KV cache per token: K and V for every softmax layer and KV head."""
    return 2 * softmax_layers * kv_heads * head_dim * elem


def storeall_blocks(n_nodes: int) -> int:
    """Full-state snapshotting keeps the committed state plus one state per draft node."""
    return n_nodes + 1


def verify_bytes_per_head(N: int, elem: int, d: int = D) -> int:
    """S0 read + per node (q, k, v rows, alpha, beta read; O, U rows and gamma written)."""
    return 4 * d * d + N * (3 * d * elem + 8 + 2 * 4 * d + 4)


def commit_bytes_per_head(depth_a: int, elem: int, d: int = D) -> int:
    """Accepted head: S read + written, and depth(a) path rows of U (fp32), K and gamma."""
    if depth_a <= 0:
        return 0
    return 2 * 4 * d * d + depth_a * (4 * d + elem * d + 4)


def snapshot_verify_bytes_per_head(N: int, elem: int, d: int = D) -> int:
    """S0 read + per node (q, k, v, alpha, beta read; O row and a full fp32 state written)."""
    return 4 * d * d + N * (3 * d * elem + 8 + 4 * d + 4 * d * d)


def snapshot_commit_bytes_per_head(accepted: int, d: int = D) -> int:
    """Accepted head: copy its snapshot over S (read + write); nothing when a = -1."""
    return 0 if accepted < 0 else 2 * 4 * d * d


def step_bytes(parent: np.ndarray, accepted: np.ndarray, H: int, N: int, elem: int,
               layers: int = 1) -> dict:
    """Algorithmic bytes of one verify+commit pass over all layers, from the actual draws."""
    B = parent.shape[0]
    v = layers * (B * H * verify_bytes_per_head(N, elem) + B * 4 * N)
    c = 0
    for b in range(B):
        a = int(accepted[b])
        c += 4
        if a >= 0:
            da = int(tree_depths(parent[b])[a])
            c += 4 * N + H * commit_bytes_per_head(da, elem)
    c *= layers
    return dict(verify=v, commit=c, total=v + c)


def fused_step_bytes(parent_prev: np.ndarray, accepted_prev: np.ndarray, parent: np.ndarray,
                     H: int, elem: int, layers: int = 1) -> dict:
    """One fused pass (the previous step's commit folded into this step's verify), over all
    layers: per head the state read once, written back when the previous step accepted a
    node, the path rows of that node, and this step's per-node I/O; per sequence both trees
    and the accepted node."""
    B, Np = parent_prev.shape
    N = parent.shape[1]
    t = B * H * verify_bytes_per_head(N, elem) + B * 4 * (N + Np + 1)
    for b in range(B):
        a = int(accepted_prev[b])
        if a >= 0:
            da = int(tree_depths(parent_prev[b])[a])
            t += H * (4 * D * D + da * (4 * D + elem * D + 4))
    return dict(fused=layers * t, total=layers * t)


def deferred_step_bytes(parent_prev: np.ndarray, accepted_prev: np.ndarray, parent: np.ndarray,
                        H: int, elem: int, lens: np.ndarray, Lmax: int) -> tuple:
    """One step of the deferred commit over one layer, from the log lengths before it.

    Per head: the state read (once, inside the verify's count); the logged terms read (a u~
    row in fp32 and a key row each); the accepted path's rows (U, key, gamma); this step's
    per-node I/O; then either the
    path's terms appended to the log or, when they do not fit, the committed state written
    back.  They fit when len + depth <= Lmax and, up to 16 nodes, the path is no longer than
    one staged chunk (4 rows for N <= 4, else 8); above 16 nodes the log's and the path's
    terms must fit one staged chunk together (16 terms up to 48 nodes, 8 above).  Per
    sequence both trees, the accepted node and the log length.  Returns (bytes, lengths
    after the step)."""
    B, Np = parent_prev.shape
    N = parent.shape[1]
    stage = 4 if N <= 4 else 8
    keep = Lmax if N <= 48 else min(Lmax, 8)
    row = 4 * D + elem * D
    t = B * H * verify_bytes_per_head(N, elem) + B * 4 * (N + Np + 2) + B * H * 8
    after = np.array(lens, dtype=np.int64)
    for b in range(B):
        ln = int(lens[b])
        t += H * ln * row
        a = int(accepted_prev[b])
        if a < 0:
            continue
        da = int(tree_depths(parent_prev[b])[a])
        t += H * da * (row + 4)
        if ln + da > keep or (N <= 16 and da > stage):
            t += H * 4 * D * D
            after[b] = 0
        else:
            t += H * da * row
            after[b] = ln + da
    return t, after


def snapshot_step_bytes(parent: np.ndarray, accepted: np.ndarray, H: int, N: int, elem: int,
                        layers: int = 1) -> dict:
    B = parent.shape[0]
    v = layers * (B * H * snapshot_verify_bytes_per_head(N, elem) + B * 4 * N)
    c = layers * sum(4 + H * snapshot_commit_bytes_per_head(int(a)) for a in accepted)
    return dict(verify=v, commit=c, total=v + c)


def attention_call_bytes(ctx, N: int, Hkv: int, G: int, d: int = 256, elem: int = 2) -> int:
    """One tree-attention verify over a batch: each sequence's committed key and value rows
    read once (every key/value head), the draft's queries (Hkv G heads), keys and values
    (Hkv heads) read, and O (fp32, Hkv G heads) written.  The split partials are the
    kernel's own traffic, not the method's."""
    ctx = np.asarray(ctx, dtype=np.int64)
    B = ctx.shape[0]
    return int(ctx.sum() * Hkv * d * elem * 2 + B * N * (Hkv * G + 2 * Hkv) * d * elem
               + B * N * Hkv * G * d * 4)
