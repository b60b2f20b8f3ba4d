"""CPU oracle for the tree-aware softmax-attention verify -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module.  The product path never routes through it.

The definition, in float64 numpy: a softmax-attention layer attends query q_t to its keys
and values with softmax(q_t K^T / sqrt(d)) V (the technical review "TreeWY: Removing the
Memory Wall in Speculative Decoding for Gated DeltaNet Hybrids", §2.3 "KV cache attention",
Eq. (2)).  During a tree verify the draft tokens' keys and values are appended after the
committed cache, and draft node t sees the committed prefix plus its own ancestors-or-self
among the draft nodes (tree-structured drafting, §2.2 of the same page; the same ancestor
sets as the GDN path).  Query head hq reads key/value head hq // G (G query heads per
key/value head).  Committing an accepted node appends its root-to-node path's keys and
values to the cache; rejected branches are simply not kept.

Pinned by ``tests/test_oracle_attention.py``.
"""

from __future__ import annotations

import numpy as np


def ancestors(parent_b: np.ndarray):
    """For each node the list of its ancestors-or-self, root first, by walking parents."""
    out = []
    for t in range(len(parent_b)):
        path = []
        i = t
        while i >= 0:
            path.append(i)
            i = int(parent_b[i])
        out.append(path[::-1])
    return out


def tree_attention(Kc, Vc, ctx, Qd, Kd, Vd, parent, G: int):
    """Kc, Vc [B, Hkv, T, d]; ctx [B]; Qd [B, N, Hq, d]; Kd, Vd [B, N, Hkv, d]; parent [B, N].

    Returns O [B, N, Hq, d] in float64."""
    Kc, Vc, Qd, Kd, Vd = (np.asarray(x, dtype=np.float64) for x in (Kc, Vc, Qd, Kd, Vd))
    B, N, Hq, d = Qd.shape
    O = np.zeros((B, N, Hq, d))
    for b in range(B):
        anc = ancestors(parent[b])
        c = int(ctx[b])
        for t in range(N):
            vis = anc[t]
            for hq in range(Hq):
                kv = hq // G
                keys = np.concatenate([Kc[b, kv, :c], Kd[b, vis, kv]], axis=0)
                vals = np.concatenate([Vc[b, kv, :c], Vd[b, vis, kv]], axis=0)
                s = keys @ Qd[b, t, hq] / np.sqrt(d)
                s = s - s.max()
                p = np.exp(s)
                O[b, t, hq] = (p @ vals) / p.sum()
    return O


def kv_commit(Kc, Vc, ctx, Kd, Vd, parent, accepted):
    """Append the accepted node's root-to-node path (keys and values of every KV head) after
    each sequence's committed prefix.  Returns new (Kc, Vc, ctx); accepted = -1 keeps all."""
    Kc, Vc = np.array(Kc, copy=True), np.array(Vc, copy=True)
    ctx = np.array(ctx, copy=True)
    for b in range(Kc.shape[0]):
        a = int(accepted[b])
        if a < 0:
            continue
        path = ancestors(parent[b])[a]
        c = int(ctx[b])
        for i, n in enumerate(path):
            Kc[b, :, c + i] = Kd[b, n]
            Vc[b, :, c + i] = Vd[b, n]
        ctx[b] = c + len(path)
    return Kc, Vc, ctx
