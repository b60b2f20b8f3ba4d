"""Pins of the tree-attention oracle against what the definition fixes: textbook causal
attention on a chain, brute force, invariances and closed forms, and commit consistency."""

import numpy as np
import pytest
from scipy.special import softmax

from linear_attention_speculative_head_amd import inputs
from oracle import attention as att


def problem(seed, B=2, Hkv=2, G=3, N=6, T=24, ctx=(10, 0), tree=(3, 2), d=8):
    return inputs.make_attention_problem(seed, B=B, Hkv=Hkv, G=G, N=N, T_max=T,
                                         ctx=np.array(ctx[:B]), tree=tree, d=d)


def test_chain_is_causal_attention_over_the_appended_sequence():
    """A chain's verify is ordinary causal attention over [cache; drafts] (textbook form:
    one masked score matrix, a library softmax, one product)."""
    P = problem(1, tree="chain")
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    for b in range(P.B):
        c = int(P.ctx[b])
        for hq in range(P.Hq):
            kv = hq // P.G
            K = np.concatenate([P.Kc[b, kv, :c], P.Kd[b, :, kv]]).astype(np.float64)
            V = np.concatenate([P.Vc[b, kv, :c], P.Vd[b, :, kv]]).astype(np.float64)
            Qm = P.Qd[b, :, hq].astype(np.float64)
            S = Qm @ K.T / np.sqrt(P.d)
            mask = np.arange(c + P.N)[None, :] <= (c + np.arange(P.N))[:, None]
            S = np.where(mask, S, -np.inf)
            ref = softmax(S, axis=1) @ V
            np.testing.assert_allclose(O[b, :, hq], ref, rtol=1e-12, atol=1e-12)


def test_brute_force_loops():
    P = problem(2, B=1, Hkv=1, G=2, N=5, T=9, ctx=(4,), d=4)
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    for t in range(P.N):
        vis = []
        i = t
        while i >= 0:
            vis.append(i)
            i = int(P.parent[0, i])
        for hq in range(P.Hq):
            q = [float(x) for x in P.Qd[0, t, hq]]
            keys = [P.Kc[0, 0, j] for j in range(int(P.ctx[0]))] + [P.Kd[0, i, 0] for i in vis]
            vals = [P.Vc[0, 0, j] for j in range(int(P.ctx[0]))] + [P.Vd[0, i, 0] for i in vis]
            sc = [sum(q[e] * float(k[e]) for e in range(P.d)) / (P.d ** 0.5) for k in keys]
            w = [np.exp(x - max(sc)) for x in sc]
            ref = [sum(w[j] * float(vals[j][e]) for j in range(len(w))) / sum(w) for e in range(P.d)]
            np.testing.assert_allclose(O[0, t, hq], ref, rtol=1e-12, atol=1e-13)


def test_shifting_every_key_changes_nothing():
    """Adding one vector to every key adds the same amount to all of a query's scores."""
    P = problem(3)
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    w = np.random.default_rng(0).standard_normal(P.d)
    O2 = att.tree_attention(P.Kc + w, P.Vc, P.ctx, P.Qd, P.Kd + w, P.Vd, P.parent, P.G)
    np.testing.assert_allclose(O2, O, rtol=1e-10, atol=1e-12)


def test_zero_query_averages_visible_values():
    P = problem(4)
    Qz = np.zeros_like(P.Qd)
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, Qz, P.Kd, P.Vd, P.parent, P.G)
    anc = [att.ancestors(P.parent[b]) for b in range(P.B)]
    for b in range(P.B):
        c = int(P.ctx[b])
        for t in range(P.N):
            for hq in range(P.Hq):
                kv = hq // P.G
                vals = np.concatenate([P.Vc[b, kv, :c], P.Vd[b, anc[b][t], kv]]).astype(np.float64)
                np.testing.assert_allclose(O[b, t, hq], vals.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_a_root_with_an_empty_cache_returns_its_own_value():
    P = problem(5, ctx=(0, 0))
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    for b in range(P.B):
        for t in range(P.N):
            if P.parent[b, t] == -1:
                for hq in range(P.Hq):
                    assert np.array_equal(O[b, t, hq], P.Vd[b, t, hq // P.G].astype(np.float64))


def test_non_ancestors_do_not_matter():
    P = problem(6, tree=(3, 3))
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    anc = att.ancestors(P.parent[0])
    t = P.N - 1
    others = [i for i in range(P.N) if i not in anc[t]]
    assert others
    Kd, Vd = P.Kd.copy(), P.Vd.copy()
    Kd[0, others] += 3.0
    Vd[0, others] -= 2.0
    O2 = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, Kd, Vd, P.parent, P.G)
    assert np.array_equal(O2[0, t], O[0, t])


def test_relabeling_permutes_outputs():
    """The same tree numbered breadth-first instead of depth-first gives permuted outputs."""
    par = inputs.full_tree((2, 2))                # DFS: 0 1 2 3 4 5
    bfs = [0, 3, 1, 2, 4, 5]                      # new index of each DFS node
    new_par = np.empty_like(par)
    for n in range(len(par)):
        new_par[bfs[n]] = -1 if par[n] < 0 else bfs[par[n]]
    P = inputs.make_attention_problem(7, B=1, Hkv=1, G=2, N=6, T_max=16, ctx=np.array([9]),
                                      parent=par[None], d=8)
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    Qb, Kb, Vb = (np.empty_like(x) for x in (P.Qd, P.Kd, P.Vd))
    for n in range(6):
        Qb[0, bfs[n]], Kb[0, bfs[n]], Vb[0, bfs[n]] = P.Qd[0, n], P.Kd[0, n], P.Vd[0, n]
    O2 = att.tree_attention(P.Kc, P.Vc, P.ctx, Qb, Kb, Vb, new_par[None], P.G)
    np.testing.assert_allclose(O2[0, bfs], O[0], rtol=1e-12, atol=1e-13)


def test_query_heads_read_their_own_kv_head():
    P = problem(8, Hkv=2, G=3)
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    Kc, Kd = P.Kc.copy(), P.Kd.copy()
    Kc[:, 1] += 1.5
    Kd[:, :, 1] -= 0.5
    O2 = att.tree_attention(Kc, P.Vc, P.ctx, P.Qd, Kd, P.Vd, P.parent, P.G)
    assert np.array_equal(O2[:, :, :P.G], O[:, :, :P.G])       # heads of KV head 0
    assert not np.allclose(O2[:, :, P.G:], O[:, :, P.G:])


def test_commit_appends_the_accepted_path():
    P = problem(9, tree=(3, 2))
    acc = np.array([P.N - 1, -1])
    Kc, Vc, ctx = att.kv_commit(P.Kc, P.Vc, P.ctx, P.Kd, P.Vd, P.parent, acc)
    path = att.ancestors(P.parent[0])[P.N - 1]
    c = int(P.ctx[0])
    assert ctx[0] == c + len(path) and ctx[1] == P.ctx[1]
    for i, n in enumerate(path):
        assert np.array_equal(Kc[0, :, c + i], P.Kd[0, n])
        assert np.array_equal(Vc[0, :, c + i], P.Vd[0, n])
    assert np.array_equal(Kc[1], P.Kc[1]) and np.array_equal(Kc[0, :, :c], P.Kc[0, :, :c])


def test_verify_equals_attention_after_committing_the_parents_path():
    """Node t's output equals a root's output over the cache into which the path of t's
    parent was committed: the mask and the commit agree on what t sees."""
    P = problem(10, tree=(3, 3), ctx=(5, 3))
    O = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    for b in range(P.B):
        for t in range(P.N):
            p = int(P.parent[b, t])
            acc = np.full(P.B, -1)
            acc[b] = p
            Kc, Vc, ctx = att.kv_commit(P.Kc, P.Vc, P.ctx, P.Kd, P.Vd, P.parent, acc)
            one = lambda x: x[:, t:t + 1]
            O1 = att.tree_attention(Kc, Vc, ctx, one(P.Qd), one(P.Kd), one(P.Vd),
                                    np.full((P.B, 1), -1), P.G)
            np.testing.assert_allclose(O1[b, 0], O[b, t], rtol=1e-12, atol=1e-13)
