"""GPU parity of the tree-aware softmax-attention verify and its cache commit against the
oracle (float64 numpy, oracle/attention.py), through the C ABI.

Gate: per (sequence, query head), max|O - O_oracle| / max|O_oracle| over the head's draft
nodes <= 1e-3; the commit's cache rows and lengths bit-exact.  Cases: chains and trees up to
64 nodes, empty and ragged committed prefixes (several cache ranges and a ragged last 32-row
step), query blocks of 32 with a ragged tail, malformed trees, and cache rows past the prefix
that must not be read (they hold a loud constant).
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import TOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


def upload(P):
    import torch
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16).contiguous()
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    return dict(Kc=bf(P.Kc), Vc=bf(P.Vc), ctx=i32(P.ctx), Qd=bf(P.Qd), Kd=bf(P.Kd), Vd=bf(P.Vd),
                parent=i32(P.parent), accepted=i32(P.accepted))


def run_attention(P, status_check=True):
    import torch
    from linear_attention_speculative_head_amd import binding
    d = upload(P)
    O = torch.full((P.B, P.N, P.Hq, 256), float("nan"), device="cuda")
    ws = torch.empty(binding.treewy_tree_attention_workspace(P.B, P.Hkv, P.G, P.N, P.T_max),
                     dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.treewy_tree_attention(d["Kc"], d["Vc"], d["ctx"], d["Qd"], d["Kd"], d["Vd"],
                                  d["parent"], O, ws, status)
    torch.cuda.synchronize()
    if status_check:
        assert int(status.item()) == 0
    return O.cpu().numpy(), int(status.item())


def check(P, O, label):
    from oracle import attention as att
    ref = att.tree_attention(P.Kc, P.Vc, P.ctx, P.Qd, P.Kd, P.Vd, P.parent, P.G)
    assert np.all(np.isfinite(O)), f"{label}: non-finite outputs"
    worst = 0.0
    for b in range(P.B):
        for hq in range(P.Hq):
            e = np.abs(O[b, :, hq] - ref[b, :, hq]).max() / np.abs(ref[b, :, hq]).max()
            worst = max(worst, e)
            assert e <= TOL, f"{label}: b={b} hq={hq} rel err {e:.3e}"
    say(f"  {label}: worst head-wise rel err {worst:.2e}")


@pytest.mark.parametrize("B,G,N,tree,T,ctx,seed", [
    (3, 8, 4, "chain", 1200, (1100, 0, 513), 1),       # splits, an empty prefix, ragged tails
    (2, 8, 16, (5, 4), 700, (600, 37), 2),             # 128 queries: four blocks
    (2, 3, 7, (3, 3), 200, (31, 190), 3),              # a ragged block of 21 queries
    (2, 8, 64, "chain", 600, (500, 1), 4),             # 64-node chain: 512 queries
    (2, 8, 33, (6, 4), 2100, (2050, 1024), 5),         # five splits
])
def test_tree_attention(B, G, N, tree, T, ctx, seed):
    say(f"[attention] B={B} G={G} N={N} tree={tree} T={T} ctx={ctx}")
    P = inputs.make_attention_problem(seed, B=B, Hkv=2, G=G, N=N, T_max=T, ctx=np.array(ctx),
                                      tree=tree)
    O, _ = run_attention(P)
    check(P, O, f"N={N} G={G}")


def test_configuration_one_shape():
    """The benchmark's shape (B=32, 2 KV heads x 8 query heads, depth-3 chain + root) at a
    shorter prefix, every head compared."""
    P = inputs.make_attention_problem(11, B=32, N=4, T_max=1040, ctx=np.full(32, 1024))
    O, _ = run_attention(P)
    check(P, O, "B32 chain-4")


def test_benchmark_shape_full_prefix():
    """The benchmark's launch at 8192 committed rows (B=32, 2 KV heads x 8 query heads, chain
    of 4: ten cache ranges per (sequence, KV head), the last one ragged), three sequences
    compared with the oracle (which is run on those alone)."""
    say("[attention] B=32 chain-4 at 8192 committed rows, sequences 0, 13, 31")
    P = inputs.make_attention_problem(12, B=32, N=4, T_max=8200, ctx=np.full(32, 8192))
    O, _ = run_attention(P)
    from oracle import attention as att
    sel = np.array([0, 13, 31])
    ref = att.tree_attention(P.Kc[sel], P.Vc[sel], P.ctx[sel], P.Qd[sel], P.Kd[sel], P.Vd[sel],
                             P.parent[sel], P.G)
    assert np.all(np.isfinite(O[sel])), "non-finite outputs"
    worst = 0.0
    for i, b in enumerate(sel):
        for hq in range(P.Hq):
            e = np.abs(O[b, :, hq] - ref[i, :, hq]).max() / np.abs(ref[i, :, hq]).max()
            worst = max(worst, e)
            assert e <= TOL, f"b={b} hq={hq} rel err {e:.3e}"
    say(f"  worst head-wise rel err {worst:.2e}")


@pytest.mark.parametrize("N,node,bad", [(5, 3, 4), (40, 35, 39), (40, 2, -5)])
def test_malformed_tree_is_reported(N, node, bad):
    """A parent outside [-1, t-1] is reported; the node then counts as a root of the draft
    (its ancestors are not seen), and every other output is unaffected."""
    import dataclasses
    from linear_attention_speculative_head_amd import binding
    say(f"[attention] malformed parent: N={N}, parent[{node}] = {bad}")
    P = inputs.make_attention_problem(12, B=2, G=2, N=N, T_max=N + 64, ctx=np.array([10, 20]))
    par = P.parent.copy()
    par[1, node] = bad
    O, st = run_attention(dataclasses.replace(P, parent=par), status_check=False)
    assert st == binding.TREEWY_ETREE
    fixed = par.copy()
    fixed[1, node] = -1
    check(dataclasses.replace(P, parent=fixed), O, "malformed parent read as a root")


def test_kv_commit_appends_the_accepted_path():
    import torch
    from linear_attention_speculative_head_amd import binding
    from oracle import attention as att
    P = inputs.make_attention_problem(13, B=4, G=2, N=10, T_max=80, ctx=np.array([0, 30, 70, 5]),
                                      tree=(4, 3), accepted=np.array([9, -1, 0, 6]))
    d = upload(P)
    ctx_out = torch.full((P.B,), -7, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.treewy_kv_commit(d["Kc"], d["Vc"], d["ctx"], ctx_out, d["Kd"], d["Vd"], d["parent"],
                             d["accepted"], status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    Kc, Vc, ctx = att.kv_commit(P.Kc, P.Vc, P.ctx, P.Kd, P.Vd, P.parent, P.accepted)
    assert np.array_equal(ctx_out.cpu().numpy(), ctx)
    got = d["Kc"].float().cpu().numpy(), d["Vc"].float().cpu().numpy()
    assert np.array_equal(got[0], Kc) and np.array_equal(got[1], Vc)


def test_kv_commit_then_verify_sees_the_committed_path():
    """Commit of step 1's accepted path, then a verify of step 2's drafts over the longer
    prefix, against the oracle doing the same."""
    import torch
    from linear_attention_speculative_head_amd import binding
    from oracle import attention as att
    P1 = inputs.make_attention_problem(14, B=3, G=8, N=6, T_max=900, ctx=np.array([800, 0, 511]),
                                       tree=(3, 2), accepted=np.array([5, 2, -1]))
    d = upload(P1)
    ctx2 = torch.zeros(3, dtype=torch.int32, device="cuda")
    binding.treewy_kv_commit(d["Kc"], d["Vc"], d["ctx"], ctx2, d["Kd"], d["Vd"], d["parent"],
                             d["accepted"])
    Kc, Vc, c2 = att.kv_commit(P1.Kc, P1.Vc, P1.ctx, P1.Kd, P1.Vd, P1.parent, P1.accepted)
    P2 = inputs.make_attention_problem(15, B=3, G=8, N=6, T_max=900, ctx=c2, tree=(3, 2))
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16).contiguous()
    O = torch.empty((3, 6, 16, 256), device="cuda")
    ws = torch.empty(binding.treewy_tree_attention_workspace(3, 2, 8, 6, 900), dtype=torch.uint8,
                     device="cuda")
    parent2 = torch.from_numpy(P2.parent).cuda()
    binding.treewy_tree_attention(d["Kc"], d["Vc"], ctx2, bf(P2.Qd), bf(P2.Kd), bf(P2.Vd),
                                  parent2, O, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ctx2.cpu().numpy(), c2)
    P2.Kc, P2.Vc = Kc, Vc            # the committed cache (rows past c2 are never read)
    check(P2, O.cpu().numpy(), "after commit")
