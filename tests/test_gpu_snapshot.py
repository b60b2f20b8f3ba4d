"""GPU parity of the store-all comparison path (every node's state materialised).

Each snapshot Snap[b,h,t] must equal the oracle's replayed state at node t, O the oracle's
outputs, and the rollback S <- Snap[a] the oracle's committed state; same head-wise 1e-3 bar.
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import TOL, headwise_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_snapshot(P, heads, nodes_per_head=None):
    import torch
    import oracle
    from linear_attention_speculative_head_amd import binding, device
    L = P.layers[0]
    dl = device.upload_layer(L, P.dtype)
    parent, accepted = device.upload_tree(P)
    B, H, N = P.B, P.H, P.N
    O = torch.full((B, N, H, 128), float("nan"), device="cuda")
    Snap = torch.empty((B, H, N, 128, 128), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.treewy_verify_snapshot(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, parent, O, Snap,
                                   status)
    S = dl.S0.clone()
    binding.treewy_commit_snapshot(S, Snap, accepted, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    worst = dict(O=0.0, Snap=0.0, S_new=0.0)
    for (b, h) in heads:
        args = (L.S0[b, h], L.q[b, :, h], L.k[b, :, h], L.v[b, :, h], L.alpha[b, :, h],
                L.beta[b, :, h], P.parent[b])
        ref = oracle.head(*args, int(P.accepted[b]))
        o = O[b, :, h].cpu().numpy().astype(np.float64)
        e = headwise_rel(o[None], ref["O"][None])[0]
        worst["O"] = max(worst["O"], e)
        s = S[b, h].cpu().numpy().astype(np.float64)
        worst["S_new"] = max(worst["S_new"], headwise_rel(s[None], ref["S_new"][None])[0])
        ts = range(N) if nodes_per_head is None else sorted({0, N - 1, *nodes_per_head})
        for t in ts:
            st = oracle.head(*args, t)["S_new"]
            g = Snap[b, h, t].cpu().numpy().astype(np.float64)
            worst["Snap"] = max(worst["Snap"], headwise_rel(g[None], st[None])[0])
    say("  snapshot worst head-wise rel err: " + ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= TOL, (k, v)


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_snapshot_small_configs(cfg):
    say(f"[snapshot] config {cfg}")
    P = inputs.make_problem(cfg)
    heads = [(b, h) for b in range(P.B) for h in range(P.H)]
    if len(heads) > 48:
        rng = np.random.default_rng(cfg)
        heads = [heads[i] for i in sorted(rng.choice(len(heads), 48, replace=False))]
    run_snapshot(P, heads)


@pytest.mark.parametrize("N,tree,dtype,seed", [(1, "chain", "bf16", 21), (64, "chain", "f32", 22),
                                               (40, (6, 4), "bf16", 23)])
def test_snapshot_edges(N, tree, dtype, seed):
    say(f"[snapshot] edge N={N} tree={tree}")
    P = inputs.make_custom(seed, B=2, H=3, N=N, dtype=dtype, tree=tree)
    run_snapshot(P, [(b, h) for b in range(2) for h in range(3)])


def test_snapshot_config4_sampled():
    """Full config 4 (32 GiB of snapshots), sampled heads and nodes."""
    say("[snapshot] config 4 full size")
    P = inputs.make_problem(4)
    run_snapshot(P, [(0, 0), (255, 63), (100, 17), (31, 40)], nodes_per_head=[5, 13, 20])
