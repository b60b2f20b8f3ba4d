"""The decoding step as a captured HIP graph: one treewy_commit_verify per graph, captured
once for each parity of the alternating per-step buffers, then replayed as a decode loop.
Every replay is checked against the same calls made eagerly, bit for bit (same kernels, same
inputs, same order), with unrelated eager work and synchronisations between replays; the
first replay is also checked against the oracle.
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import check_fused, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


@pytest.mark.parametrize("N,tree", [(6, (4, 2)), (4, "chain"), (16, (5, 4))])
def test_fused_step_graph_replays_match_eager(N, tree):
    import torch
    from linear_attention_speculative_head_amd import binding, device
    say(f"[graph] fused step, N={N} {tree}")
    B, H = 4, 3
    P = [inputs.make_custom(60 + 2 * N, B=B, H=H, N=N, tree=tree),
         inputs.make_custom(61 + 2 * N, B=B, H=H, N=N, tree=tree)]
    dl = [device.upload_layer(p.layers[0], p.dtype) for p in P]
    tr = [device.upload_tree(p) for p in P]

    def side():
        outs = [device.alloc_outputs(B, H, N, fill=float("nan")) for _ in range(2)]
        anc = torch.zeros((B, N), dtype=torch.int64, device="cuda")
        dep = torch.zeros((B, N), dtype=torch.int32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        S = dl[0].S0.clone()
        binding.treewy_verify(S, dl[0].Q, dl[0].K, dl[0].V, dl[0].alpha, dl[0].beta, tr[0][0],
                              outs[0].O, outs[0].U, outs[0].gamma, status=status)
        return dict(outs=outs, anc=anc, dep=dep, status=status, S=S)

    def step(x, r):
        # step r commits the previous step's accepted node (drafts of P[r % 2]) and verifies
        # the drafts of P[(r + 1) % 2]; outputs alternate between the two buffer sets
        p, c = r % 2, (r + 1) % 2
        prev, cur = x["outs"][p], x["outs"][c]
        binding.treewy_commit_verify(x["S"], prev.U, dl[p].K, prev.gamma, tr[p][0], tr[p][1],
                                     dl[c].Q, dl[c].K, dl[c].V, dl[c].alpha, dl[c].beta,
                                     tr[c][0], cur.O, cur.U, cur.gamma, x["anc"], x["dep"],
                                     x["status"])

    g_side, e_side = side(), side()
    torch.cuda.synchronize()
    graphs = []
    for r in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(g_side, r)
        graphs.append(g)
    torch.cuda.synchronize()

    junk = torch.randn(1 << 20, device="cuda")
    for r in range(6):
        graphs[r % 2].replay()
        junk.mul_(0.5).add_(1.0)                       # unrelated eager work between replays
        torch.cuda.synchronize()
        step(e_side, r)
        torch.cuda.synchronize()
        c = (r + 1) % 2
        for name in ("O", "U", "gamma"):
            a = getattr(g_side["outs"][c], name)
            b = getattr(e_side["outs"][c], name)
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
        assert torch.equal(g_side["S"], e_side["S"]), f"replay {r}: state differs"
        assert torch.equal(g_side["anc"], e_side["anc"]) and torch.equal(g_side["dep"], e_side["dep"])
        assert int(g_side["status"].item()) == 0 and int(e_side["status"].item()) == 0
        if r == 0:
            o = g_side["outs"][1]
            gpu = dict(O=o.O.cpu().numpy(), U=o.U.cpu().numpy(), gamma=o.gamma.cpu().numpy(),
                       S=g_side["S"].cpu().numpy(),
                       anc=g_side["anc"].cpu().numpy().view(np.uint64),
                       depth=g_side["dep"].cpu().numpy())
            check_fused(P[0], P[1], gpu, label=f"graph replay 0, N={N}")
    say(f"  six replays equal to the eager calls; the first matches the oracle")
