"""The tree-attention entry point that allocates nothing (treewy_tree_attention_noalloc),
through the C ABI, against the workspace form (treewy_tree_attention) on the same inputs:
two calls in a row, the second with smaller sizes, so the second also shows that nothing the
first left in the library's fixed device array leaks into it.  Both forms run the same kernels,
so the outputs are compared bit for bit (stricter than the 1e-3 head-wise gate)."""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu


def upload(P):
    import torch
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16).contiguous()
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    return dict(Kc=bf(P.Kc), Vc=bf(P.Vc), ctx=i32(P.ctx), Qd=bf(P.Qd), Kd=bf(P.Kd), Vd=bf(P.Vd),
                parent=i32(P.parent))


def both_forms(P):
    import torch
    from linear_attention_speculative_head_amd import binding
    d = upload(P)
    out = []
    for form in ("workspace", "noalloc"):
        O = torch.full((P.B, P.N, P.Hq, 256), float("nan"), device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if form == "workspace":
            ws = torch.empty(binding.treewy_tree_attention_workspace(P.B, P.Hkv, P.G, P.N, P.T_max),
                             dtype=torch.uint8, device="cuda")
            binding.treewy_tree_attention(d["Kc"], d["Vc"], d["ctx"], d["Qd"], d["Kd"], d["Vd"],
                                          d["parent"], O, ws, status)
        else:
            binding.treewy_tree_attention_noalloc(d["Kc"], d["Vc"], d["ctx"], d["Qd"], d["Kd"],
                                                  d["Vd"], d["parent"], O, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, (form, int(status.item()))
        out.append(O.cpu().numpy())
    return out


def test_noalloc_matches_workspace_form_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    # a larger call (several cache ranges per query block, a 64-node tree), then a smaller one
    cases = [dict(seed=901, B=6, N=64, T_max=3000, tree=(6, 8)),
             dict(seed=902, B=2, N=5, T_max=300, tree="chain")]
    for c in cases:
        say(f"[noalloc] B={c['B']} N={c['N']} T_max={c['T_max']} tree={c['tree']}")
        P = inputs.make_attention_problem(c["seed"], B=c["B"], N=c["N"], T_max=c["T_max"],
                                          tree=c["tree"])
        need = binding.treewy_tree_attention_workspace(P.B, P.Hkv, P.G, P.N, P.T_max)
        assert 0 < need <= (48 << 20)
        ref, got = both_forms(P)
        assert np.all(np.isfinite(ref))
        assert np.array_equal(got, ref), f"max |diff| {np.abs(got - ref).max():.3e}"

