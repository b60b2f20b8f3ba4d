"""The allocating forms of the calls (``api``) return exactly what the out-parameter calls
write, and ``check=True`` turns a device-reported error into an exception."""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


def test_verify_commit_forms_match():
    import torch
    import oracle
    import linear_attention_speculative_head_amd as tw
    from linear_attention_speculative_head_amd import binding, device
    P = inputs.make_custom(81, B=3, H=4, N=6, tree=(3, 2))
    dl = device.upload_layer(P.layers[0], P.dtype)
    par, acc = device.upload_tree(P)
    out = device.alloc_outputs(3, 4, 6, fill=float("nan"))
    binding.treewy_verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, par, out.O, out.U, out.gamma)
    O, U, g, anc, dep = tw.verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, par, with_tree=True,
                                  check=True)
    assert torch.equal(O, out.O) and torch.equal(U, out.U) and torch.equal(g, out.gamma)
    for b in range(3):
        d, _ = oracle.index_tree(P.parent[b])
        assert np.array_equal(dep[b].cpu().numpy(), d)
    S1, S2 = dl.S0.clone(), dl.S0.clone()
    binding.treewy_commit(S1, out.U, dl.K, out.gamma, par, acc)
    assert tw.commit(S2, U, dl.K, g, par, acc, check=True) is S2
    assert torch.equal(S1, S2)
    P2 = inputs.make_custom(82, B=3, H=4, N=5, tree=(3, 2))
    d2 = device.upload_layer(P2.layers[0], P2.dtype)
    par2, _ = device.upload_tree(P2)
    S3, S4 = dl.S0.clone(), dl.S0.clone()
    o2 = device.alloc_outputs(3, 4, 5)
    binding.treewy_commit_verify(S3, out.U, dl.K, out.gamma, par, acc, d2.Q, d2.K, d2.V, d2.alpha,
                                 d2.beta, par2, o2.O, o2.U, o2.gamma)
    O2, U2, g2 = tw.commit_verify(S4, U, dl.K, g, par, acc, d2.Q, d2.K, d2.V, d2.alpha, d2.beta,
                                  par2, check=True)
    assert torch.equal(S3, S4) and torch.equal(O2, o2.O) and torch.equal(U2, o2.U)


def test_check_raises_on_a_malformed_tree():
    import linear_attention_speculative_head_amd as tw
    from linear_attention_speculative_head_amd import binding, device
    P = inputs.make_custom(83, B=2, H=2, N=4, tree="chain")
    dl = device.upload_layer(P.layers[0], P.dtype)
    par, _ = device.upload_tree(P)
    par[1, 2] = 3                                   # after its child: malformed
    with pytest.raises(binding.TreeWYError) as e:
        tw.verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, par, check=True)
    assert e.value.code == binding.TREEWY_ETREE


def test_attention_forms_match():
    import torch
    import linear_attention_speculative_head_amd as tw
    from linear_attention_speculative_head_amd import binding
    P = inputs.make_attention_problem(84, B=2, G=4, N=5, T_max=700, ctx=np.array([600, 3]),
                                      tree=(3, 2), accepted=np.array([4, 1]))
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16).contiguous()
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    Kc, Vc, Qd, Kd, Vd = bf(P.Kc), bf(P.Vc), bf(P.Qd), bf(P.Kd), bf(P.Vd)
    ctx, par, acc = i32(P.ctx), i32(P.parent), i32(P.accepted)
    O1 = torch.empty((2, 5, P.Hq, 256), device="cuda")
    ws = torch.empty(binding.treewy_tree_attention_workspace(2, P.Hkv, 4, 5, 700),
                     dtype=torch.uint8, device="cuda")
    binding.treewy_tree_attention(Kc, Vc, ctx, Qd, Kd, Vd, par, O1, ws)
    O2 = tw.tree_attention(Kc, Vc, ctx, Qd, Kd, Vd, par, check=True)
    assert torch.equal(O1, O2)
    Kc2, Vc2 = Kc.clone(), Vc.clone()
    c1 = torch.empty_like(ctx)
    binding.treewy_kv_commit(Kc, Vc, ctx, c1, Kd, Vd, par, acc)
    c2 = tw.kv_commit(Kc2, Vc2, ctx, Kd, Vd, par, acc, check=True)
    assert torch.equal(c1, c2) and torch.equal(Kc, Kc2) and torch.equal(Vc, Vc2)
