"""GPU parity of treewy_commit_verify: the previous step's commit followed by this step's
verify against the committed state, through the C ABI, against the oracle composed the same
way (replay of step 1 up to its accepted node, then a fresh verify of step 2 from there).

Gate as for the separate calls: per (sequence, head), max|x - oracle| / max|oracle| <= 1e-3
for this step's O, U, gamma and for the committed state; sequences with nothing accepted in
the previous step keep their state bit for bit; ancestor masks and depths are bit-exact.
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import TOL, check_fused, gather_heads, headwise_rel, run_fused, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_fused_config_full(cfg):
    """Two consecutive draws of a configuration: the fused kernel at full size, every head."""
    say(f"[fused] config {cfg}: {inputs.CONFIGS[cfg]['desc']}")
    P1 = inputs.make_problem(cfg, instance=0)
    P2 = inputs.make_problem(cfg, instance=1)
    gpu = run_fused(P1, P2)
    check_fused(P1, P2, gpu, label=f"cfg{cfg}")


@pytest.mark.parametrize("cfg", [3, 4])
def test_fused_config_every_head(cfg):
    """The large-tree fused kernels at the full sizes the benchmark times (config 3: one of its
    layers at full B x H, 64-node trees; config 4: 32-node trees), two consecutive draws,
    every head against the oracle (every round of the persistent grid)."""
    say(f"[fused] config {cfg} (full B x H, every head)")
    P1 = inputs.make_problem(cfg, instance=0, layers=1)
    P2 = inputs.make_problem(cfg, instance=1, layers=1)
    gpu = run_fused(P1, P2)
    check_fused(P1, P2, gpu, label=f"cfg{cfg}")


@pytest.mark.parametrize("N1,tree1,N2,tree2,seed", [
    (4, "chain", 4, "chain", 21),
    (12, (5, 3), 5, (3, 2), 22),      # previous tree larger than this step's
    (3, (2, 2), 16, (5, 4), 23),      # previous tree smaller
    (20, "chain", 8, (4, 3), 24),     # previous paths up to depth 20: chunks of 8 rows
    (64, "chain", 16, "chain", 25),   # depth up to 64: eight chunks
    (40, (6, 4), 1, "chain", 26),
    (7, (3, 3), 9, (4, 3), 27),
    (40, "chain", 24, (5, 4), 28),    # the large-tree kernel's fused commit, paths of 5 chunks
    (64, "chain", 32, "chain", 29),   # ... at its largest tree, paths of up to 8 chunks
    (3, (2, 2), 17, (4, 4), 30),      # ... at its smallest
    (20, (5, 3), 40, (6, 4), 31),     # the unstaged large-tree kernel's fused commit
    (64, "chain", 64, (6, 4), 32),    # ... at 64 nodes, previous paths of up to 64 rows
    (48, "chain", 48, (6, 8), 33),    # the three-tile head kernel, previous paths of 6 chunks
    (33, (6, 4), 45, (6, 8), 34),
])
def test_fused_shapes(N1, tree1, N2, tree2, seed):
    """Ragged node counts on both steps, deep previous paths, every head compared."""
    say(f"[fused] N_prev={N1} {tree1} -> N={N2} {tree2}")
    B, H = 5, 6
    P1 = inputs.make_custom(seed, B=B, H=H, N=N1, tree=tree1)
    # accepted nodes: the deepest node of some sequences, none in one, random elsewhere
    d = np.array([inputs.tree_depths(P1.parent[b]) for b in range(B)])
    acc = P1.accepted.copy()
    acc[0] = int(np.argmax(d[0]))
    acc[1] = -1
    acc[2] = N1 - 1
    P1 = inputs.Problem(cfg=-1, B=B, H=H, N=N1, dtype=P1.dtype, parent=P1.parent,
                        accepted=acc.astype(np.int32), layers=P1.layers)
    P2 = inputs.make_custom(seed + 1000, B=B, H=H, N=N2, tree=tree2)
    gpu = run_fused(P1, P2)
    check_fused(P1, P2, gpu, label=f"N_prev={N1} N={N2}")


@pytest.mark.parametrize("N1,tree1,N2,tree2,seed", [
    (4, "chain", 4, "chain", 51),     # the configuration-0 shape: the register-resident form
    (3, (2, 2), 2, "chain", 52),
    (1, "chain", 4, (3, 2), 53),
    (4, (3, 2), 1, "chain", 54),
    (6, (3, 2), 4, "chain", 55),      # previous tree of 6 nodes: the general fp32 kernel
    (4, "chain", 5, (3, 2), 56),      # 5 nodes: the general fp32 kernel
])
def test_fp32_small_trees(N1, tree1, N2, tree2, seed):
    """fp32 inputs on trees of up to four nodes (and either side of that bound), fused, with
    the deepest, no, and the last accepted node among the sequences; every head compared."""
    say(f"[fused] fp32 N_prev={N1} {tree1} -> N={N2} {tree2}")
    B, H = 5, 6
    P1 = inputs.make_custom(seed, B=B, H=H, N=N1, tree=tree1, dtype="f32")
    d = np.array([inputs.tree_depths(P1.parent[b]) for b in range(B)])
    acc = P1.accepted.copy()
    acc[0] = int(np.argmax(d[0]))
    acc[1] = -1
    acc[2] = N1 - 1
    P1 = inputs.Problem(cfg=-1, B=B, H=H, N=N1, dtype=P1.dtype, parent=P1.parent,
                        accepted=acc.astype(np.int32), layers=P1.layers)
    P2 = inputs.make_custom(seed + 1000, B=B, H=H, N=N2, tree=tree2, dtype="f32")
    gpu = run_fused(P1, P2)
    check_fused(P1, P2, gpu, label=f"fp32 N_prev={N1} N={N2}")


@pytest.mark.parametrize("case", ["accepted", "parent_prev", "parent"])
def test_fp32_small_trees_bad_inputs(case):
    """The register-resident fp32 form on a bad accepted node, a bad previous parent on the
    accepted path, or a bad parent in this step's tree: the error is reported on the status
    word, the offending sequence's state is left as it was (bad accepted node or path), and
    the other sequences match the oracle."""
    say(f"[fused] fp32 four-node trees, bad {case}")
    B, H = 3, 4
    P1 = inputs.make_custom(57, B=B, H=H, N=4, tree="chain", dtype="f32",
                            accepted=np.array([3, 2, 3]))
    P2 = inputs.make_custom(58, B=B, H=H, N=4, tree="chain", dtype="f32")
    if case == "accepted":
        acc = P1.accepted.copy()
        acc[0] = 9
        P1b = inputs.Problem(cfg=-1, B=B, H=H, N=4, dtype=P1.dtype, parent=P1.parent,
                             accepted=acc, layers=P1.layers)
        P2b, want = P2, binding_code("TREEWY_EACCEPT")
    elif case == "parent_prev":
        par = P1.parent.copy()
        par[0, 2] = 3                  # a parent after its child, on node 3's path
        P1b = inputs.Problem(cfg=-1, B=B, H=H, N=4, dtype=P1.dtype, parent=par,
                             accepted=P1.accepted, layers=P1.layers)
        P2b, want = P2, binding_code("TREEWY_ETREE")
    else:
        par = P2.parent.copy()
        par[0, 1] = 2
        P1b = P1
        P2b = inputs.Problem(cfg=-1, B=B, H=H, N=4, dtype=P2.dtype, parent=par,
                             accepted=P2.accepted, layers=P2.layers)
        want = binding_code("TREEWY_ETREE")
    gpu = run_fused(P1b, P2b, status_check=False)
    assert gpu["status"] == want, (gpu["status"], want)
    if case != "parent":
        # the offending sequence keeps its state bit for bit
        assert np.array_equal(gpu["S"][0], P1.layers[0].S0[0])
    heads = [(b, h) for b in (1, 2) for h in range(H)]
    check_fused(P1, P2, gpu, heads=heads, label=f"fp32 bad {case}: valid sequences")


def binding_code(name):
    from linear_attention_speculative_head_amd import binding
    return getattr(binding, name)


@pytest.mark.parametrize("N2,dtype", [(32, "bf16"), (64, "bf16"), (6, "f32")])
def test_unfused_shapes_match(N2, dtype):
    """Every kernel shape under the same contract: the large-tree kernels (bf16, fused) and
    fp32 inputs (commit then verify)."""
    say(f"[fused] two-kernel shape N={N2} {dtype}")
    P1 = inputs.make_custom(31, B=3, H=4, N=10, dtype=dtype, tree=(4, 3))
    P2 = inputs.make_custom(32, B=3, H=4, N=N2, dtype=dtype, tree=(6, 4))
    gpu = run_fused(P1, P2)
    check_fused(P1, P2, gpu, label=f"N={N2} {dtype}")


def test_fused_steps_chain_like_decoding():
    """Three steps in a row with alternating per-step buffers, against the oracle stepping
    the same way (commit of step s, then verify of step s + 1)."""
    import torch
    import oracle
    from linear_attention_speculative_head_amd import binding, device
    B, H, N = 4, 3, 6
    steps = [inputs.make_custom(40 + s, B=B, H=H, N=N, tree=(4, 2)) for s in range(4)]
    heads = [(b, h) for b in range(B) for h in range(H)]
    # GPU: verify step 0, then commit_verify steps 1..3
    dls = [device.upload_layer(P.layers[0], P.dtype) for P in steps]
    trees = [device.upload_tree(P) for P in steps]
    outs = [device.alloc_outputs(B, H, N, fill=float("nan")) for _ in range(2)]
    S = dls[0].S0.clone()
    d0 = dls[0]
    binding.treewy_verify(S, d0.Q, d0.K, d0.V, d0.alpha, d0.beta, trees[0][0],
                          outs[0].O, outs[0].U, outs[0].gamma)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(1, 4):
        prev, cur = outs[(s - 1) % 2], outs[s % 2]
        dp, dc = dls[s - 1], dls[s]
        binding.treewy_commit_verify(S, prev.U, dp.K, prev.gamma, trees[s - 1][0], trees[s - 1][1],
                                     dc.Q, dc.K, dc.V, dc.alpha, dc.beta, trees[s][0],
                                     cur.O, cur.U, cur.gamma, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # oracle: the same sequence of commits and verifies, state carried in float32
    S_ref = steps[0].layers[0].S0.copy()
    for s in range(0, 4):
        L = steps[s].layers[0]
        layer = inputs.Layer(S0=S_ref, q=L.q, k=L.k, v=L.v, alpha=L.alpha, beta=L.beta)
        r = oracle.batch(layer, steps[s].parent, steps[s].accepted, heads=heads, commit=True)
        if s == 3:
            break
        S_ref = r["S_new"].reshape(B, H, 128, 128).astype(np.float32)
    last = outs[3 % 2]
    for key, ref in (("O", r["O"]), ("U", r["U"])):
        g = gather_heads(getattr(last, key).cpu().numpy(), heads, "node").astype(np.float64)
        e = headwise_rel(g, ref)
        assert e.max() <= TOL, f"{key}: worst {e.max():.3e}"
    e = headwise_rel(S.cpu().numpy().reshape(B * H, -1).astype(np.float64),
                     S_ref.reshape(B * H, -1).astype(np.float64))
    assert e.max() <= TOL, f"S: worst {e.max():.3e}"
    say(f"  three fused steps: worst O/U/S rel err within {TOL}")


def test_fused_reports_bad_previous_step():
    """An accepted node outside the previous tree, or a malformed parent on its path, is
    reported; that sequence keeps its state, the others commit and verify normally."""
    from linear_attention_speculative_head_amd import binding
    B, H = 4, 2
    P1 = inputs.make_custom(51, B=B, H=H, N=6, tree="chain",
                            accepted=np.array([5, 9, 3, 4], dtype=np.int32))
    P2 = inputs.make_custom(52, B=B, H=H, N=5, tree=(3, 2))
    gpu = run_fused(P1, P2, status_check=False)
    assert gpu["status"] == binding.TREEWY_EACCEPT
    assert np.array_equal(gpu["S"][1], P1.layers[0].S0[1])
    ok = [(b, h) for b in (0, 2, 3) for h in range(H)]
    P1ok = inputs.Problem(cfg=-1, B=B, H=H, N=6, dtype=P1.dtype, parent=P1.parent,
                          accepted=np.array([5, -1, 3, 4], dtype=np.int32), layers=P1.layers)
    check_fused(P1ok, P2, gpu, heads=ok, label="beside a bad accepted node")

    bad = P1.parent.copy()
    bad[2, 3] = 5                      # node 3's parent after it: on the path of accepted 3
    P1b = inputs.Problem(cfg=-1, B=B, H=H, N=6, dtype=P1.dtype, parent=bad,
                         accepted=np.array([5, -1, 3, 4], dtype=np.int32), layers=P1.layers)
    gpu = run_fused(P1b, P2, status_check=False)
    assert gpu["status"] == binding.TREEWY_ETREE
    assert np.array_equal(gpu["S"][2], P1.layers[0].S0[2])
