"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Gate: per (layer, sequence, head), max|x - oracle| / max|oracle| <= 1e-3 for O, U, gamma and
the committed state; depth and ancestor masks bit-exact.  Small cases are compared on every
head; the full-size configurations run in the same launch configuration as the benchmark
and are compared on every head too (config 3: two whole layers).
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import check_against_oracle, run_verify_commit, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_config_full(cfg):
    """Small configurations: every head of every sequence."""
    say(f"[parity] config {cfg}: {inputs.CONFIGS[cfg]['desc']}")
    P = inputs.make_problem(cfg)
    gpu = run_verify_commit(P)
    check_against_oracle(P, gpu, label=f"cfg{cfg}")


def test_config3_whole_layers():
    """B128 x H32, N=64 trees: two of the 30 layers at full size, every head (the persistent
    grid's every round)."""
    say("[parity] config 3 (2 of 30 layers, full B x H, every head)")
    P = inputs.make_problem(3, layers=2)
    for l in range(2):
        gpu = run_verify_commit(P, layer_idx=l)
        check_against_oracle(P, gpu, layer_idx=l, label=f"cfg3 layer{l}")


def test_config4_every_head():
    """B256 x H64, N=32 trees at full size, every head."""
    say("[parity] config 4 (full size, every head)")
    P = inputs.make_problem(4)
    gpu = run_verify_commit(P)
    check_against_oracle(P, gpu, label="cfg4")


@pytest.mark.parametrize("N,tree,dtype,seed", [
    (1, "chain", "bf16", 1),
    (1, "chain", "f32", 2),
    (3, (2, 2), "bf16", 3),
    (7, (3, 3), "f32", 4),
    (33, (6, 4), "bf16", 5),
    (64, "chain", "bf16", 6),      # deepest tree: depth 64, 2080 ancestor pairs
    (64, (6, 8), "f32", 7),
    (64, (2, 64), "bf16", 8),      # all 64 nodes hang off S0 (a star: depth 1)
    (17, (5, 4), "bf16", 9),
    (48, (6, 8), "bf16", 10),      # the largest tree of the three-tile head kernel
    (49, "chain", "bf16", 11),     # the smallest of the four-tile one
])
def test_edge_trees(N, tree, dtype, seed):
    """Ragged and degenerate trees, both input types, every head compared."""
    say(f"[parity] edge N={N} tree={tree} dtype={dtype}")
    if tree == (2, 64):
        par = np.full((3, N), -1, dtype=np.int32)
        P = inputs.make_custom(seed, B=3, H=5, N=N, dtype=dtype, parent=par)
    else:
        P = inputs.make_custom(seed, B=3, H=5, N=N, dtype=dtype, tree=tree)
    gpu = run_verify_commit(P)
    check_against_oracle(P, gpu, label=f"edge N={N}")


def test_nothing_accepted_is_a_bit_exact_noop():
    """a = -1 leaves S untouched, bit for bit."""
    P = inputs.make_custom(11, B=4, H=3, N=8, accepted=np.full(4, -1))
    gpu = run_verify_commit(P)
    assert np.array_equal(gpu["S_new"], P.layers[0].S0)


def test_deterministic_and_stream_independent():
    """Two runs (default stream, then a side stream) give bit-identical results."""
    import torch
    P = inputs.make_custom(12, B=8, H=4, N=24, tree=(6, 4))
    r1 = run_verify_commit(P)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r2 = run_verify_commit(P, stream=s)
    for k in ("O", "U", "gamma", "S_new", "anc", "depth"):
        assert np.array_equal(r1[k], r2[k]), k


def test_malformed_tree_sets_status():
    """A parent outside [-1, t-1] is reported on the device status word; sequences with a
    valid tree are still computed correctly."""
    import torch
    from linear_attention_speculative_head_amd import binding, device
    P = inputs.make_custom(13, B=3, H=2, N=6, tree="chain", accepted=np.array([5, 5, 5]))
    bad = P.parent.copy()
    bad[1, 3] = 4                      # a parent after its child
    P_bad = inputs.Problem(cfg=-1, B=3, H=2, N=6, dtype=P.dtype, parent=bad,
                           accepted=P.accepted, layers=P.layers)
    gpu = run_verify_commit(P_bad, status_check=False)
    assert gpu["status"] == binding.TREEWY_ETREE
    P_ok = inputs.Problem(cfg=-1, B=3, H=2, N=6, dtype=P.dtype, parent=P.parent,
                          accepted=P.accepted, layers=P.layers)
    heads = [(b, h) for b in (0, 2) for h in range(2)]
    gpu.pop("anc"); gpu.pop("depth")
    check_against_oracle(P_ok, gpu, heads=heads, label="valid sequences beside a bad one")


def test_bad_accepted_sets_status():
    import torch
    from linear_attention_speculative_head_amd import binding, device
    P = inputs.make_custom(14, B=2, H=2, N=5, accepted=np.array([7, 2]))
    L = P.layers[0]
    dl = device.upload_layer(L, P.dtype)
    parent, accepted = device.upload_tree(P)
    out = device.alloc_outputs(P.B, P.H, P.N)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.treewy_verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, parent, out.O, out.U,
                          out.gamma, status=status)
    S = dl.S0.clone()
    binding.treewy_commit(S, out.U, dl.K, out.gamma, parent, accepted, status)
    torch.cuda.synchronize()
    assert int(status.item()) == binding.TREEWY_EACCEPT
    assert np.array_equal(S[0].cpu().numpy(), L.S0[0])       # offending sequence untouched


def max_heads_problem(seed: int, N: int, dtype: str, tree, H: int = 65536, base: int = 512):
    """One sequence with the most heads a call takes (H = 65536), so that the last node's rows
    sit at the largest byte offsets the kernels form (about 63 x 65536 x 512 B for O and U).
    A base draw of `base` heads is repeated across the heads, and every head's state and
    values get a head-dependent shift, so that a head read in place of another shows."""
    Pb = inputs.make_custom(seed, B=1, H=base, N=N, dtype=dtype, tree=tree)
    L = Pb.layers[0]
    rep = H // base
    hs = (np.arange(H) % 1009).astype(np.float32)
    S0 = np.tile(L.S0, (1, rep, 1, 1))
    S0 += (1e-4 * hs)[None, :, None, None]
    v = np.tile(L.v, (1, 1, rep, 1))
    v += (1e-3 * hs)[None, None, :, None]
    if dtype == "bf16":
        v = inputs.round_bf16(v)
    layer = inputs.Layer(S0=S0, q=np.tile(L.q, (1, 1, rep, 1)), k=np.tile(L.k, (1, 1, rep, 1)),
                         v=v, alpha=np.tile(L.alpha, (1, 1, rep)),
                         beta=np.tile(L.beta, (1, 1, rep)))
    P = inputs.Problem(cfg=-1, B=1, H=H, N=N, dtype=dtype, parent=Pb.parent,
                       accepted=Pb.accepted)
    P.layers.append(layer)
    return P


@pytest.mark.parametrize("N,dtype,tree,seed", [
    (64, "bf16", (6, 8), 41),      # the one-head-per-item kernel, the last node's rows far out
    (4, "f32", "chain", 42),       # the fp32 kernel: 8 workgroups per head, 524 288 in all
])
def test_max_heads(N, dtype, tree, seed):
    """H = 65536 (the ABI's limit), one sequence: verify then commit, compared with the oracle
    on heads spread over the whole range (the first, the last, and the middle)."""
    say(f"[parity] H=65536 N={N} {dtype}")
    P = max_heads_problem(seed, N, dtype, tree)
    P.accepted[0] = int(np.argmax(inputs.tree_depths(P.parent[0])))   # the deepest node
    gpu = run_verify_commit(P)
    heads = [(0, h) for h in (0, 1, 511, 512, 1009, 20000, 32767, 32768, 49999, 65534, 65535)]
    check_against_oracle(P, gpu, heads=heads, label=f"H=65536 N={N} {dtype}")
