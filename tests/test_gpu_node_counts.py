"""GPU parity of every per-node-count form of the small-tree kernel against the oracle.

Trees of 1 to 8 nodes run a kernel compiled for the exact node count in each mode (plain
verify, the fused commit -> verify, the deferred commit), with that count's LDS offsets, loop
bounds and pointer-jumping rounds as constants.  Each form is checked here, through the C ABI:
  - treewy_verify + treewy_commit on random trees of N nodes (accepted: the last node, none,
    a middle node);
  - treewy_commit_verify with a previous tree of another size (9 - N nodes, ragged);
  - treewy_commit_verify_deferred over four steps of N-node trees with a 5-term log (appends
    and write-backs interleave), then a flush.
Gate as everywhere: max|x - oracle| / max|oracle| <= 1e-3 per (sequence, head) and tensor;
depths and ancestor masks bit for bit.
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import TOL, check_against_oracle, check_fused, gather_heads, headwise_rel, \
    run_fused, run_verify_commit, say
from test_gpu_deferred import expected_lengths, oracle_steps, run_steps

pytestmark = pytest.mark.gpu

B, H = 3, 4
NODES = list(range(1, 9))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


def problem(seed, N, accepted=None):
    if accepted is None:
        accepted = np.array([N - 1, -1, N // 2], dtype=np.int32)
    return inputs.make_custom(seed, B=B, H=H, N=N, tree=(4, 3), accepted=accepted)


@pytest.mark.parametrize("N", NODES)
def test_verify_commit_per_node_count(N):
    say(f"[node counts] verify + commit, N={N}")
    P = problem(1100 + N, N)
    check_against_oracle(P, run_verify_commit(P), label=f"N={N}")


@pytest.mark.parametrize("N", NODES)
def test_fused_per_node_count(N):
    Np = 9 - N
    say(f"[node counts] fused, N_prev={Np} -> N={N}")
    P1 = problem(1200 + N, Np)
    P2 = problem(1300 + N, N)
    # the same committed states feed both steps (one layer per step, S0 of step 1)
    P2 = inputs.Problem(cfg=-1, B=B, H=H, N=N, dtype=P2.dtype, parent=P2.parent,
                        accepted=P2.accepted,
                        layers=[inputs.Layer(S0=P1.layers[0].S0, q=P2.layers[0].q,
                                             k=P2.layers[0].k, v=P2.layers[0].v,
                                             alpha=P2.layers[0].alpha, beta=P2.layers[0].beta)])
    check_fused(P1, P2, run_fused(P1, P2), label=f"N_prev={Np} N={N}")


@pytest.mark.parametrize("N", NODES)
def test_deferred_per_node_count(N):
    say(f"[node counts] deferred, N={N}, Lmax 5, four steps")
    steps = [problem(1400 + 10 * N + s, N,
                     accepted=np.array([N - 1, (s + N) % N - (s % 2), N // 2], dtype=np.int32))
             for s in range(4)]
    gpu, flushed = run_steps(steps, 5, flush_at=(3,))
    heads, ref, states = oracle_steps(steps)
    want = expected_lengths(steps, 5)
    for s in range(4):
        for key in ("O", "U"):
            g = gather_heads(gpu[s][key], heads, "node").astype(np.float64)
            e = headwise_rel(g, ref[s][key])
            assert e.max() <= TOL, f"N={N} step {s} {key}: worst {e.max():.3e}"
        if s > 0:
            assert np.array_equal(gpu[s]["len"], want[s]), (N, s, gpu[s]["len"], want[s])
    S = flushed[3].reshape(B * H, -1).astype(np.float64)
    e = headwise_rel(S, states[2].reshape(B * H, -1))
    assert e.max() <= TOL, f"N={N} flushed state: worst {e.max():.3e}"
