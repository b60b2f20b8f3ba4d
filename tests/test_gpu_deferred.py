"""GPU parity of the deferred commit (treewy_commit_verify_deferred, treewy_deferred_flush):
several decoding steps in a row with the committed state kept as scale * (S + logged rank-one
terms), against the oracle stepping the same way (replay up to each step's accepted node,
then a fresh verify of the next step's tree from there).

Checked at every step: this step's O, U and gamma (max|x - oracle| / max|oracle| <= 1e-3 per
head); the log header (length and emptying) against the rule it follows; and, after a flush,
the written-back state against the oracle's committed state.
"""

import numpy as np
import pytest

from linear_attention_speculative_head_amd import inputs
from parity import TOL, gather_heads, headwise_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_speculative_head_amd import binding
    binding.lib()


def run_steps(steps, Lmax, flush_at=()):
    """GPU: a plain verify of step 0, then one deferred step per later step; flushes after
    the steps listed.  Returns per-step host outputs, headers and the flushed states."""
    import torch
    from linear_attention_speculative_head_amd import binding, device
    B, H = steps[0].B, steps[0].H
    dls = [device.upload_layer(P.layers[0], P.dtype) for P in steps]
    trees = [device.upload_tree(P) for P in steps]
    outs = [device.alloc_outputs(B, H, P.N, fill=float("nan")) for P in steps]
    log = device.alloc_log(B, H, Lmax)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    S = dls[0].S0.clone()
    d0 = dls[0]
    binding.treewy_verify(S, d0.Q, d0.K, d0.V, d0.alpha, d0.beta, trees[0][0],
                          outs[0].O, outs[0].U, outs[0].gamma, status=status)
    res = [dict(O=outs[0].O.cpu().numpy(), U=outs[0].U.cpu().numpy())]
    flushed = {}
    for s in range(1, len(steps)):
        prev, cur = outs[s - 1], outs[s]
        dp, dc = dls[s - 1], dls[s]
        si, so, li, lo = log.headers()
        binding.treewy_commit_verify_deferred(S, log.U, log.K, si, so, li, lo, prev.U, dp.K,
                                              prev.gamma, trees[s - 1][0], trees[s - 1][1],
                                              dc.Q, dc.K, dc.V, dc.alpha, dc.beta, trees[s][0],
                                              cur.O, cur.U, cur.gamma, status=status)
        log.flip()
        torch.cuda.synchronize()
        r = dict(O=cur.O.cpu().numpy(), U=cur.U.cpu().numpy(), gamma=cur.gamma.cpu().numpy(),
                 len=log.headers()[2].cpu().numpy().copy(), scale=log.headers()[0].cpu().numpy().copy(),
                 S_raw=S.cpu().numpy().copy())
        res.append(r)
        if s in flush_at:
            si, so, li, lo = log.headers()
            binding.treewy_deferred_flush(S, log.U, log.K, si, so, li, lo, status=status)
            log.flip()
            torch.cuda.synchronize()
            flushed[s] = S.cpu().numpy().copy()
            assert (log.headers()[2].cpu().numpy() == 0).all()
            assert (log.headers()[0].cpu().numpy() == 1).all()
    assert int(status.item()) == 0, f"device status {int(status.item())}"
    return res, flushed


def oracle_steps(steps):
    """Per step: the oracle's outputs from the state committed up to the previous step, and
    the state committed after each step."""
    import oracle
    B, H = steps[0].B, steps[0].H
    heads = [(b, h) for b in range(B) for h in range(H)]
    S_ref = steps[0].layers[0].S0.copy()
    outs, states = [], []
    for P in steps:
        L = P.layers[0]
        layer = inputs.Layer(S0=S_ref, q=L.q, k=L.k, v=L.v, alpha=L.alpha, beta=L.beta)
        r = oracle.batch(layer, P.parent, P.accepted, heads=heads, commit=True)
        outs.append(r)
        S_ref = r["S_new"].reshape(B, H, 128, 128).astype(np.float32)
        states.append(r["S_new"].reshape(B, H, 128, 128))
    return heads, outs, states


def chunk_terms(N):
    """Commit terms the 17-64-node kernel stages per chunk."""
    return 16 if N <= 48 else 8


def expected_lengths(steps, Lmax):
    """The header rule: the accepted path's terms join the log when they fit; otherwise the
    log is emptied into S.  Up to 16 nodes the path must also be short enough to stage with
    the next step (4 nodes for N <= 4, else 8); above 16 nodes the log and the path together
    must fit one chunk of staged terms (16 up to 48 nodes, 8 above).  No accepted node
    leaves the log as it is."""
    B = steps[0].B
    lens = np.zeros(B, dtype=np.int64)
    out = [None]
    for s in range(1, len(steps)):
        P_prev, P = steps[s - 1], steps[s]
        for b in range(B):
            a = int(P_prev.accepted[b])
            if a < 0:
                # nothing to append; above 16 nodes a log longer than the staged chunk is
                # written back all the same
                if P.N > 16 and lens[b] > min(Lmax, chunk_terms(P.N)):
                    lens[b] = 0
                continue
            d = int(inputs.tree_depths(P_prev.parent[b])[a])
            if P.N <= 16:
                stage = 4 if P.N <= 4 else 8
                full = lens[b] + d > Lmax or d > stage
            else:
                full = lens[b] + d > min(Lmax, chunk_terms(P.N))
            lens[b] = 0 if full else lens[b] + d
        out.append(lens.copy())
    return out


@pytest.mark.parametrize("N,tree,Lmax,nsteps,seed,B,H", [
    (4, "chain", 16, 6, 61, 5, 4),     # the configuration-1 chain: the log only grows
    (4, "chain", 4, 7, 62, 5, 4),      # small log: appends and write-backs interleave
    (6, (3, 2), 5, 7, 63, 5, 4),
    (16, (5, 4), 8, 6, 64, 5, 4),      # 16-node trees
    (3, (2, 2), 1, 6, 65, 5, 4),       # a one-term log
    (32, (6, 4), 8, 6, 66, 5, 4),      # 17-32 nodes: items of half a head
    (20, (6, 4), 3, 7, 67, 3, 8),      # a ragged tile, a three-term log
    (64, (6, 8), 8, 6, 68, 9, 32),     # 33-64 nodes: 288 heads, some workgroups take two
    (64, (6, 8), 16, 5, 69, 5, 4),     # a 16-term log behaves as 8 terms above 48 nodes
    (40, (6, 8), 5, 6, 70, 5, 4),
    (40, (6, 8), 16, 7, 73, 5, 4),     # 17-48 nodes: a 16-term log fills up to 16
    (32, (6, 4), 12, 7, 74, 3, 8),
    (64, "chain", 8, 5, 71, 3, 4),     # deep paths: flushes over several chunks of terms
    (24, "chain", 8, 5, 72, 3, 4),
    (16, "chain", 16, 6, 75, 3, 4),    # 9-16 nodes, deep paths: two staged chunks of 8
    (12, (4, 3), 16, 7, 76, 5, 4),     # 9-16 nodes: a log of up to 16 terms in one product
])
def test_deferred_steps(N, tree, Lmax, nsteps, seed, B, H):
    say(f"[deferred] N={N} tree={tree} Lmax={Lmax} steps={nsteps} B={B} H={H}")
    steps = [inputs.make_custom(seed * 10 + s, B=B, H=H, N=N, tree=tree) for s in range(nsteps)]
    flush_at = (nsteps - 1,)
    gpu, flushed = run_steps(steps, Lmax, flush_at=flush_at)
    heads, ref, states = oracle_steps(steps)
    want_len = expected_lengths(steps, Lmax)
    worst = 0.0
    for s in range(nsteps):
        for key in ("O", "U"):
            g = gather_heads(gpu[s][key], heads, "node").astype(np.float64)
            e = headwise_rel(g, ref[s][key])
            assert e.max() <= TOL, f"step {s} {key}: worst {e.max():.3e}"
            worst = max(worst, float(e.max()))
        if s > 0:
            assert np.array_equal(gpu[s]["len"], want_len[s]), (s, gpu[s]["len"], want_len[s])
    # after the last step's call the state stands for the commits of steps 0 .. nsteps - 2
    S = flushed[nsteps - 1].reshape(B * H, -1).astype(np.float64)
    e = headwise_rel(S, states[nsteps - 2].reshape(B * H, -1))
    assert e.max() <= TOL, f"flushed state: worst {e.max():.3e}"
    say(f"  worst O/U head-wise rel err {worst:.2e}, flushed state {e.max():.2e}")


def test_deferred_matches_fused_path():
    """The same steps through treewy_commit_verify (state written every step) and through
    the deferred commit give the same outputs to the tolerance, and the same state after a
    flush."""
    import torch
    from linear_attention_speculative_head_amd import binding, device
    B, H, N = 4, 3, 4
    steps = [inputs.make_custom(70 + s, B=B, H=H, N=N, tree="chain") for s in range(5)]
    gpu, flushed = run_steps(steps, 16, flush_at=(4,))
    dls = [device.upload_layer(P.layers[0], P.dtype) for P in steps]
    trees = [device.upload_tree(P) for P in steps]
    outs = [device.alloc_outputs(B, H, N) for _ in steps]
    S = dls[0].S0.clone()
    binding.treewy_verify(S, dls[0].Q, dls[0].K, dls[0].V, dls[0].alpha, dls[0].beta,
                          trees[0][0], outs[0].O, outs[0].U, outs[0].gamma)
    for s in range(1, 5):
        binding.treewy_commit_verify(S, outs[s - 1].U, dls[s - 1].K, outs[s - 1].gamma,
                                     trees[s - 1][0], trees[s - 1][1], dls[s].Q, dls[s].K,
                                     dls[s].V, dls[s].alpha, dls[s].beta, trees[s][0],
                                     outs[s].O, outs[s].U, outs[s].gamma)
    torch.cuda.synchronize()
    n = B * H
    for s in range(1, 5):
        f = outs[s].O.cpu().numpy().transpose(0, 2, 1, 3).reshape(n, -1).astype(np.float64)
        d = gpu[s]["O"].transpose(0, 2, 1, 3).reshape(n, -1).astype(np.float64)
        assert headwise_rel(d, f).max() <= TOL
    e = headwise_rel(flushed[4].reshape(n, -1).astype(np.float64),
                     S.cpu().numpy().reshape(n, -1).astype(np.float64))
    assert e.max() <= TOL


def test_deferred_mixed_tree_sizes():
    """Consecutive steps on trees of different sizes: the log written by one kernel (up to 16
    nodes, 17-32, 33-64) is read by another."""
    B, H, Lmax = 4, 6, 8
    sizes = [(5, (3, 2)), (40, (6, 8)), (20, (6, 4)), (64, (6, 8)), (12, (4, 3)), (33, (6, 8)),
             (3, "chain")]
    steps = [inputs.make_custom(900 + i, B=B, H=H, N=n, tree=t) for i, (n, t) in enumerate(sizes)]
    nsteps = len(steps)
    gpu, flushed = run_steps(steps, Lmax, flush_at=(nsteps - 1,))
    heads, ref, states = oracle_steps(steps)
    want_len = expected_lengths(steps, Lmax)
    for s in range(nsteps):
        for key in ("O", "U"):
            g = gather_heads(gpu[s][key], heads, "node").astype(np.float64)
            e = headwise_rel(g, ref[s][key])
            assert e.max() <= TOL, f"step {s} (N={steps[s].N}) {key}: worst {e.max():.3e}"
        if s > 0:
            assert np.array_equal(gpu[s]["len"], want_len[s]), (s, gpu[s]["len"], want_len[s])
    S = flushed[nsteps - 1].reshape(B * H, -1).astype(np.float64)
    e = headwise_rel(S, states[nsteps - 2].reshape(B * H, -1))
    assert e.max() <= TOL, f"flushed state: worst {e.max():.3e}"


@pytest.mark.parametrize("n_big,kept", [(64, False), (40, True)])
def test_deferred_long_log_meets_large_tree(n_big, kept):
    """A 12-term log built on 4-node chains (Lmax 16), then steps on n_big-, 24- and 33-node
    trees.  The first accepts nothing in some sequences: at 64 nodes their log is written
    back all the same (it does not fit the 8 terms staged there), at 40 nodes it stays (16
    staged terms).  The later steps append again."""
    say(f"[deferred] long log meets N={n_big}")
    B, H, Lmax = 4, 3, 16
    steps = []
    for s, (n, tree) in enumerate([(4, "chain"), (4, "chain"), (4, "chain"), (4, "chain"),
                                   (n_big, (6, 8)), (24, (6, 4)), (33, (6, 8))]):
        acc = None
        if n == 4:
            acc = np.full(B, 3, dtype=np.int32)          # depth 4 each step: 4, 8, 12
        if s == 3:
            acc = np.array([-1, -1, 3, 0], dtype=np.int32)
        steps.append(inputs.make_custom(950 + s, B=B, H=H, N=n, tree=tree, accepted=acc))
    nsteps = len(steps)
    gpu, flushed = run_steps(steps, Lmax, flush_at=(nsteps - 1,))
    heads, ref, states = oracle_steps(steps)
    want_len = expected_lengths(steps, Lmax)
    assert want_len[3].tolist() == [12, 12, 12, 12]
    assert want_len[4].tolist()[:2] == ([12, 12] if kept else [0, 0])
    for s in range(nsteps):
        for key in ("O", "U"):
            g = gather_heads(gpu[s][key], heads, "node").astype(np.float64)
            e = headwise_rel(g, ref[s][key])
            assert e.max() <= TOL, f"step {s} (N={steps[s].N}) {key}: worst {e.max():.3e}"
        if s > 0:
            assert np.array_equal(gpu[s]["len"], want_len[s]), (s, gpu[s]["len"], want_len[s])
    S = flushed[nsteps - 1].reshape(B * H, -1).astype(np.float64)
    e = headwise_rel(S, states[nsteps - 2].reshape(B * H, -1))
    assert e.max() <= TOL, f"flushed state: worst {e.max():.3e}"


@pytest.mark.parametrize("cfg", [3, 4])
def test_deferred_full_size_sampled(cfg):
    """The deferred step at the benchmark's launches (configuration 3: B128 x H32, 64-node
    trees, eight staged terms, write-backs over two chunks; configuration 4: B256 x H64,
    32-node trees, 64 heads per workgroup), four steps with Lmax 8: the log lengths of every
    sequence against the header rule, O and U of 48 sampled heads (spread over the persistent
    grid's rounds) against the oracle each step, and the flushed state of those heads after
    the last step."""
    import torch
    import oracle
    from linear_attention_speculative_head_amd import binding, device
    say(f"[deferred] config {cfg} full size, 4 steps, Lmax 8, 48 sampled heads")
    Lmax = 8
    steps = [inputs.make_problem(cfg, instance=s, layers=1) for s in range(4)]
    B, H = steps[0].B, steps[0].H
    rng = np.random.default_rng(7)
    hid = np.unique(np.concatenate([[0, B * H - 1], rng.choice(B * H, 46, replace=False)]))
    heads = [(int(x) // H, int(x) % H) for x in hid]
    hb = np.array([x[0] for x in heads])
    hh = np.array([x[1] for x in heads])
    # GPU: a plain verify of step 0, then deferred steps, then a flush
    dls = [device.upload_layer(P.layers[0], P.dtype) for P in steps]
    trees = [device.upload_tree(P) for P in steps]
    outs = [device.alloc_outputs(B, H, P.N) for P in steps[:2]]
    log = device.alloc_log(B, H, Lmax)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    S = dls[0].S0.clone()
    d0 = dls[0]
    binding.treewy_verify(S, d0.Q, d0.K, d0.V, d0.alpha, d0.beta, trees[0][0],
                          outs[0].O, outs[0].U, outs[0].gamma, status=status)
    gpu = []
    for s_ in range(1, len(steps)):
        prev, cur = outs[(s_ - 1) % 2], outs[s_ % 2]
        dp, dc = dls[s_ - 1], dls[s_]
        si, so, li, lo = log.headers()
        binding.treewy_commit_verify_deferred(S, log.U, log.K, si, so, li, lo, prev.U, dp.K,
                                              prev.gamma, trees[s_ - 1][0], trees[s_ - 1][1],
                                              dc.Q, dc.K, dc.V, dc.alpha, dc.beta, trees[s_][0],
                                              cur.O, cur.U, cur.gamma, status=status)
        log.flip()
        torch.cuda.synchronize()
        ti_b = torch.from_numpy(hb).cuda()
        ti_h = torch.from_numpy(hh).cuda()
        gpu.append(dict(O=cur.O[ti_b, :, ti_h].cpu().numpy(), U=cur.U[ti_b, :, ti_h].cpu().numpy(),
                        len=log.headers()[2].cpu().numpy().copy()))
    si, so, li, lo = log.headers()
    binding.treewy_deferred_flush(S, log.U, log.K, si, so, li, lo, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, f"device status {int(status.item())}"
    S_flushed = S[torch.from_numpy(hb).cuda(), torch.from_numpy(hh).cuda()].cpu().numpy()
    # oracle on the sampled heads only, the committed state carried from step to step
    want_len = expected_lengths(steps, Lmax)
    S_ref = steps[0].layers[0].S0.copy()
    for s_, P in enumerate(steps):
        L = P.layers[0]
        layer = inputs.Layer(S0=S_ref, q=L.q, k=L.k, v=L.v, alpha=L.alpha, beta=L.beta)
        r = oracle.batch(layer, P.parent, P.accepted, heads=heads, commit=True)
        if s_ > 0:
            g = gpu[s_ - 1]
            for key in ("O", "U"):
                e = headwise_rel(g[key].astype(np.float64), r[key])
                assert e.max() <= TOL, f"step {s_} {key}: worst {e.max():.3e}"
            assert np.array_equal(g["len"], want_len[s_]), f"step {s_} lengths"
        if s_ == len(steps) - 1:
            break                       # the flush holds the state committed before this step
        S_new = r["S_new"].reshape(len(heads), 128, 128).astype(np.float32)
        S_ref = S_ref.copy()
        S_ref[hb, hh] = S_new
    e = headwise_rel(S_flushed.astype(np.float64), S_ref[hb, hh].astype(np.float64))
    say(f"  flushed state worst head-wise rel err {e.max():.2e}")
    assert e.max() <= TOL, f"flushed state: worst {e.max():.3e}"


def test_deferred_rejects_unsupported_shapes():
    """fp32 inputs have no deferred commit."""
    import torch
    from linear_attention_speculative_head_amd import binding, device
    P = inputs.make_custom(80, B=2, H=2, N=20, tree=(5, 4), dtype="f32")
    d = device.upload_layer(P.layers[0], P.dtype)
    par, acc = device.upload_tree(P)
    o = device.alloc_outputs(2, 2, 20)
    o2 = device.alloc_outputs(2, 2, 20)
    log = device.alloc_log(2, 2, 8)
    si, so, li, lo = log.headers()
    with pytest.raises(binding.TreeWYError):
        binding.treewy_commit_verify_deferred(d.S0, log.U, log.K, si, so, li, lo, o.U, d.K,
                                              o.gamma, par, acc, d.Q, d.K, d.V, d.alpha,
                                              d.beta, par, o2.O, o2.U, o2.gamma)


@pytest.mark.parametrize("N", [4, 24, 40])
def test_deferred_reports_bad_header(N):
    """A log length outside [0, Lmax] is reported (and clamped, so nothing leaves the log)."""
    import torch
    from linear_attention_speculative_head_amd import binding, device
    B, H = 3, 2
    P1 = inputs.make_custom(90, B=B, H=H, N=N, tree="chain")
    P2 = inputs.make_custom(91, B=B, H=H, N=N, tree="chain")
    d1, d2 = device.upload_layer(P1.layers[0], "bf16"), device.upload_layer(P2.layers[0], "bf16")
    par1, acc1 = device.upload_tree(P1)
    par2, _ = device.upload_tree(P2)
    o1, o2 = device.alloc_outputs(B, H, N), device.alloc_outputs(B, H, N)
    binding.treewy_verify(d1.S0, d1.Q, d1.K, d1.V, d1.alpha, d1.beta, par1, o1.O, o1.U, o1.gamma)
    log = device.alloc_log(B, H, 4)
    log.length[0].fill_(99)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    si, so, li, lo = log.headers()
    binding.treewy_commit_verify_deferred(d1.S0, log.U, log.K, si, so, li, lo, o1.U, d1.K,
                                          o1.gamma, par1, acc1, d2.Q, d2.K, d2.V, d2.alpha,
                                          d2.beta, par2, o2.O, o2.U, o2.gamma, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == binding.TREEWY_ELOG


def test_deferred_mixed_sizes_and_deep_paths():
    """Node counts that change between steps: an 8-node chain accepted to its end cannot be
    staged by a 3-node step (4 rows), so that step writes the state back."""
    say("[deferred] mixed node counts, deep accepted paths")
    B, H = 4, 3
    sizes = (8, 3, 8, 3, 8, 4)
    steps = []
    for s, n in enumerate(sizes):
        acc = np.full(B, n - 1, dtype=np.int32)
        acc[1] = -1
        acc[2] = min(1, n - 1)
        steps.append(inputs.make_custom(100 + s, B=B, H=H, N=n, tree="chain", accepted=acc))
    gpu, flushed = run_steps(steps, 16, flush_at=(len(sizes) - 1,))
    heads, ref, states = oracle_steps(steps)
    want_len = expected_lengths(steps, 16)
    for s in range(len(sizes)):
        for key in ("O", "U"):
            g = gather_heads(gpu[s][key], heads, "node").astype(np.float64)
            e = headwise_rel(g, ref[s][key])
            assert e.max() <= TOL, f"step {s} {key}: worst {e.max():.3e}"
        if s > 0:
            assert np.array_equal(gpu[s]["len"], want_len[s]), (s, gpu[s]["len"], want_len[s])
    S = flushed[len(sizes) - 1].reshape(B * H, -1).astype(np.float64)
    e = headwise_rel(S, states[len(sizes) - 2].reshape(B * H, -1))
    assert e.max() <= TOL
