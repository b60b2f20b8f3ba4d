"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerance (the bar for fp32 state with bf16 or fp32 inputs): for every (layer, sequence,
head) and every tensor x in {O, U, gamma, S_new},
    max|x - x_oracle| / max|x_oracle| <= 1e-3.
A norm-wise bound per head: an elementwise relative bound is ill-posed for outputs that
cross zero.  Indexing outputs (depth, ancestor masks) must match bit for bit.
"""

from __future__ import annotations

import sys

import numpy as np

TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def headwise_rel(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """x, ref: [n_heads, ...] -> per-head max-abs error over max-abs reference."""
    n = x.shape[0]
    e = np.abs(x.reshape(n, -1) - ref.reshape(n, -1)).max(axis=1)
    s = np.abs(ref.reshape(n, -1)).max(axis=1)
    return e / np.maximum(s, 1e-30)


def gather_heads(t: np.ndarray, heads, kind: str) -> np.ndarray:
    """Pick (b, h) heads out of a device-layout array.
    kind 'node': [B,N,H,...] -> [n,N,...]; 'state': [B,H,...] -> [n,...]."""
    b = np.array([x[0] for x in heads])
    h = np.array([x[1] for x in heads])
    if kind == "node":
        return t[b, :, h]
    return t[b, h]


def run_verify_commit(problem, layer_idx=0, anc=True, status_check=True, stream=None):
    """Upload one layer, run treewy_verify then treewy_commit, return host arrays."""
    import torch
    from linear_attention_speculative_head_amd import binding, device

    L = problem.layers[layer_idx]
    dl = device.upload_layer(L, problem.dtype)
    parent, accepted = device.upload_tree(problem)
    B, H, N = problem.B, problem.H, problem.N
    out = device.alloc_outputs(B, H, N, fill=float("nan"))
    anc_t = torch.zeros((B, N), dtype=torch.int64, device="cuda") if anc else None
    dep_t = torch.zeros((B, N), dtype=torch.int32, device="cuda") if anc else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.treewy_verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, parent, out.O, out.U,
                          out.gamma, anc_t, dep_t, status, stream=stream)
    S = dl.S0.clone()
    binding.treewy_commit(S, out.U, dl.K, out.gamma, parent, accepted, status, stream=stream)
    torch.cuda.synchronize()
    res = dict(O=out.O.cpu().numpy(), U=out.U.cpu().numpy(), gamma=out.gamma.cpu().numpy(),
               S_new=S.cpu().numpy(), status=int(status.item()))
    if anc:
        res["anc"] = anc_t.cpu().numpy().view(np.uint64)
        res["depth"] = dep_t.cpu().numpy()
    if status_check:
        assert res["status"] == 0, f"device status {res['status']}"
    return res


def check_against_oracle(problem, gpu, heads=None, layer_idx=0, tol=TOL, label=""):
    """Compare GPU results with the oracle on the given heads (default: all)."""
    import oracle
    if heads is None:
        heads = [(b, h) for b in range(problem.B) for h in range(problem.H)]
    ref = oracle.batch(problem.layers[layer_idx], problem.parent, problem.accepted, heads=heads)
    worst = {}
    for key, kind in (("O", "node"), ("U", "node"), ("gamma", "node"), ("S_new", "state")):
        g = gather_heads(gpu[key], heads, kind).astype(np.float64)
        r = ref[key]
        assert np.all(np.isfinite(g)), f"{label} {key}: non-finite GPU values"
        e = headwise_rel(g, r)
        worst[key] = float(e.max())
        bad = np.flatnonzero(e > tol)
        assert len(bad) == 0, (f"{label} {key}: {len(bad)} heads above {tol}; worst "
                               f"{e.max():.3e} at head {heads[int(np.argmax(e))]}")
    if "anc" in gpu:
        for b in sorted({x[0] for x in heads}):
            d, a = oracle.index_tree(problem.parent[b])
            assert np.array_equal(gpu["depth"][b], d), f"{label} depth mismatch at b={b}"
            assert np.array_equal(gpu["anc"][b], a), f"{label} anc mismatch at b={b}"
    say(f"  {label} worst head-wise rel err: " + ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    return worst
