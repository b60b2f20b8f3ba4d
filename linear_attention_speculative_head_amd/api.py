"""Allocating forms of the library calls, for callers that want tensors back.

Each function allocates its outputs with torch on the inputs' device (and, for the
attention call, the workspace), then enqueues the C-ABI call of the same name through
``binding`` on torch's current stream.  Nothing is computed here.  With ``check=True`` the
call synchronises and raises ``TreeWYError`` if the device reported a malformed tree, an
accepted node out of range or a bad context length.
"""

from __future__ import annotations

from . import binding

D = 128


def _status(dev):
    import torch
    return torch.zeros(1, dtype=torch.int32, device=dev)


def _raise_on(status):
    code = int(status.item())
    if code != binding.TREEWY_OK:
        raise binding.TreeWYError(code, "device status")


def verify(S0, Q, K, V, alpha, beta, parent, with_tree=False, check=False):
    """Tree verification of one layer: returns (O, U, gamma), plus (anc, depth) when
    ``with_tree``.  S0 is only read."""
    import torch
    B, N, H, _ = Q.shape
    dev = S0.device
    O = torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
    U = torch.empty_like(O)
    gamma = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    anc = torch.empty((B, N), dtype=torch.int64, device=dev) if with_tree else None
    depth = torch.empty((B, N), dtype=torch.int32, device=dev) if with_tree else None
    status = _status(dev)
    binding.treewy_verify(S0, Q, K, V, alpha, beta, parent, O, U, gamma, anc, depth, status)
    if check:
        _raise_on(status)
    return (O, U, gamma, anc, depth) if with_tree else (O, U, gamma)


def commit(S, U, K, gamma, parent, accepted, check=False):
    """The accepted node's commit, in place on S (returned)."""
    status = _status(S.device)
    binding.treewy_commit(S, U, K, gamma, parent, accepted, status)
    if check:
        _raise_on(status)
    return S


def commit_verify(S, U_prev, K_prev, gamma_prev, parent_prev, accepted_prev,
                  Q, K, V, alpha, beta, parent, check=False):
    """The previous step's commit into S (in place) and this step's verify against it:
    returns (O, U, gamma) of this step."""
    import torch
    B, N, H, _ = Q.shape
    dev = S.device
    O = torch.empty((B, N, H, D), dtype=torch.float32, device=dev)
    U = torch.empty_like(O)
    gamma = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    status = _status(dev)
    binding.treewy_commit_verify(S, U_prev, K_prev, gamma_prev, parent_prev, accepted_prev,
                                 Q, K, V, alpha, beta, parent, O, U, gamma, status=status)
    if check:
        _raise_on(status)
    return O, U, gamma


def tree_attention(Kc, Vc, ctx, Qd, Kd, Vd, parent, check=False):
    """Softmax-attention verify of the draft tree over the committed cache: returns O
    [B, N, Hq, 256] float32."""
    import torch
    B, Hkv, T_max, d = Kc.shape
    N, Hq = Qd.shape[1], Qd.shape[2]
    dev = Kc.device
    O = torch.empty((B, N, Hq, d), dtype=torch.float32, device=dev)
    nbytes = binding.treewy_tree_attention_workspace(B, Hkv, Hq // Hkv if Hkv else 0, N, T_max)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    status = _status(dev)
    binding.treewy_tree_attention(Kc, Vc, ctx, Qd, Kd, Vd, parent, O, ws, status)
    if check:
        _raise_on(status)
    return O


def kv_commit(Kc, Vc, ctx, Kd, Vd, parent, accepted, check=False):
    """Append the accepted path to the cache (in place): returns the new lengths."""
    import torch
    ctx_out = torch.empty_like(ctx)
    status = _status(Kc.device)
    binding.treewy_kv_commit(Kc, Vc, ctx, ctx_out, Kd, Vd, parent, accepted, status)
    if check:
        _raise_on(status)
    return ctx_out
