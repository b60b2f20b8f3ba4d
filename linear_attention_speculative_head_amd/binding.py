"""Thin Python binding of the TreeWY C ABI (include/treewy.h).

Argument marshalling only: torch tensors on the GPU are checked for device, dtype,
shape and contiguity, then their device pointers and torch's current HIP stream are
passed to the library.  Every step of the computation runs in the HIP kernels of
``libtreewy.so``; there is no fallback, and a missing library raises at once.

The functions carry the C names and take caller-owned output tensors, like the ABI.  With
``prepare=True`` the launch functions check and marshal their arguments once and return a
``PreparedCall`` that re-issues exactly that call (for launch loops).
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtreewy.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "treewy.h")

TREEWY_OK, TREEWY_EINVAL, TREEWY_EHIP, TREEWY_ETREE, TREEWY_EACCEPT, TREEWY_ELOG = 0, 1, 2, 3, 4, 5
TREEWY_ECTX = 6
TREEWY_ESCRATCH = 7
TREEWY_F32, TREEWY_BF16 = 0, 1
D = 128

_lib = None


class TreeWYError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().treewy_strerror(code).decode() if _lib is not None else str(code)
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


def lib():
    """Load libtreewy.so (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.treewy_verify.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, P, P, P, P, P, P]
        L.treewy_commit.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P]
        L.treewy_verify_snapshot.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, P, P, P]
        L.treewy_commit_snapshot.argtypes = [P, P, P, I, I, I, P, P]
        L.treewy_commit_verify.argtypes = ([P, P, P, P, P, P, I] + [P] * 6 + [I] * 4 +
                                           [P] * 7)
        L.treewy_commit_verify_deferred.argtypes = ([P] * 7 + [I] + [P] * 5 + [I] + [P] * 6 +
                                                    [I] * 4 + [P] * 7)
        L.treewy_deferred_flush.argtypes = [P] * 7 + [I] * 4 + [P, P]
        L.treewy_tree_attention.argtypes = ([P, P, P, I, P, P, P, P, I, I, I, I, P, P,
                                             ctypes.c_size_t, P, P])
        L.treewy_tree_attention_noalloc.argtypes = [P, P, P, I, P, P, P, P, I, I, I, I, P, P, P]
        L.treewy_tree_attention_workspace.argtypes = [I] * 5
        L.treewy_tree_attention_workspace.restype = ctypes.c_size_t
        L.treewy_kv_commit.argtypes = [P, P, P, P, I, P, P, P, P, I, I, I, P, P]
        L.treewy_strerror.argtypes = [I]
        L.treewy_strerror.restype = ctypes.c_char_p
        L.treewy_version.argtypes = []
        for f in ("treewy_verify", "treewy_commit", "treewy_verify_snapshot",
                  "treewy_commit_snapshot", "treewy_commit_verify",
                  "treewy_commit_verify_deferred", "treewy_deferred_flush",
                  "treewy_tree_attention", "treewy_tree_attention_noalloc", "treewy_kv_commit",
                  "treewy_version"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def header_symbols():
    """Function names declared in include/treewy.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(treewy_\w+)\s*\(", text, re.M)))


# ------------------------------------------------------------------ marshalling

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(t, name, shape, dtypes, device):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _qkv_dtype(Q):
    import torch
    if Q.dtype == torch.bfloat16:
        return TREEWY_BF16, (torch.bfloat16,)
    if Q.dtype == torch.float32:
        return TREEWY_F32, (torch.float32,)
    raise ValueError(f"Q/K/V dtype {Q.dtype} is not supported (float32 or bfloat16)")


def _rc(code: int, where: str):
    if code != TREEWY_OK:
        raise TreeWYError(code, where)


class PreparedCall:
    """A C ABI call whose arguments were checked and marshalled once: calling it re-issues
    exactly that call (the same tensors, sizes and stream), with the arguments already in
    ctypes form.  For launch loops whose host cost per launch should be the ctypes call
    alone; the library still checks every argument it can on each call."""

    __slots__ = ("fn", "args", "name")

    def __init__(self, fn, args, name):
        conv = []
        for t, a in zip(fn.argtypes, args):
            conv.append(a if a is None else t(a))
        self.fn, self.args, self.name = fn, tuple(conv), name

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != TREEWY_OK:
            raise TreeWYError(rc, self.name)


def _issue(name: str, args, prepare: bool):
    fn = getattr(lib(), name)
    if prepare:
        return PreparedCall(fn, args, name)
    _rc(fn(*args), name)
    return None


def treewy_verify(S0, Q, K, V, alpha, beta, parent, O, U, gamma,
                  anc_out=None, depth_out=None, status=None, stream=None, prepare=False):
    """Enqueue tree verification: fills O, U, gamma (and anc_out, depth_out if given)."""
    import torch
    B, N, H, _ = Q.shape
    dev = S0.device
    dt, qdt = _qkv_dtype(Q)
    f32 = (torch.float32,)
    _check(S0, "S0", (B, H, D, D), f32, dev)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check(t, n, (B, N, H, D), qdt, dev)
    for n, t in (("alpha", alpha), ("beta", beta), ("gamma", gamma)):
        _check(t, n, (B, N, H), f32, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(O, "O", (B, N, H, D), f32, dev)
    _check(U, "U", (B, N, H, D), f32, dev)
    _check(anc_out, "anc_out", (B, N), (torch.int64, torch.uint64), dev)
    _check(depth_out, "depth_out", (B, N), (torch.int32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    args = (_ptr(S0), _ptr(Q), _ptr(K), _ptr(V), _ptr(alpha), _ptr(beta), _ptr(parent),
            B, H, N, dt, _ptr(O), _ptr(U), _ptr(gamma), _ptr(anc_out), _ptr(depth_out),
            _ptr(status), _stream(stream))
    return _issue("treewy_verify", args, prepare)


def treewy_commit(S, U, K, gamma, parent, accepted, status=None, stream=None, prepare=False):
    """Enqueue the in-place commit of the accepted node's state into S."""
    import torch
    B, N, H, _ = K.shape
    dev = S.device
    dt, kdt = _qkv_dtype(K)
    f32 = (torch.float32,)
    _check(S, "S", (B, H, D, D), f32, dev)
    _check(U, "U", (B, N, H, D), f32, dev)
    _check(K, "K", (B, N, H, D), kdt, dev)
    _check(gamma, "gamma", (B, N, H), f32, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(accepted, "accepted", (B,), (torch.int32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    args = (_ptr(S), _ptr(U), _ptr(K), _ptr(gamma), _ptr(parent), _ptr(accepted), B, H, N,
            dt, _ptr(status), _stream(stream))
    return _issue("treewy_commit", args, prepare)


def treewy_commit_verify(S, U_prev, K_prev, gamma_prev, parent_prev, accepted_prev,
                         Q, K, V, alpha, beta, parent, O, U, gamma,
                         anc_out=None, depth_out=None, status=None, stream=None, prepare=False):
    """Enqueue the previous step's commit into S followed by this step's verify against the
    committed S (one kernel where the library fuses them)."""
    import torch
    B, N, H, _ = Q.shape
    Np = K_prev.shape[1]
    dev = S.device
    dt, qdt = _qkv_dtype(Q)
    f32 = (torch.float32,)
    _check(S, "S", (B, H, D, D), f32, dev)
    _check(U_prev, "U_prev", (B, Np, H, D), f32, dev)
    _check(K_prev, "K_prev", (B, Np, H, D), qdt, dev)
    _check(gamma_prev, "gamma_prev", (B, Np, H), f32, dev)
    _check(parent_prev, "parent_prev", (B, Np), (torch.int32,), dev)
    _check(accepted_prev, "accepted_prev", (B,), (torch.int32,), dev)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check(t, n, (B, N, H, D), qdt, dev)
    for n, t in (("alpha", alpha), ("beta", beta), ("gamma", gamma)):
        _check(t, n, (B, N, H), f32, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(O, "O", (B, N, H, D), f32, dev)
    _check(U, "U", (B, N, H, D), f32, dev)
    _check(anc_out, "anc_out", (B, N), (torch.int64, torch.uint64), dev)
    _check(depth_out, "depth_out", (B, N), (torch.int32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    args = (_ptr(S), _ptr(U_prev), _ptr(K_prev), _ptr(gamma_prev), _ptr(parent_prev),
            _ptr(accepted_prev), Np, _ptr(Q), _ptr(K), _ptr(V), _ptr(alpha), _ptr(beta),
            _ptr(parent), B, H, N, dt, _ptr(O), _ptr(U), _ptr(gamma), _ptr(anc_out),
            _ptr(depth_out), _ptr(status), _stream(stream))
    return _issue("treewy_commit_verify", args, prepare)


def _check_log(logU, logK, scale_in, scale_out, len_in, len_out, B, H, dev):
    import torch
    Lmax = logU.shape[2]
    _check(logU, "logU", (B, H, Lmax, D), (torch.float32,), dev)
    _check(logK, "logK", (B, H, Lmax, D), (torch.bfloat16,), dev)
    for n, t in (("scale_in", scale_in), ("scale_out", scale_out)):
        _check(t, n, (B, H), (torch.float32,), dev)
    for n, t in (("len_in", len_in), ("len_out", len_out)):
        _check(t, n, (B,), (torch.int32,), dev)
    return Lmax


def treewy_commit_verify_deferred(S, logU, logK, scale_in, scale_out, len_in, len_out,
                                  U_prev, K_prev, gamma_prev, parent_prev, accepted_prev,
                                  Q, K, V, alpha, beta, parent, O, U, gamma,
                                  anc_out=None, depth_out=None, status=None, stream=None,
                                  prepare=False):
    """Enqueue one step with the commit deferred into the log (logU, logK, header in/out)."""
    import torch
    B, N, H, _ = Q.shape
    Np = K_prev.shape[1]
    dev = S.device
    dt, qdt = _qkv_dtype(Q)
    f32 = (torch.float32,)
    _check(S, "S", (B, H, D, D), f32, dev)
    Lmax = _check_log(logU, logK, scale_in, scale_out, len_in, len_out, B, H, dev)
    _check(U_prev, "U_prev", (B, Np, H, D), f32, dev)
    _check(K_prev, "K_prev", (B, Np, H, D), qdt, dev)
    _check(gamma_prev, "gamma_prev", (B, Np, H), f32, dev)
    _check(parent_prev, "parent_prev", (B, Np), (torch.int32,), dev)
    _check(accepted_prev, "accepted_prev", (B,), (torch.int32,), dev)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check(t, n, (B, N, H, D), qdt, dev)
    for n, t in (("alpha", alpha), ("beta", beta), ("gamma", gamma)):
        _check(t, n, (B, N, H), f32, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(O, "O", (B, N, H, D), f32, dev)
    _check(U, "U", (B, N, H, D), f32, dev)
    _check(anc_out, "anc_out", (B, N), (torch.int64, torch.uint64), dev)
    _check(depth_out, "depth_out", (B, N), (torch.int32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    args = (_ptr(S), _ptr(logU), _ptr(logK), _ptr(scale_in), _ptr(scale_out), _ptr(len_in),
            _ptr(len_out), Lmax, _ptr(U_prev), _ptr(K_prev), _ptr(gamma_prev),
            _ptr(parent_prev), _ptr(accepted_prev), Np, _ptr(Q), _ptr(K), _ptr(V),
            _ptr(alpha), _ptr(beta), _ptr(parent), B, H, N, dt, _ptr(O), _ptr(U), _ptr(gamma),
            _ptr(anc_out), _ptr(depth_out), _ptr(status), _stream(stream))
    return _issue("treewy_commit_verify_deferred", args, prepare)


def treewy_deferred_flush(S, logU, logK, scale_in, scale_out, len_in, len_out, status=None,
                          stream=None):
    """Enqueue the write-back of the state a deferred-commit log stands for, emptying it."""
    import torch
    B, H = S.shape[:2]
    dev = S.device
    _check(S, "S", (B, H, D, D), (torch.float32,), dev)
    Lmax = _check_log(logU, logK, scale_in, scale_out, len_in, len_out, B, H, dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    rc = lib().treewy_deferred_flush(_ptr(S), _ptr(logU), _ptr(logK), _ptr(scale_in),
                                     _ptr(scale_out), _ptr(len_in), _ptr(len_out), Lmax, B, H,
                                     TREEWY_BF16, _ptr(status), _stream(stream))
    _rc(rc, "treewy_deferred_flush")


def treewy_tree_attention_workspace(B: int, Hkv: int, G: int, N: int, T_max: int) -> int:
    return int(lib().treewy_tree_attention_workspace(B, Hkv, G, N, T_max))


def treewy_tree_attention(Kc, Vc, ctx, Qd, Kd, Vd, parent, O, workspace, status=None,
                          stream=None):
    """Enqueue the tree-aware softmax-attention verify (bf16 inputs, head dim 256)."""
    import torch
    B, Hkv, T_max, _ = Kc.shape
    N, Hq = Qd.shape[1], Qd.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    G = Hq // Hkv
    dev = Kc.device
    bf = (torch.bfloat16,)
    _check(Kc, "Kc", (B, Hkv, T_max, 256), bf, dev)
    _check(Vc, "Vc", (B, Hkv, T_max, 256), bf, dev)
    _check(ctx, "ctx", (B,), (torch.int32,), dev)
    _check(Qd, "Qd", (B, N, Hq, 256), bf, dev)
    _check(Kd, "Kd", (B, N, Hkv, 256), bf, dev)
    _check(Vd, "Vd", (B, N, Hkv, 256), bf, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(O, "O", (B, N, Hq, 256), (torch.float32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    rc = lib().treewy_tree_attention(_ptr(Kc), _ptr(Vc), _ptr(ctx), T_max, _ptr(Qd), _ptr(Kd),
                                     _ptr(Vd), _ptr(parent), B, Hkv, G, N, _ptr(O),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _ptr(status), _stream(stream))
    _rc(rc, "treewy_tree_attention")


def treewy_tree_attention_noalloc(Kc, Vc, ctx, Qd, Kd, Vd, parent, O, status=None, stream=None):
    """treewy_tree_attention with its split partials in the library's fixed device array (no
    workspace argument; calls that overlap on one GPU race on that array)."""
    import torch
    B, Hkv, T_max, _ = Kc.shape
    N, Hq = Qd.shape[1], Qd.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    G = Hq // Hkv
    dev = Kc.device
    bf = (torch.bfloat16,)
    _check(Kc, "Kc", (B, Hkv, T_max, 256), bf, dev)
    _check(Vc, "Vc", (B, Hkv, T_max, 256), bf, dev)
    _check(ctx, "ctx", (B,), (torch.int32,), dev)
    _check(Qd, "Qd", (B, N, Hq, 256), bf, dev)
    _check(Kd, "Kd", (B, N, Hkv, 256), bf, dev)
    _check(Vd, "Vd", (B, N, Hkv, 256), bf, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(O, "O", (B, N, Hq, 256), (torch.float32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    rc = lib().treewy_tree_attention_noalloc(_ptr(Kc), _ptr(Vc), _ptr(ctx), T_max, _ptr(Qd),
                                             _ptr(Kd), _ptr(Vd), _ptr(parent), B, Hkv, G, N,
                                             _ptr(O), _ptr(status), _stream(stream))
    _rc(rc, "treewy_tree_attention_noalloc")


def treewy_kv_commit(Kc, Vc, ctx_in, ctx_out, Kd, Vd, parent, accepted, status=None, stream=None):
    """Enqueue the softmax layers' cache commit of the accepted path."""
    import torch
    B, Hkv, T_max, _ = Kc.shape
    N = Kd.shape[1]
    dev = Kc.device
    bf = (torch.bfloat16,)
    _check(Kc, "Kc", (B, Hkv, T_max, 256), bf, dev)
    _check(Vc, "Vc", (B, Hkv, T_max, 256), bf, dev)
    _check(ctx_in, "ctx_in", (B,), (torch.int32,), dev)
    _check(ctx_out, "ctx_out", (B,), (torch.int32,), dev)
    _check(Kd, "Kd", (B, N, Hkv, 256), bf, dev)
    _check(Vd, "Vd", (B, N, Hkv, 256), bf, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(accepted, "accepted", (B,), (torch.int32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    rc = lib().treewy_kv_commit(_ptr(Kc), _ptr(Vc), _ptr(ctx_in), _ptr(ctx_out), T_max,
                                _ptr(Kd), _ptr(Vd), _ptr(parent), _ptr(accepted), B, Hkv, N,
                                _ptr(status), _stream(stream))
    _rc(rc, "treewy_kv_commit")


def treewy_verify_snapshot(S0, Q, K, V, alpha, beta, parent, O, Snap, status=None, stream=None,
                           prepare=False):
    """Enqueue store-all verification: every node's state into Snap, outputs into O."""
    import torch
    B, N, H, _ = Q.shape
    dev = S0.device
    dt, qdt = _qkv_dtype(Q)
    f32 = (torch.float32,)
    _check(S0, "S0", (B, H, D, D), f32, dev)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check(t, n, (B, N, H, D), qdt, dev)
    for n, t in (("alpha", alpha), ("beta", beta)):
        _check(t, n, (B, N, H), f32, dev)
    _check(parent, "parent", (B, N), (torch.int32,), dev)
    _check(O, "O", (B, N, H, D), f32, dev)
    _check(Snap, "Snap", (B, H, N, D, D), f32, dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    args = (_ptr(S0), _ptr(Q), _ptr(K), _ptr(V), _ptr(alpha), _ptr(beta), _ptr(parent),
            B, H, N, dt, _ptr(O), _ptr(Snap), _ptr(status), _stream(stream))
    return _issue("treewy_verify_snapshot", args, prepare)


def treewy_commit_snapshot(S, Snap, accepted, status=None, stream=None, prepare=False):
    """Enqueue store-all rollback: S <- Snap[accepted] per sequence."""
    import torch
    B, H, N = Snap.shape[:3]
    dev = S.device
    f32 = (torch.float32,)
    _check(S, "S", (B, H, D, D), f32, dev)
    _check(Snap, "Snap", (B, H, N, D, D), f32, dev)
    _check(accepted, "accepted", (B,), (torch.int32,), dev)
    _check(status, "status", (1,), (torch.int32,), dev)
    args = (_ptr(S), _ptr(Snap), _ptr(accepted), B, H, N, _ptr(status), _stream(stream))
    return _issue("treewy_commit_snapshot", args, prepare)


def treewy_strerror(code: int) -> str:
    return lib().treewy_strerror(int(code)).decode()


def treewy_version() -> int:
    return lib().treewy_version()
