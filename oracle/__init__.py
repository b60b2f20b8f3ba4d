"""CPU oracle for TreeWY verify/commit -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path never routes through it.

The oracle is the plain definition: Eq. (1) of "TreeWY: Speculative Verification for
Gated DeltaNet Hybrids" (§1) replayed token by token, in float64, along every
root-to-node path of the draft tree (§3 "Verifying a draft"), recording each node's
pseudo-value (§3 "Key rewrite") and, for commit, the replayed state at the accepted
node (§3 "Reconstruct on commit").  It lives in ``treewy_oracle.c`` (plain C, built
with gcc) and is driven from here through ctypes.

Every function is pinned by the tests in ``tests/test_oracle_pins.py`` (brute force,
the paper's closed form solved by a library triangular solver, the chain special
case, closed-form special cases and invariances).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "treewy_oracle.c")
LIB = os.path.join(HERE, "libtreewy_oracle.so")

OK, EINVAL, ETREE, EACCEPT = 0, 1, 3, 4

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_index_tree.argtypes = [I, P, P, P]
        lib.oracle_head.argtypes = [I, I, I, P, P, P, P, P, P, P, I, P, P, P, P]
        lib.oracle_batch.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I, P, P, P, P, P, I]
        lib.oracle_max_threads.argtypes = []
        for f in (lib.oracle_index_tree, lib.oracle_head, lib.oracle_batch, lib.oracle_max_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle error {code}")
        self.code = code


def index_tree(parent: np.ndarray):
    """depth [N] int32 and inclusive ancestor bitmask anc [N] uint64 of one tree."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    n = parent.shape[0]
    depth = np.zeros(n, dtype=np.int32)
    anc = np.zeros(n, dtype=np.uint64)
    rc = _load().oracle_index_tree(n, _p(parent), _p(depth), _p(anc))
    if rc:
        raise OracleError(rc)
    return depth, anc


def head(S0, q, k, v, alpha, beta, parent, accepted: int = -1):
    """One head in float64.  S0 [dv,dk], q/k [N,dk], v [N,dv], alpha/beta [N], parent [N].

    Returns dict(O [N,dv], U [N,dv], gamma [N], S_new [dv,dk]).
    """
    f = lambda x: np.ascontiguousarray(x, dtype=np.float64)
    S0, q, k, v, alpha, beta = map(f, (S0, q, k, v, alpha, beta))
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    n, dk = k.shape
    dv = v.shape[1]
    O = np.zeros((n, dv)); U = np.zeros((n, dv)); gamma = np.zeros(n)
    S_new = np.zeros((dv, dk))
    rc = _load().oracle_head(n, dk, dv, _p(S0), _p(q), _p(k), _p(v), _p(alpha), _p(beta),
                             _p(parent), int(accepted), _p(O), _p(U), _p(gamma), _p(S_new))
    if rc:
        raise OracleError(rc)
    return dict(O=O, U=U, gamma=gamma, S_new=S_new)


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def batch(layer, parent, accepted=None, heads: Optional[Sequence] = None,
          threads: Optional[int] = None, commit: bool = True):
    """Run the oracle over a layer in the device layout (see ``inputs``).

    ``heads``: optional list of (b, h) pairs; default every head in (b, h) order.
    Returns dict(O, U [n,N,dv], gamma [n,N], S_new [n,dv,dk] or None) in float64.
    """
    S0, q, k, v, al, be = (np.ascontiguousarray(x, dtype=np.float32) for x in
                           (layer.S0, layer.q, layer.k, layer.v, layer.alpha, layer.beta))
    B, H, dv, dk = S0.shape
    N = q.shape[1]
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    acc = None if accepted is None else np.ascontiguousarray(accepted, dtype=np.int32)
    sel = None
    n = B * H
    if heads is not None:
        sel = np.ascontiguousarray(np.asarray(heads, dtype=np.int32).reshape(-1, 2))
        n = sel.shape[0]
    O = np.zeros((n, N, dv)); U = np.zeros((n, N, dv)); gamma = np.zeros((n, N))
    S_new = np.zeros((n, dv, dk)) if commit else None
    rc = _load().oracle_batch(B, H, N, dk, dv, _p(S0), _p(q), _p(k), _p(v), _p(al), _p(be),
                              _p(parent), _p(acc), n, _p(sel), _p(O), _p(U), _p(gamma),
                              _p(S_new), int(threads or default_threads()))
    if rc:
        raise OracleError(rc)
    return dict(O=O, U=U, gamma=gamma, S_new=S_new)
