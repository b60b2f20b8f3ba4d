"""TreeWY speculative tree verification + commit for Gated DeltaNet layers, on MI355X.

The compute path is ``libtreewy.so`` (HIP kernels for gfx950 behind the C ABI of
``include/treewy.h``); ``binding`` marshals torch tensors into it.  ``inputs`` draws
seeded synthetic workloads and ``accounting`` counts the algorithmic bytes.  ``api`` has
allocating forms of the calls (``verify``, ``commit``, ``commit_verify``, ``tree_attention``,
``kv_commit``).
"""

from .binding import (  # noqa: F401
    TREEWY_BF16, TREEWY_EACCEPT, TREEWY_ECTX, TREEWY_EHIP, TREEWY_EINVAL, TREEWY_ELOG,
    TREEWY_ESCRATCH, TREEWY_ETREE, TREEWY_F32, TREEWY_OK, TreeWYError, treewy_commit,
    treewy_commit_snapshot, treewy_commit_verify, treewy_commit_verify_deferred,
    treewy_deferred_flush, treewy_kv_commit, treewy_strerror, treewy_tree_attention,
    treewy_tree_attention_noalloc, treewy_tree_attention_workspace, treewy_verify,
    treewy_verify_snapshot, treewy_version,
)
from .api import commit, commit_verify, kv_commit, tree_attention, verify  # noqa: F401,E402
