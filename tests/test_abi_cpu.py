"""CPU-side checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU (no compute calls here)."""

import ctypes

import pytest

from linear_attention_speculative_head_amd import binding


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(binding.LIB_PATH):
        from linear_attention_speculative_head_amd import build
        build.build()
    return binding.lib()


def test_exports_every_header_symbol(lib):
    names = binding.header_symbols()
    assert set(names) == {"treewy_verify", "treewy_commit", "treewy_verify_snapshot",
                          "treewy_commit_snapshot", "treewy_commit_verify",
                          "treewy_commit_verify_deferred", "treewy_deferred_flush",
                          "treewy_tree_attention", "treewy_tree_attention_workspace",
                          "treewy_tree_attention_noalloc", "treewy_kv_commit",
                          "treewy_strerror", "treewy_version"}
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_strerror(lib):
    assert lib.treewy_version() == 4
    for code in range(8):
        assert lib.treewy_strerror(code) != b"unknown error code"
    assert lib.treewy_strerror(99) == b"unknown error code"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def verify_args(**kw):
    a = dict(S0=FAKE, Q=FAKE, K=FAKE, V=FAKE, alpha=FAKE, beta=FAKE, parent=FAKE, B=1, H=1, N=4,
             dt=binding.TREEWY_BF16, O=FAKE, U=FAKE, gamma=FAKE, anc=None, depth=None,
             status=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("bad", [dict(S0=None), dict(Q=None), dict(parent=None), dict(gamma=None),
                                 dict(N=0), dict(N=65), dict(B=0), dict(H=-1), dict(H=65537), dict(dt=7),
                                 dict(B=1 << 20, H=1 << 10)])
def test_verify_rejects(lib, bad):
    assert lib.treewy_verify(*verify_args(**bad)) == binding.TREEWY_EINVAL


@pytest.mark.parametrize("bad", [dict(S=None), dict(U=None), dict(accepted=None), dict(N=100),
                                 dict(dt=-1)])
def test_commit_rejects(lib, bad):
    a = dict(S=FAKE, U=FAKE, K=FAKE, gamma=FAKE, parent=FAKE, accepted=FAKE, B=2, H=2, N=8,
             dt=binding.TREEWY_F32, status=None, stream=None)
    a.update(bad)
    assert lib.treewy_commit(*a.values()) == binding.TREEWY_EINVAL


def test_snapshot_rejects(lib):
    assert lib.treewy_verify_snapshot(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 4, 1,
                                      FAKE, None, None, None) == binding.TREEWY_EINVAL
    assert lib.treewy_commit_snapshot(FAKE, FAKE, None, 1, 1, 4, None, None) == binding.TREEWY_EINVAL
    assert lib.treewy_commit_snapshot(FAKE, FAKE, FAKE, 1, 1, 0, None, None) == binding.TREEWY_EINVAL


def fused_args(**kw):
    """Arguments of treewy_commit_verify; distinct fake addresses far apart by default."""
    f = lambda x: ctypes.c_void_p(x)
    a = dict(S=f(0x10000000), U_prev=f(0x20000000), K_prev=f(0x30000000),
             gamma_prev=f(0x40000000), parent_prev=f(0x50000000), accepted_prev=f(0x60000000),
             Np=4, Q=f(0x70000000), K=f(0x80000000), V=f(0x90000000), alpha=f(0xa0000000),
             beta=f(0xb0000000), parent=f(0xc0000000), B=2, H=2, N=4, dt=binding.TREEWY_BF16,
             O=f(0xd0000000), U=f(0xe0000000), gamma=f(0xf0000000), anc=None, depth=None,
             status=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("bad", [dict(S=None), dict(U_prev=None), dict(K_prev=None),
                                 dict(gamma_prev=None), dict(parent_prev=None),
                                 dict(accepted_prev=None), dict(Q=None), dict(parent=None),
                                 dict(O=None), dict(U=None), dict(gamma=None),
                                 dict(Np=0), dict(Np=65), dict(N=0), dict(N=65), dict(B=0),
                                 dict(dt=3)])
def test_commit_verify_rejects(lib, bad):
    assert lib.treewy_commit_verify(*fused_args(**bad)) == binding.TREEWY_EINVAL


@pytest.mark.parametrize("which", ["U", "O", "gamma"])
def test_commit_verify_rejects_outputs_over_previous_factors(lib, which):
    """This step's outputs may not overlap the previous step's U, K or gamma."""
    # U_prev spans B*Np*H*128*4 = 8 KiB from 0x20000000; an output starting inside it overlaps
    inside = ctypes.c_void_p(0x20000000 + 4096)
    assert lib.treewy_commit_verify(*fused_args(**{which: inside})) == binding.TREEWY_EINVAL
    # K_prev (bf16, 4 KiB) and gamma_prev (64 B)
    assert lib.treewy_commit_verify(*fused_args(**{which: ctypes.c_void_p(0x30000000 + 100)})) \
        == binding.TREEWY_EINVAL
    assert lib.treewy_commit_verify(*fused_args(**{which: ctypes.c_void_p(0x40000000)})) \
        == binding.TREEWY_EINVAL


def deferred_args(**kw):
    f = lambda x: ctypes.c_void_p(x)
    a = dict(S=f(0x10000000), logU=f(0x11000000), logK=f(0x12000000), scale_in=f(0x13000000),
             scale_out=f(0x14000000), len_in=f(0x15000000), len_out=f(0x16000000), Lmax=8,
             U_prev=f(0x20000000), K_prev=f(0x30000000), gamma_prev=f(0x40000000),
             parent_prev=f(0x50000000), accepted_prev=f(0x60000000), Np=4, Q=f(0x70000000),
             K=f(0x80000000), V=f(0x90000000), alpha=f(0xa0000000), beta=f(0xb0000000),
             parent=f(0xc0000000), B=2, H=2, N=4, dt=binding.TREEWY_BF16, O=f(0xd0000000),
             U=f(0xe0000000), gamma=f(0xf0000000), anc=None, depth=None, status=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("bad", [dict(logU=None), dict(logK=None), dict(scale_in=None),
                                 dict(len_out=None), dict(U_prev=None), dict(Q=None),
                                 dict(Lmax=0), dict(Lmax=17), dict(N=65), dict(Np=65),
                                 dict(dt=binding.TREEWY_F32),
                                 dict(scale_out=ctypes.c_void_p(0x13000000)),   # = scale_in
                                 dict(len_out=ctypes.c_void_p(0x15000000)),     # = len_in
                                 dict(U=ctypes.c_void_p(0x20000000))])           # = U_prev
def test_commit_verify_deferred_rejects(lib, bad):
    assert lib.treewy_commit_verify_deferred(*deferred_args(**bad)) == binding.TREEWY_EINVAL


def test_deferred_flush_rejects(lib):
    f = lambda x: ctypes.c_void_p(x)
    ok = [f(0x10000000), f(0x11000000), f(0x12000000), f(0x13000000), f(0x14000000),
          f(0x15000000), f(0x16000000), 8, 2, 2, binding.TREEWY_BF16, None, None]
    for i, v in ((0, None), (1, None), (7, 0), (7, 17), (10, binding.TREEWY_F32),
                 (4, f(0x13000000)), (6, f(0x15000000))):
        args = list(ok)
        args[i] = v
        assert lib.treewy_deferred_flush(*args) == binding.TREEWY_EINVAL


def test_attention_workspace_size(lib):
    # (sequence, head, query block) triples x cache splits x one partial; the splits aim at about
    # 640 workgroups, whole 32-row tiles, with at least 256 rows each (8256 rows over 64
    # triples: 10 ranges of 832 rows)
    assert lib.treewy_tree_attention_workspace(2, 2, 8, 4, 8192) == 2 * 2 * 1 * 32 * (32 * 256 + 64) * 4
    assert lib.treewy_tree_attention_workspace(32, 2, 8, 4, 8256) == 32 * 2 * 1 * 10 * (32 * 256 + 64) * 4
    assert lib.treewy_tree_attention_workspace(512, 8, 8, 4, 8192) == 512 * 8 * 1 * 1 * (32 * 256 + 64) * 4
    assert lib.treewy_tree_attention_workspace(1, 1, 8, 16, 100) == 1 * 1 * 4 * 1 * (32 * 256 + 64) * 4
    assert lib.treewy_tree_attention_workspace(0, 2, 8, 4, 64) == 0
    assert lib.treewy_tree_attention_workspace(1, 2, 8, 65, 64) == 0


def attn_args(**kw):
    f = lambda x: ctypes.c_void_p(x)
    a = dict(Kc=f(0x1000000), Vc=f(0x2000000), ctx=f(0x3000000), T=64, Qd=f(0x4000000),
             Kd=f(0x5000000), Vd=f(0x6000000), parent=f(0x7000000), B=2, Hkv=2, G=8, N=4,
             O=f(0x8000000), ws=f(0x9000000), wsb=1 << 30, status=None, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("bad", [dict(Kc=None), dict(ctx=None), dict(Qd=None), dict(O=None),
                                 dict(ws=None), dict(wsb=16), dict(N=0), dict(N=65), dict(G=0),
                                 dict(Hkv=0), dict(T=0), dict(B=70000)])
def test_tree_attention_rejects(lib, bad):
    assert lib.treewy_tree_attention(*attn_args(**bad)) == binding.TREEWY_EINVAL


def noalloc_args(**kw):
    a = attn_args(**kw)
    del a[13:15]                        # no workspace pointer, no workspace size
    return a


@pytest.mark.parametrize("bad", [dict(Kc=None), dict(ctx=None), dict(Qd=None), dict(O=None),
                                 dict(N=0), dict(N=65), dict(G=0), dict(Hkv=0), dict(T=0),
                                 dict(B=70000)])
def test_tree_attention_noalloc_rejects(lib, bad):
    assert lib.treewy_tree_attention_noalloc(*noalloc_args(**bad)) == binding.TREEWY_EINVAL


def test_tree_attention_noalloc_rejects_sizes_past_its_array(lib):
    # the fixed device array holds 48 MiB of split partials; 4096 sequences x 8 KV heads need
    # one 33 KB partial each (1.08 GB), refused before anything is enqueued
    assert lib.treewy_tree_attention_workspace(4096, 8, 8, 4, 8192) > 48 << 20
    assert lib.treewy_tree_attention_noalloc(*noalloc_args(B=4096, Hkv=8, T=8192)) == \
        binding.TREEWY_ESCRATCH
    # the benchmark's shape fits: B = 32, 2 x 8 heads, 8256 cache rows
    assert lib.treewy_tree_attention_workspace(32, 2, 8, 4, 8256) <= 48 << 20


def test_kv_commit_rejects(lib):
    f = lambda x: ctypes.c_void_p(x)
    ok = [f(0x1000000), f(0x2000000), f(0x3000000), f(0x3100000), 64, f(0x5000000),
          f(0x6000000), f(0x7000000), f(0x7100000), 2, 2, 4, None, None]
    for i, v in ((0, None), (2, None), (3, f(0x3000000)), (4, 0), (11, 65), (8, None)):
        args = list(ok)
        args[i] = v
        assert lib.treewy_kv_commit(*args) == binding.TREEWY_EINVAL
