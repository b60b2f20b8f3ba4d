"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, run on the CPU.

* The oracle (oracle/treewy_oracle.c) is rebuilt by gcc with -fsanitize=address,undefined
  and driven in a child process (the sanitizer runtimes preloaded) over small problems,
  edge-case trees and malformed trees; its outputs must equal the normal build's.
* The HIP library is rebuilt with the sanitizers on its host code only (-Xarch_host before
  each -fsanitize=; the device code is compiled as usual but never runs here), and the
  C-ABI argument checks of tests/test_abi_cpu.py run against it in a child process with
  clang's ASan runtime preloaded.

Any sanitizer report aborts the child (halt_on_error), which fails the test.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _gcc_runtime(name: str) -> str:
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                       check=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.fail(f"gcc has no {name}")
    return p


def _child(code: str, preload: str, timeout: int = 600) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    env["PYTHONPATH"] = os.pathsep.join([ROOT, TESTS, env.get("PYTHONPATH", "")])
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


# ------------------------------------------------------------------------------ the oracle

def _trees():
    """Edge-case and malformed trees: (name, parent array)."""
    rng = np.random.default_rng(7)
    wide = np.array([-1] + [int(rng.integers(0, t)) for t in range(1, 64)], dtype=np.int32)
    return [
        ("single", np.array([-1], dtype=np.int32)),
        ("chain64", np.arange(-1, 63, dtype=np.int32)),
        ("star64", np.array([-1] + [0] * 63, dtype=np.int32)),
        ("forest", np.array([-1, -1, 0, 1, 2, 3], dtype=np.int32)),
        ("wide64", wide),
        ("forward_ref", np.array([-1, 2, 0], dtype=np.int32)),   # parent after the node
        ("self_ref", np.array([-1, 1], dtype=np.int32)),
        ("out_of_range", np.array([-1, 0, 9], dtype=np.int32)),
        ("below_minus_one", np.array([-1, -2], dtype=np.int32)),
    ]


def oracle_outputs(lib_path: str) -> dict:
    """Every oracle entry point on small inputs, with the library at lib_path."""
    import oracle
    from linear_attention_speculative_head_amd import inputs
    oracle.LIB = lib_path
    oracle._lib = None
    out = {}
    for name, par in _trees():
        try:
            d, a = oracle.index_tree(par)
            out[f"tree_{name}_depth"] = d
            out[f"tree_{name}_anc"] = a
        except oracle.OracleError as e:
            out[f"tree_{name}_err"] = np.array([e.code])
    problems = [("cfg0", inputs.make_problem(0, layers=1)),
                ("chain", inputs.make_tree_shape((1, 1, 1), B=2, H=2)),
                ("full39", inputs.make_tree_shape((3, 3, 3), B=2, H=2))]
    for name, P in problems:
        L = P.layers[0]
        heads = [(b, h) for b in range(P.B) for h in range(P.H)]
        r = oracle.batch(L, P.parent, P.accepted, heads=heads, commit=True)
        for k in ("O", "U", "gamma", "S_new"):
            out[f"{name}_{k}"] = np.asarray(r[k])
        # one head through the single-head entry point, with and without a commit
        f = lambda x: np.asarray(x[0, ..., 0, :] if x.ndim == 4 else x[0, ..., 0], dtype=np.float64)
        o1 = oracle.head(L.S0[0, 0].astype(np.float64), f(L.q), f(L.k), f(L.v),
                         L.alpha[0, :, 0].astype(np.float64), L.beta[0, :, 0].astype(np.float64),
                         P.parent[0], int(P.accepted[0]))
        for k, v in o1.items():
            out[f"{name}_head_{k}"] = np.asarray(v)
    return out


def _save_oracle_outputs(lib_path: str, npz: str) -> None:
    np.savez(npz, **oracle_outputs(lib_path))


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitizers")


def test_oracle_under_asan_ubsan(san_dir):
    import oracle
    src = os.path.join(ROOT, "oracle", "treewy_oracle.c")
    lib = str(san_dir / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", src, "-o", lib, "-lm"], check=True)
    npz = str(san_dir / "oracle_san.npz")
    preload = ":".join([_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")])
    r = _child("import test_sanitizers_cpu as t; "
               f"t._save_oracle_outputs({lib!r}, {npz!r})", preload)
    assert r.returncode == 0, f"sanitized oracle run failed:\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    got = np.load(npz)
    ref = oracle_outputs(oracle.build(force=False))
    assert sorted(got.files) == sorted(ref), "different result sets"
    for k in ref:
        a, b = got[k], ref[k]
        assert a.shape == b.shape and a.dtype == b.dtype, k
        if a.dtype.kind == "f":
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-300, err_msg=k)
        else:
            assert np.array_equal(a, b), k


# ------------------------------------------------------------------ the C-ABI host checks

def _clang_asan() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.fail("clang's ASan runtime is missing")
    return hits[-1]


def test_abi_host_checks_under_asan_ubsan(san_dir):
    from linear_attention_speculative_head_amd import build as B
    csrc = B.CSRC
    lib = str(san_dir / "libtreewy_san.so")
    hipcc = shutil.which(B.HIPCC) or B.HIPCC
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           *[os.path.join(csrc, s) for s in B.SOURCES], "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    code = ("import sys; from linear_attention_speculative_head_amd import binding; "
            f"binding.LIB_PATH = {lib!r}; import pytest; "
            f"sys.exit(pytest.main([{os.path.join(TESTS, 'test_abi_cpu.py')!r}, '-q', "
            "'-p', 'no:cacheprovider', '-m', 'not gpu']))")
    r = _child(code, _clang_asan())
    assert r.returncode == 0, f"ABI checks under the sanitizers failed:\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert "passed" in r.stdout and "runtime error" not in r.stderr, r.stdout[-2000:] + r.stderr[-2000:]
