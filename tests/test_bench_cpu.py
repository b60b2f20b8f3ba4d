"""Host logic of the measurement: the benchmark's one-GPU contract and the algorithmic byte
counts it divides by, pinned to their closed forms on small hand-checked cases."""

import os
import subprocess
import sys

import numpy as np

from linear_attention_speculative_head_amd import accounting

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
D = 128


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_verify_bytes_closed_form():
    # per head: the state once (fp32 128 x 128), per node q/k/v rows, alpha, beta, O and U rows
    # (fp32), gamma
    for N in (1, 4, 16, 64):
        assert accounting.verify_bytes_per_head(N, 2) == 4 * D * D + N * (3 * D * 2 + 8 + 8 * D + 4)
        assert accounting.verify_bytes_per_head(N, 2) == 65536 + 1804 * N


def test_commit_bytes_closed_form():
    # nothing accepted (no path) touches nothing; otherwise the state read and written, plus
    # per path node a U row (fp32), a key row, a gamma
    assert accounting.commit_bytes_per_head(0, 2) == 0
    assert accounting.commit_bytes_per_head(1, 2) == 2 * 4 * D * D + (4 * D + 2 * D + 4)
    assert accounting.commit_bytes_per_head(3, 2) == 2 * 4 * D * D + 3 * (4 * D + 2 * D + 4)


def test_step_and_fused_bytes_on_a_chain():
    # one sequence, two heads, chain of 4; accepted node 2 (depth 3) and then nothing accepted
    parent = np.array([[-1, 0, 1, 2]], dtype=np.int32)
    H, N = 2, 4
    v = H * (65536 + 1804 * N) + 4 * N
    sep = accounting.step_bytes(parent, np.array([2], dtype=np.int32), H, N, 2)
    assert sep["verify"] == v
    assert sep["commit"] == 4 + 4 * N + H * (2 * 4 * D * D + 3 * (4 * D + 2 * D + 4))
    fused = accounting.fused_step_bytes(parent, np.array([2], dtype=np.int32), parent, H, 2)
    # the state is read once: the fused step saves exactly one state read per head (the
    # per-sequence words, both trees and the accepted node, are the same in total)
    assert fused["total"] == v + 4 * (N + N + 1) - 4 * N + H * (4 * D * D + 3 * (4 * D + 2 * D + 4))
    assert fused["total"] == sep["total"] - H * 4 * D * D
    none = accounting.fused_step_bytes(parent, np.array([-1], dtype=np.int32), parent, H, 2)
    assert none["total"] == v + 4 * (2 * N + 1) - 4 * N
    layers = accounting.fused_step_bytes(parent, np.array([2], dtype=np.int32), parent, H, 2,
                                         layers=3)
    assert layers["total"] == 3 * fused["total"]


def test_deferred_bytes_log_and_flush():
    # Lmax 4: a depth-3 path fits an empty log (appended, no state write); with 2 terms logged
    # it does not (state written, log emptied).  The state is read once (in base).
    parent = np.array([[-1, 0, 1, 2]], dtype=np.int32)
    H, N, row = 1, 4, 4 * D + 2 * D
    base = 65536 + 1804 * N + 4 * (2 * N + 2) + 8
    t, after = accounting.deferred_step_bytes(parent, np.array([2]), parent, H, 2,
                                              np.array([0]), 4)
    assert after.tolist() == [3]
    assert t == base + 3 * (row + 4) + 3 * row
    t, after = accounting.deferred_step_bytes(parent, np.array([2]), parent, H, 2,
                                              np.array([2]), 4)
    assert after.tolist() == [0]
    assert t == base + 2 * row + 3 * (row + 4) + 4 * D * D
    # above 16 nodes the log and the path share one staged chunk: 16 terms up to 48 nodes
    # (40-node chain: 6 logged + 3 fit, 14 + 3 do not), 8 above (64-node chain: 5 + 3 fit,
    # 6 + 3 do not)
    mid = np.array([list(range(-1, 39))], dtype=np.int32)
    t, after = accounting.deferred_step_bytes(mid, np.array([2]), mid, H, 2, np.array([6]), 16)
    assert after.tolist() == [9]
    t, after = accounting.deferred_step_bytes(mid, np.array([2]), mid, H, 2, np.array([14]), 16)
    assert after.tolist() == [0]
    big = np.array([list(range(-1, 63))], dtype=np.int32)
    t, after = accounting.deferred_step_bytes(big, np.array([2]), big, H, 2, np.array([6]), 16)
    assert after.tolist() == [0]
    t, after = accounting.deferred_step_bytes(big, np.array([2]), big, H, 2, np.array([5]), 16)
    assert after.tolist() == [8]


def test_attention_bytes_closed_form():
    # B = 32, 2 KV heads x 8 query heads, d = 256, 4 draft nodes, 8192 cached rows each:
    # 536 870 912 bytes of cache, 1 310 720 of draft q/k/v, 2 097 152 of O
    assert accounting.attention_call_bytes(np.full(32, 8192), 4, 2, 8) == 540278784
    # ragged prefixes count row by row; an empty cache leaves only the draft's I/O
    assert (accounting.attention_call_bytes([3, 0], 1, 1, 1)
            == 3 * 256 * 2 * 2 + 2 * 1 * 3 * 256 * 2 + 2 * 256 * 4)


def test_warmup_count():
    # an explicit --warmup is taken as given; the default is about a quarter second of steps at
    # 4 TB/s of algorithmic bytes, between 5 and 20000 steps
    import argparse
    sys.path.insert(0, ROOT)
    import bench
    given = argparse.Namespace(warmup=3)
    auto = argparse.Namespace(warmup=None)
    assert bench.auto_warmup(given, 131e6) == 3
    assert bench.auto_warmup(auto, 131e6) == 7634          # ceil(0.25 * 4e12 / 131e6)
    assert bench.auto_warmup(auto, 1e12) == 5
    assert bench.auto_warmup(auto, 1.0) == 20000


def test_source_digest_ignores_comments_only(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    # a traffic count stays attached to a kernel through comment and layout edits, not code
    # edits (string literals, with '//' inside, are code)
    a = 'int x = 1; // one\n/* two */ const char* s = "a // b";\n'
    b = 'int  x = 1;\n\nconst char* s = "a // b";  // another comment\n'
    c = 'int x = 2;\nconst char* s = "a // b";\n'
    d = 'int x = 1; const char* s = "a //  b";\n'
    h = []
    for i, t in enumerate((a, b, c, d)):
        f = tmp_path / f"k{i}.hip"
        f.write_text(t)
        h.append(bench.source_digest(str(f)))
    assert h[0] == h[1] and h[0] != h[2] and h[0] != h[3]
