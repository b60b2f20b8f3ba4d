#!/usr/bin/env python3
"""Benchmark of the TreeWY hot path on one MI355X: tree verify + commit.

A step is one pass of the whole path over one batch, on inputs already resident in HBM.
By default it is the steady state of decoding: one treewy_commit_verify launch per layer,
which commits the previous step's accepted node into the state and verifies this step's
draft tree against it (the state is read and written once).  ``--separate`` times the same
work as treewy_verify for every layer then treewy_commit for every layer; the default run
also times that beside the fused step and reports it under ``separate_calls``.
``--snapshot`` times the store-all comparison scheme instead.

Steps cycle through a pool of independently drawn instances whose total footprint exceeds
the 256 MB Infinity Cache, so the state stream is served from HBM rather than from the
cache.  Every instance's "previous step" is its own last one (same tree and accepted node).

Prints one JSON line: throughput in draft-nodes*heads per second, the roofline of the
dominant kernel (algorithmic bytes per launch over its mean launch time: HIP events on the
launch stream around the timed region, over the launches in it, where a step is one launch
per layer; otherwise events around each launch in a second pass of the same steps), and the
CPU oracle's rate on a bounded sample of the same workload as a reported baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published

# HBM byte counts per launch taken with rocprofv3 (FETCH_SIZE, WRITE_SIZE, scaled by the same
# counters on a plain copy of known size), per workload; used while the kernel source is the
# one they were taken on
TRAFFIC_FILES = {0: "profiles/traffic_fp32_chain4_b1h1.json",
                 1: "profiles/traffic_chain4_b32h32.json",
                 2: "profiles/traffic_tree16_b64h32.json",
                 3: "profiles/traffic_tree64_b128h32_l30.json",
                 4: "profiles/traffic_tree32_b256h64.json",
                 "attention-8192": "profiles/traffic_attention_b32_chain4_ctx8192.json",
                 "attention-32768": "profiles/traffic_attention_b32_chain4_ctx32768.json"}


WARMUP_S = 0.25           # default warm-up: about this long ...
WARMUP_RATE = 4.0e12      # ... estimated at this many algorithmic bytes per second
WARMUP_MAX = 20000        # launch-bound workloads: at most this many steps


def auto_warmup(args, step_bytes):
    """The warm-up step count: --warmup when given, else about WARMUP_S seconds of steps of
    `step_bytes` algorithmic bytes at WARMUP_RATE (at least 5, at most WARMUP_MAX).  On
    MI355X kernel durations fall over the first tens of milliseconds of sustained launches
    (a 750 us step measured 840 us as the 2nd launch and 650 us from the 60th on), so a
    count of a few steps would time that ramp instead of the steady state."""
    if args.warmup is not None:
        return args.warmup
    return min(WARMUP_MAX, max(5, math.ceil(WARMUP_S * WARMUP_RATE / max(step_bytes, 1.0))))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as take about "
                         f"{WARMUP_S} s at {WARMUP_RATE / 1e12:.0f} TB/s of the workload's "
                         "algorithmic bytes, at least 5: kernel durations fall over the first "
                         "tens of milliseconds of sustained launches)")
    ap.add_argument("--config", type=int, default=3,
                    help="workload 0..4 (default 3: B128 x H32, 64-node trees, 30 layers, the "
                         "largest one-GPU workload)")
    ap.add_argument("--tree", type=str, default=None,
                    help="instead of a config: every sequence drafts the full tree W1,W2,W3 "
                         "(B x H of config 1, accepted node uniform)")
    ap.add_argument("--sweep", action="store_true",
                    help="every full-tree shape of the paper's Tables 2 and 4 (N = 3..39) in "
                         "turn; one JSON line per shape")
    ap.add_argument("--pool-gib", type=float, default=1.25,
                    help="minimum device footprint of the rotating instance pool")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--deferred", type=int, default=0, metavar="LMAX",
                    help="steady state of the deferred commit with a log of LMAX terms "
                         "(treewy_commit_verify_deferred); 0 = off")
    ap.add_argument("--attention", type=int, default=0, metavar="CTX",
                    help="time the tree-aware softmax-attention verify instead (B=32, 2 KV heads "
                         "x 8 query heads, head dim 256, the config-1 chain, CTX committed rows)")
    ap.add_argument("--separate", action="store_true",
                    help="time treewy_verify then treewy_commit (two launches per layer)")
    ap.add_argument("--snapshot", action="store_true",
                    help="time the store-all comparison path instead of TreeWY")
    ap.add_argument("--with-snapshot", type=int, default=None, choices=(0, 1),
                    help="also time the store-all comparison path on the same inputs in the "
                         "same run and report it under 'snapshot' (default: on for config 4)")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="size of the plain device copy timed in the same run (0 = skip)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each instance's step as a captured HIP graph (the fused step: "
                         "one graph per parity of its alternating per-step buffers)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a kernel of "
                         "known traffic, used to scale HBM byte counters taken with rocprofv3)")
    return ap.parse_args()


class Workload:
    """What a run measures: sizes, a description and a seeded draw per instance."""

    def __init__(self, args):
        from linear_attention_speculative_head_amd import inputs
        if args.tree is not None:
            widths = tuple(int(w) for w in args.tree.split(","))
            c1 = inputs.CONFIGS[1]
            self.B, self.H, self.nl, self.dtype = c1["B"], c1["H"], 1, "bf16"
            self.N = len(inputs.full_tree(widths))
            self.name = f"tree {','.join(map(str, widths))}"
            self.desc = (f"B{self.B} x H{self.H}, full tree {widths} (N={self.N}), bf16 q/k/v, "
                         f"accepted uniform")
            self.draw = lambda i: inputs.make_tree_shape(widths, instance=i, B=self.B, H=self.H)
            self.rotate = True
            self.traffic_key = None
        else:
            c = inputs.CONFIGS[args.config]
            self.B, self.H, self.N, self.nl, self.dtype = c["B"], c["H"], c["N"], c["layers"], c["dtype"]
            self.name = f"config {args.config}"
            self.desc = c["desc"]
            self.draw = lambda i: inputs.make_problem(args.config, instance=i)
            self.rotate = args.config != 0
            self.traffic_key = args.config


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); every "
              "(sequence, head) is independent, so N GPUs would each run this same "
              "single-GPU pass on their share.", file=sys.stderr)
        sys.exit(2)
    assert sum([bool(args.separate), bool(args.snapshot), bool(args.deferred)]) <= 1, \
        "--separate, --snapshot and --deferred are exclusive"
    mode = ("snapshot" if args.snapshot else "separate" if args.separate else
            "deferred" if args.deferred else "fused")
    assert not (args.graph and mode == "deferred"), "--graph does not apply to --deferred"

    import torch
    from linear_attention_speculative_head_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()
    if args.attention:
        print(json.dumps(run_attention(args)), flush=True)
        return
    if args.sweep:
        rows = []
        for w in inputs.PAPER_TREE_SHAPES:
            args.tree = ",".join(map(str, w))
            line = run(args, mode, Workload(args))
            print(json.dumps(line), flush=True)
            rows.append((w, line))
        log("[bench] sweep: shape, N, fused us/step, separate us/step (verify + commit us), "
            "fused GB/s")
        for w, l in rows:
            sep = l["separate_calls"] or {}
            k = sep.get("kernels_us", {})
            log(f"[bench]   {w} N={l['config']['N']:2d}: {l['ms_per_step'] * 1e3:7.1f} "
                f"{sep.get('ms_per_step', float('nan')) * 1e3:7.1f} "
                f"({k.get('treewy_verify', float('nan')):.1f} + {k.get('treewy_commit', float('nan')):.1f}) "
                f"{l['roofline']['achieved']:.0f}")
        return
    print(json.dumps(run(args, mode, Workload(args))), flush=True)


def run(args, mode, wl):
    """Measure one workload; returns the JSON line as a dict."""
    import torch
    from linear_attention_speculative_head_amd import accounting, binding, device

    B, H, N, nl, dtype = wl.B, wl.H, wl.N, wl.nl, wl.dtype
    elem = 2 if dtype == "bf16" else 4

    # ---- rotating pool of instances (each: all layers of the workload)
    with_snap = mode == "snapshot" or (mode == "fused" and bool(
        args.with_snapshot if args.with_snapshot is not None else getattr(args, "config", None) == 4
        and args.tree is None))
    per_layer = (B * H * 128 * 128 * 4 + 3 * B * N * H * 128 * elem + 2 * B * N * H * 128 * 4
                 + (2 * B * N * H * 128 * 4 if mode in ("fused", "deferred") else 0)
                 + (B * H * args.deferred * 128 * 6 if mode == "deferred" else 0))
    n_inst = max(1, math.ceil(args.pool_gib * 2 ** 30 / (per_layer * nl))) if wl.rotate else 1
    n_inst = min(n_inst, 32)
    log(f"[bench] {wl.name}: {wl.desc}; {mode} path; {n_inst} instance(s) of "
        f"{nl} layer(s), {per_layer * nl * n_inst / 2 ** 30:.2f} GiB on device")
    t0 = time.time()
    pool = []
    first = None
    for i in range(n_inst):
        P = wl.draw(i)
        parent, accepted = device.upload_tree(P)
        layers = []
        for L in P.layers:
            dl = device.upload_layer(L, dtype)
            out = device.alloc_outputs(B, H, N)
            extra = None
            if mode in ("fused", "deferred"):  # second set of per-step outputs, alternated
                extra = device.alloc_outputs(B, H, N)
            dlog = device.alloc_log(B, H, args.deferred) if mode == "deferred" else None
            layers.append((dl, out, extra, dlog))
        nbytes = {
            "fused": accounting.fused_step_bytes(P.parent, P.accepted, P.parent, H, elem,
                                                 layers=nl),
            "separate": accounting.step_bytes(P.parent, P.accepted, H, N, elem, layers=nl),
            "snapshot": accounting.snapshot_step_bytes(P.parent, P.accepted, H, N, elem,
                                                       layers=nl),
        }
        if i == 0:
            W = auto_warmup(args, nbytes["fused" if mode == "deferred" else mode]["total"])
        seq = []
        if mode == "deferred":
            # the log evolves the same way on every call of this instance: its bytes per call,
            # worked out here so that no host work sits between the timed launches
            lens = np.zeros(B, dtype=np.int64)
            calls = math.ceil((W + 2 * args.steps) / n_inst) + 1
            for _ in range(calls):
                nb, lens = accounting.deferred_step_bytes(P.parent, P.accepted, P.parent, H,
                                                          elem, lens, args.deferred)
                seq.append(nb * nl)
        pool.append(dict(parent=parent, accepted=accepted, layers=layers, flip=0, bytes=nbytes,
                         dseq=seq, calls=0))
        if i == 0:
            first = P
    # the store-all scheme's snapshots of one layer (every node's state), shared by all layers
    # and instances: its verify and rollback run layer by layer
    snap = torch.empty((B, H, N, 128, 128), device="cuda") if with_snap else None
    torch.cuda.synchronize()
    log(f"[bench] inputs drawn and uploaded in {time.time() - t0:.1f} s")

    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if mode in ("fused", "deferred"):
        # the previous step of every instance: a plain verify, so that its U and gamma exist
        for x in pool:
            for dl, out, _, _ in x["layers"]:
                binding.treewy_verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, x["parent"],
                                      out.O, out.U, out.gamma, status=status)
        torch.cuda.synchronize()

    # Every launch of the timed loops is prepared once (arguments checked and marshalled), so
    # that a launch costs the host one ctypes call; under --graph the calls stay unprepared,
    # since a capture needs them issued on its own stream.
    prep = not args.graph

    def prepare_instance(x):
        c = {"fused": [], "deferred": [], "verify": [], "commit": [], "snap_v": [], "snap_c": []}
        for dl, o0, o1, dlog in x["layers"]:
            if mode == "fused":
                c["fused"].append([binding.treewy_commit_verify(
                    dl.S0, prev.U, dl.K, prev.gamma, x["parent"], x["accepted"], dl.Q, dl.K,
                    dl.V, dl.alpha, dl.beta, x["parent"], cur.O, cur.U, cur.gamma,
                    status=status, prepare=True) for prev, cur in ((o0, o1), (o1, o0))])
            if mode == "deferred":
                pair = []
                for prev, cur in ((o0, o1), (o1, o0)):
                    si, so, li, lo = dlog.headers()
                    pair.append(binding.treewy_commit_verify_deferred(
                        dl.S0, dlog.U, dlog.K, si, so, li, lo, prev.U, dl.K, prev.gamma,
                        x["parent"], x["accepted"], dl.Q, dl.K, dl.V, dl.alpha, dl.beta,
                        x["parent"], cur.O, cur.U, cur.gamma, status=status, prepare=True))
                    dlog.flip()
                c["deferred"].append(pair)
            if mode in ("fused", "separate"):
                c["verify"].append(binding.treewy_verify(
                    dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, x["parent"], o0.O, o0.U,
                    o0.gamma, status=status, prepare=True))
                c["commit"].append(binding.treewy_commit(
                    dl.S0, o0.U, dl.K, o0.gamma, x["parent"], x["accepted"], status,
                    prepare=True))
            if snap is not None:
                c["snap_v"].append(binding.treewy_verify_snapshot(
                    dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, x["parent"], o0.O, snap, status,
                    prepare=True))
                c["snap_c"].append(binding.treewy_commit_snapshot(
                    dl.S0, snap, x["accepted"], status, prepare=True))
        return c

    if prep:
        for x in pool:
            x["prepared"] = prepare_instance(x)

    def fused_step(x, ev=None):
        for j, (dl, o0, o1, _) in enumerate(x["layers"]):
            prev, cur = (o0, o1) if x["flip"] == 0 else (o1, o0)
            if ev is not None:
                ev[0][j].record()
            if prep:
                x["prepared"]["fused"][j][x["flip"]]()
            else:
                binding.treewy_commit_verify(dl.S0, prev.U, dl.K, prev.gamma, x["parent"],
                                             x["accepted"], dl.Q, dl.K, dl.V, dl.alpha, dl.beta,
                                             x["parent"], cur.O, cur.U, cur.gamma, status=status)
            if ev is not None:
                ev[1][j].record()
        x["flip"] ^= 1
        return x["bytes"]["fused"]["total"]

    def deferred_step(x, ev=None):
        nb = x["dseq"][x["calls"]]
        x["calls"] += 1
        for j, (dl, o0, o1, dlog) in enumerate(x["layers"]):
            # the prepared call of this parity reads and writes this parity's log header
            if ev is not None:
                ev[0][j].record()
            x["prepared"]["deferred"][j][x["flip"]]()
            if ev is not None:
                ev[1][j].record()
            dlog.flip()
        x["flip"] ^= 1
        return nb

    def two_call_step(x, ev=None):
        # verify for every layer, then commit for every layer
        for j, (dl, out, extra, _) in enumerate(x["layers"]):
            if ev is not None:
                ev[0][j].record()
            if prep:
                x["prepared"]["verify"][j]()
            else:
                binding.treewy_verify(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta, x["parent"],
                                      out.O, out.U, out.gamma, status=status)
            if ev is not None:
                ev[1][j].record()
        for j, (dl, out, extra, _) in enumerate(x["layers"]):
            if ev is not None:
                ev[2][j].record()
            if prep:
                x["prepared"]["commit"][j]()
            else:
                binding.treewy_commit(dl.S0, out.U, dl.K, out.gamma, x["parent"],
                                      x["accepted"], status)
            if ev is not None:
                ev[3][j].record()
        return x["bytes"]["separate"]["total"]

    def snapshot_step(x, ev=None):
        # per layer: every node's state written, then the accepted node's copied back
        for j, (dl, out, _, _) in enumerate(x["layers"]):
            if ev is not None:
                ev[0][j].record()
            if prep:
                x["prepared"]["snap_v"][j]()
            else:
                binding.treewy_verify_snapshot(dl.S0, dl.Q, dl.K, dl.V, dl.alpha, dl.beta,
                                               x["parent"], out.O, snap, status)
            if ev is not None:
                ev[1][j].record()
                ev[2][j].record()
            if prep:
                x["prepared"]["snap_c"][j]()
            else:
                binding.treewy_commit_snapshot(dl.S0, snap, x["accepted"], status)
            if ev is not None:
                ev[3][j].record()
        return x["bytes"]["snapshot"]["total"]

    def step_fn(m):
        return {"fused": fused_step, "deferred": deferred_step, "separate": two_call_step,
                "snapshot": snapshot_step}[m]

    K = args.steps

    def measure(m, graphs=None):
        """Warm-up, then exactly K timed steps with nothing else on the stream.  Where a step
        is one launch per layer (fused, deferred), the mean launch duration is the HIP-event
        time of that region over its launches.  Otherwise the same K steps run again with HIP
        events around every launch, for each kernel's duration."""
        fn = step_fn(m)

        def run(i, ev=None):
            if graphs is not None and ev is None:
                if m == "fused":              # one graph per parity of the alternating buffers
                    graphs[i][pool[i]["flip"]].replay()
                    pool[i]["flip"] ^= 1
                else:
                    graphs[i].replay()
                return pool[i]["bytes"][m]["total"]
            return fn(pool[i], ev)

        for s in range(W):
            run(s % n_inst)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"device status {int(status.item())}"
        torch.cuda.synchronize()
        timed_bytes = 0
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start = time.perf_counter()
        r0.record()
        for s in range(K):
            timed_bytes += run((W + s) % n_inst)
        r1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        region_ms = r0.elapsed_time(r1)
        assert int(status.item()) == 0, f"device status {int(status.item())}"
        used = [(W + s) % n_inst for s in range(K)]
        step_bytes = timed_bytes / K
        kern = {}
        if m in ("fused", "deferred"):
            name = "treewy_commit_verify" if m == "fused" else "treewy_commit_verify_deferred"
            kern[name] = (step_bytes / nl, region_ms / (K * nl))
            return wall, kern, step_bytes, region_ms
        events = [[[torch.cuda.Event(enable_timing=True) for _ in range(nl)] for _ in range(4)]
                  for _ in range(K)]
        torch.cuda.synchronize()
        for s in range(K):
            run((W + s) % n_inst, events[s])
        torch.cuda.synchronize()
        names = (["treewy_verify_snapshot", "treewy_commit_snapshot"] if m == "snapshot" else
                 ["treewy_verify", "treewy_commit"])
        for k, (name, key) in enumerate(zip(names, ["verify", "commit"])):
            ms = np.array([[events[s][2 * k][j].elapsed_time(events[s][2 * k + 1][j])
                            for j in range(nl)] for s in range(K)])
            nbytes = np.mean([pool[i]["bytes"][m][key] for i in used]) / nl
            kern[name] = (nbytes, ms.mean())
        return wall, kern, step_bytes, region_ms

    graphs = None
    if args.graph:
        # one graph per instance: verify for every layer, then commit for every layer
        graphs = []
        fn = step_fn(mode)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n_inst):           # warm the launch path outside capture
                fn(pool[i])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i in range(n_inst):
            if mode == "fused":
                # capture both parities; fused_step flips the instance's buffers each call
                pool[i]["flip"] = 0
                pair = []
                for _ in range(2):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fn(pool[i])
                    pair.append(g)
                graphs.append(pair)
            else:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn(pool[i])
                graphs.append(g)
        torch.cuda.synchronize()

    wall, kern, step_bytes, region_ms = measure(mode, graphs)
    ms_step = wall * 1e3 / K
    nodes_heads = B * H * N * nl
    value = nodes_heads * K / wall
    dom = max(kern, key=lambda k: kern[k][1])
    d_bytes, d_ms = kern[dom]
    achieved = d_bytes / (d_ms * 1e-3) / 1e9
    log(f"[bench] {mode}: {ms_step * 1e3:.1f} us/step; " + ", ".join(
        f"{n} {t * 1e3:.1f} us per launch ({b / (t * 1e-3) / 1e9:.0f} GB/s)"
        for n, (b, t) in kern.items())
        + f"; step {step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s algorithmic")

    separate = None
    if mode == "fused":
        # the same work as two launches per layer, for comparison
        w2, k2, b2, _ = measure("separate")
        separate = {"ms_per_step": w2 * 1e3 / K, "value": nodes_heads * K / w2,
                    "hbm_frac_step": b2 / (w2 / K) / 1e9 / HBM_PEAK_GBS,
                    "kernels_us": {n: t * 1e3 for n, (b, t) in k2.items()}}
        log(f"[bench] separate calls: {w2 * 1e6 / K:.1f} us/step; " + ", ".join(
            f"{n} {t * 1e3:.1f} us" for n, (b, t) in k2.items()))

    snapshot = None
    if mode == "fused" and with_snap:
        # the store-all comparison on the same inputs, in the same run
        w3, k3, b3, _ = measure("snapshot")
        snapshot = {"ms_per_step": w3 * 1e3 / K, "value": nodes_heads * K / w3,
                    "bytes_per_step": b3, "achieved_gbs": b3 / (w3 / K) / 1e9,
                    "hbm_frac_step": b3 / (w3 / K) / 1e9 / HBM_PEAK_GBS,
                    "time_vs_treewy": (w3 / K) / (wall / K),
                    "bytes_vs_treewy": b3 / step_bytes,
                    "kernels_us": {n: t * 1e3 for n, (b, t) in k3.items()},
                    "kernels_gbs": {n: b / (t * 1e-3) / 1e9 for n, (b, t) in k3.items()}}
        log(f"[bench] store-all snapshots: {w3 * 1e6 / K:.1f} us/step "
            f"({snapshot['time_vs_treewy']:.1f}x TreeWY's time, "
            f"{snapshot['bytes_vs_treewy']:.1f}x its bytes); " + ", ".join(
                f"{n} {t * 1e3:.1f} us ({b / (t * 1e-3) / 1e9:.0f} GB/s)"
                for n, (b, t) in k3.items()))
    snap = None          # (the snapshot step's closure holds the buffer)

    copy_gbs = copy_bandwidth(args.copy_gib) if args.copy_gib > 0 else None
    if copy_gbs:
        log(f"[bench] plain device copy of {args.copy_gib:g} GiB: {copy_gbs:.0f} GB/s "
            f"(bytes read + written)")

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)

    cpu = None
    if args.cpu_seconds > 0 and not args.sweep:
        cpu = cpu_baseline(first, args.cpu_seconds)
        log(f"[bench] cpu baseline (oracle): {cpu['value']:.3g} {cpu['unit']} on "
            f"{cpu['threads']} thread(s) of {cpu['host_cores']} host core(s) "
            f"({cpu['cpu_model']}); {cpu['sample']}")

    desc = {"fused": "; steady state: previous step's commit fused into this step's verify",
            "deferred": f"; steady state: commit deferred into a log of {args.deferred} terms",
            "separate": "; verify then commit, two launches per layer",
            "snapshot": "; store-all snapshot path"}[mode]
    line = {
        "metric": "tree verify+commit draft-nodes*heads/sec",
        "value": value,
        "unit": "nodes*heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; Qwen3.5-shaped GDN heads, dk=dv=128)",
        "config": {"workload": wl.desc + desc,
                   "B": B, "H": H, "N": N, "layers": nl, "qkv_dtype": dtype,
                   "state_dtype": "f32", "instances_rotated": n_inst,
                   "launch": "hip-graph" if args.graph else "stream"},
        "hbm_frac_step": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (None if mode == "snapshot" or wl.traffic_key is None else
                                 measured_traffic(wl.traffic_key, dom)),
                     "bytes_per_launch": d_bytes, "launch_us": d_ms * 1e3,
                     "timing": ("HIP events on the launch stream around the timed region, "
                                "over the launches in it" if mode in ("fused", "deferred") else
                                "HIP events around each launch, in a second pass of the "
                                "timed steps")},
        "kernels_us": {n: t * 1e3 for n, (b, t) in kern.items()},
        "copy_gbs": copy_gbs,
        "separate_calls": separate,
        "snapshot": snapshot,
        "cpu_baseline": cpu,
    }
    del pool
    torch.cuda.empty_cache()
    return line


def run_attention(args):
    """The softmax layers' half of a tree verify pass: one treewy_tree_attention per step over
    rotated instances of a B=32 batch (2 KV heads x 8 query heads, head dim 256, a chain of 4
    draft tokens) with args.attention committed cache rows per sequence."""
    import torch
    from linear_attention_speculative_head_amd import accounting, binding, inputs
    B, Hkv, G, N, ctxn = 32, inputs.ATTN_HKV, inputs.ATTN_G, 4, args.attention
    T = ctxn + 64
    per = B * Hkv * T * 256 * 2 * 2
    n_inst = min(32, max(1, math.ceil(args.pool_gib * 2 ** 30 / per)))
    log(f"[bench] tree attention: B={B} Hkv={Hkv} G={G} N={N} ctx={ctxn}; {n_inst} instance(s), "
        f"{per * n_inst / 2 ** 30:.2f} GiB")
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16).contiguous()
    pool = []
    gen = torch.Generator(device="cuda")
    for i in range(n_inst):
        # the cache drawn on the device (a seeded normal fill): only its shape matters here
        gen.manual_seed(3000 + i)
        Kc = torch.randn((B, Hkv, T, 256), device="cuda", generator=gen).to(torch.bfloat16)
        Vc = torch.randn((B, Hkv, T, 256), device="cuda", generator=gen).to(torch.bfloat16)
        P = inputs.make_attention_problem(3000 + i, B=B, Hkv=Hkv, G=G, N=N, T_max=N + 1,
                                          ctx=np.zeros(B), tree="chain")
        pool.append(dict(Kc=Kc, Vc=Vc, ctx=torch.full((B,), ctxn, dtype=torch.int32, device="cuda"),
                         Qd=bf(P.Qd), Kd=bf(P.Kd), Vd=bf(P.Vd),
                         parent=torch.from_numpy(P.parent).cuda(), P=P))
    O = torch.empty((B, N, Hkv * G, 256), device="cuda")
    ws = torch.empty(binding.treewy_tree_attention_workspace(B, Hkv, G, N, T), dtype=torch.uint8,
                     device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(i):
        x = pool[i]
        binding.treewy_tree_attention(x["Kc"], x["Vc"], x["ctx"], x["Qd"], x["Kd"], x["Vd"],
                                      x["parent"], O, ws, status)

    W = auto_warmup(args, accounting.attention_call_bytes(np.full(B, ctxn), N, Hkv, G))
    for s in range(W):
        step(s % n_inst)
    torch.cuda.synchronize()
    K = args.steps
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record()
    for s in range(K):
        step((W + s) % n_inst)
    r1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = r0.elapsed_time(r1) / K                # one call per step: its mean duration
    assert int(status.item()) == 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for s in range(K):
        ev[s][0].record()
        step((W + s) % n_inst)
        ev[s][1].record()
    torch.cuda.synchronize()
    ms_bracketed = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # algorithmic bytes: the committed cache rows read once, the draft tokens' q/k/v read, O
    # written (the split partials are the kernel's own traffic, not the method's)
    nbytes = accounting.attention_call_bytes(np.full(B, ctxn), N, Hkv, G)
    achieved = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] tree attention: {wall * 1e6 / K:.1f} us/step, {ms * 1e3:.1f} us per call over "
        f"the timed region ({ms_bracketed * 1e3:.1f} us with events around each call), "
        f"{achieved:.0f} GB/s algorithmic")
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = attention_cpu_baseline(pool[0], ctxn, G, args.cpu_seconds)
        log(f"[bench] cpu baseline (oracle): {cpu['value']:.3g} {cpu['unit']} on {cpu['cores']} "
            f"thread(s), {cpu['sample']}")
    traffic = measured_traffic(f"attention-{ctxn}", "treewy_tree_attention")
    return {
        "metric": "tree attention verify draft-nodes*query-heads/sec",
        "value": B * N * Hkv * G * K / wall, "unit": "nodes*heads/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": wall * 1e3 / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, f32 accumulate",
        "data": "synthetic (seeded queries/keys of the draft; normal-filled cache)",
        "config": {"workload": f"tree attention: B={B}, {Hkv} KV heads x {G} query heads, "
                               f"head dim 256, chain of {N}, {ctxn} committed rows",
                   "instances_rotated": n_inst},
        "roofline": {"bound": "hbm", "kernel": "treewy_tree_attention", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "bytes_per_launch": nbytes, "launch_us": ms * 1e3,
                     "launch_us_bracketed": ms_bracketed * 1e3},
        "cpu_baseline": cpu,
    }


def blas_threads():
    """Threads numpy's BLAS may use (the attention oracle's products run there)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return 1


def attention_cpu_baseline(x, ctxn, G, seconds):
    """The attention oracle, as it stands, on whole sequences of one instance (their committed
    cache copied to the host), one after another until about ``seconds`` have been spent."""
    from oracle import attention as oattn
    P = x["P"]
    B, N = P.parent.shape
    done, elapsed, b = 0, 0.0, 0
    while elapsed < seconds and done < 4 * B:
        Kc = x["Kc"][b:b + 1, :, :ctxn].float().cpu().numpy().astype(np.float64)
        Vc = x["Vc"][b:b + 1, :, :ctxn].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oattn.tree_attention(Kc, Vc, np.array([ctxn]), P.Qd[b:b + 1], P.Kd[b:b + 1],
                             P.Vd[b:b + 1], P.parent[b:b + 1], G)
        elapsed += time.perf_counter() - t0
        done += 1
        b = (b + 1) % B
    Hq = P.Qd.shape[2]
    return {"value": done * N * Hq / elapsed, "unit": "nodes*heads/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} whole sequence(s) of {ctxn} cached rows, {N} nodes x {Hq} "
                      f"query heads each (cache conversion to float64 not timed)"}


def copy_bandwidth(gib):
    """A plain device-to-device copy of `gib` GiB, timed with HIP events over ten copies after
    two untimed ones: bytes read plus bytes written per second (GB/s), the achievable
    streaming rate of this part on this machine."""
    import torch
    n = int(gib * 2 ** 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / t / 1e9


def host_cpu():
    """(cores this process may run on, CPU model name from /proc/cpuinfo)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return cores, model


def copy_probe(mib):
    """One plain device copy of known size: a counter run scales its FETCH_SIZE / WRITE_SIZE
    readings by what the counters report for this dispatch."""
    import torch
    src_t = torch.ones(mib * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
    dst_t = torch.empty_like(src_t)
    torch.cuda.synchronize()
    dst_t.copy_(src_t)
    torch.cuda.synchronize()


def source_digest(path: str) -> str:
    """SHA-1 of a C/C++/HIP source with its comments and whitespace removed, so that a count
    taken on a kernel stays attached to it through edits of its comments, and no longer
    after any change to its code."""
    import hashlib
    text = open(path, encoding="utf-8").read()
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":                 # a literal: copied as it is
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return hashlib.sha1("".join(out).encode("utf-8")).hexdigest()


def measured_traffic(cfg, entry: str):
    """Counted HBM bytes per launch of `entry` on workload `cfg`, or None when no count was
    taken or the kernel source's code changed since."""
    rel = TRAFFIC_FILES.get(cfg)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    d = json.load(open(os.path.join(ROOT, rel)))
    k = d.get("kernels", {}).get(entry)
    if not k:
        return None
    src = os.path.join(ROOT, k["source"])
    if not os.path.exists(src) or source_digest(src) != k.get("source_digest"):
        return None
    return float(k["hbm_bytes_per_launch"])


def sample_heads(P, count, start):
    """`count` (layer, sequence, head) triples of problem P, spread over its layers and heads:
    the k-th one takes layer k mod L and head (start + k) * stride mod B*H, with a stride
    coprime to B*H near the golden fraction of it, so that consecutive picks land far apart."""
    nh = P.B * P.H
    stride = max(1, int(round(nh * 0.6180339887)))
    while math.gcd(stride, nh) != 1:
        stride += 1
    nl = len(P.layers)
    out = []
    for k in range(start, start + count):
        bh = (k * stride) % nh
        out.append((k % nl, bh // P.H, bh % P.H))
    return out


def cpu_baseline(P, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Heads spread over every layer and sequence of the measured instance (sample_heads) are
    replayed (verify + commit, fp64) in batches until about ``seconds`` of wall time have been
    spent.  The oracle runs OpenMP over heads on up to 16 host threads (the host share of one
    GPU on the machines this runs on)."""
    import oracle
    threads = oracle.default_threads()
    cores, model = host_cpu()
    done, elapsed, pos, chunk = 0, 0.0, 0, max(threads, 16)
    layers_seen = set()
    while elapsed < seconds:
        sel = sample_heads(P, chunk, pos)
        by_layer = {}
        for l, b, h in sel:
            by_layer.setdefault(l, []).append((b, h))
        t0 = time.perf_counter()
        for l, heads in by_layer.items():
            oracle.batch(P.layers[l], P.parent, P.accepted, heads=heads, threads=threads)
        dt = time.perf_counter() - t0
        elapsed += dt
        done += len(sel)
        pos += len(sel)
        layers_seen.update(by_layer)
        # grow the batch towards about a quarter of the remaining budget
        per = dt / len(sel)
        chunk = int(min(max(chunk, 0.25 * (seconds - elapsed) / max(per, 1e-9)), 2048))
        chunk = max(chunk, threads * len(P.layers) if len(P.layers) > 1 else threads)
    rate = done * P.N / elapsed
    return {"value": rate, "unit": "nodes*heads/s", "cores": threads, "threads": threads,
            "host_cores": cores, "cpu_model": model, "kind": "oracle",
            "sample": f"{done} head replays of {P.N}-node trees, spread over "
                      f"{len(layers_seen)} of {len(P.layers)} layer(s) and the {P.B * P.H} "
                      f"heads of each, verify+commit in fp64, {elapsed:.1f} s wall on "
                      f"{threads} thread(s)"}


if __name__ == "__main__":
    main()
