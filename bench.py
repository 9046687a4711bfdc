#!/usr/bin/env python3
"""Benchmark of the streaming chunk-attention hot path on one MI355X.

One "step" is one generated chunk at steady state (window full): for each
of the D denoise steps, 3D-RoPE of Q and K plus chunk attention over sinks +
window + the chunk, then the RoPE-fused append that commits the chunk and
evicts the oldest frames -- one wm_rollout_step call.  Default workload: the
Self-Forcing 1.3B DiT layer shape (12 heads, d 128, 30x52 tokens/frame,
chunk 3 frames, 1 sink + 18-frame window, 4 denoise steps), synthetic
N(0,1) bf16 inputs resident in HBM.

Printed: one JSON line.  `value` is whole-step attention throughput
(algorithmic attention flops of the timed steps / wall time of the timed
region, RoPE and append included).  `roofline` is the attention kernel alone
(algorithmic flops per launch / mean launch time from HIP events on the
launch stream) against the bf16 dense MFMA peak.  `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload.
"""

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk-attention TFLOP/s (% bf16 MFMA peak) + denoise-steps/sec per chunk"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", type=int, default=2, help="single-rollout workload id (1-4 or 6), default 2")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=12, help="q heads in the oracle sample")
    ap.add_argument("--layers", type=int, default=30,
                    help="layers of the multi-layer append measurement (0 = skip)")
    ap.add_argument("--extra-workloads", default="3,4,5,6",
                    help="comma-separated workload ids whose steady-state attention is also timed "
                         "(0 = none): drive, the 32/8-head GQA workload (key-range split and "
                         "merge), eight drive rollouts in one call and the four-view workload "
                         "by default")
    ap.add_argument("--modes-workload", type=int, default=1,
                    help="second workload whose rollout step is timed eager / finalize stream / graph "
                         "(0: none)")
    ap.add_argument("--steady-only", action="store_true",
                    help="time only the steady-state step and its kernels (no multi-layer append, "
                         "extra workloads, launch modes or whole rollout): every attention launch "
                         "then has the steady shape, as profiling runs want")
    ap.add_argument("--append-sweep", default="1,2,4,8,16,30",
                    help="layer counts of the append transfer-size sweep: one multi-layer append per "
                         "count (57.5 MB per layer at sf13b), inputs from HBM, beside a plain copy of "
                         "the same bytes (empty = skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain elementwise copy of this many MiB first (untimed), as the "
                         "known-size reference for HBM byte counters")
    return ap.parse_args()


def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed (string
    literals are left alone: the kernel sources hold no comment markers in
    strings)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest():
    """sha256 over the code of the kernel sources and the internal header
    (comments and layout ignored: they do not change the compiled kernels)
    and over the product build's compile flags."""
    import hashlib
    from autoregressive_video_world_amd import _build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "autoregressive_video_world_amd", "csrc")
    for rel in ("kernels/chunk_attn.hip", "kernels/rope_append.hip", "wm_internal.hpp"):
        with open(os.path.join(csrc, rel)) as f:
            h.update(_code_only(f.read()).encode())
    flags = {"common": [f for f in _build.COMMON if not f.startswith("-I")],
             "per_file": {k.replace(os.sep, "/"): v for k, v in sorted(_build.PER_FILE.items())}}
    h.update(json.dumps(flags, sort_keys=True).encode())
    return h.hexdigest()


def attn_kernel_name(head_dim):
    """The attention kernel the library launches."""
    return "chunk_attn_kernel<%d>" % head_dim


def profiled_traffic(workload_name, key="traffic_bytes_per_launch"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    The summary records the source digest of the kernels it measured; kernels
    changed since then get None (stale counters are not reported)."""
    path = os.path.join(ROOT, "profiles", "chunk_attn_%s_hbm_traffic.md" % workload_name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return int(fields[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, n_heads):
    """Oracle, as it stands, on one steady-state denoise step restricted to n_heads q heads."""
    import numpy as np
    from oracle.rollout import Rollout
    from wm_synth import Source

    src = Source(wl)
    ro = Rollout(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, wl.n_sink, wl.window,
                 n_views=wl.n_views)
    for n0 in range(wl.n_sink + wl.window):
        ro.commit(src.chunk(0, n0, 1, -1, "k"), src.chunk(0, n0, 1, -1, "v"), 1)
    n = wl.chunk
    n0 = ro.n_committed
    q = src.chunk(0, n0, n, 0, "q")
    k = src.chunk(0, n0, n, 0, "k")
    v = src.chunk(0, n0, n, 0, "v")
    heads = list(range(min(n_heads, wl.n_q_heads)))
    t0 = time.perf_counter()
    q_rot = ro.rope(q, n)
    k_rot = ro.rope(k, n)
    ro.attend(q_rot, k_rot, v, n, heads=heads)
    dt = time.perf_counter() - t0
    flops = wl.attn_flops() * len(heads) / wl.n_q_heads
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    cores = threads or len(os.sched_getaffinity(0))
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join("%s %s (%s threads)" % (i.get("internal_api"), i.get("version"), i.get("num_threads"))
                         for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:
        pass
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "one steady-state denoise step of %s (RoPE of the chunk's Q and K, attention "
                      "of all %d queries over %d keys) for %d of %d q heads, fp64 NumPy; %.1f s"
                      % (wl.name, wl.nq, wl.steady_keys(), len(heads), wl.n_q_heads, dt),
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model, "blas": blas}


def cpu_baseline_others():
    """The oracle on one steady-state denoise step (all heads) of the drive and
    32/8-head GQA workloads, and on the whole tiny rollout."""
    from oracle.rollout import Rollout
    from wm_synth import WORKLOADS, Source
    out = []
    for wid in (3, 4):
        r = cpu_baseline(WORKLOADS[wid], WORKLOADS[wid].n_q_heads)
        out.append({"workload": WORKLOADS[wid].name, "value": r["value"], "unit": r["unit"], "sample": r["sample"]})
    wl = WORKLOADS[1]
    src = Source(wl)
    ro = Rollout(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, wl.n_sink, wl.window)
    t0 = time.perf_counter()
    flops = 0.0
    for c in wl.chunks():
        n0 = ro.n_committed
        for s in range(wl.n_denoise):
            ro.denoise_step(src.chunk(0, n0, c, s, "q"), src.chunk(0, n0, c, s, "k"), src.chunk(0, n0, c, s, "v"), c)
            flops += wl.attn_flops(n_q=c * wl.ft, n_k=(min(n0, wl.n_sink + wl.window) + c) * wl.ft)
        ro.commit(src.chunk(0, n0, c, wl.n_denoise - 1, "k"), src.chunk(0, n0, c, wl.n_denoise - 1, "v"), c)
    dt = time.perf_counter() - t0
    out.append({"workload": wl.name, "value": flops / dt / 1e12, "unit": "TFLOP/s",
                "sample": "the whole %d-frame rollout (%d denoise steps per chunk), fp64 NumPy; %.2f s"
                          % (wl.n_gen, wl.n_denoise, dt)})
    return out


def whole_rollout(torch, wm, wl, dev, qs, ks, vs, outs, q_rot, k_rot, heat, reps=3):
    """A whole rollout from an empty ring (prefill, then every chunk, the
    window filling on the way): algorithmic attention flops of all steps /
    wall time of the whole loop, the median of `reps` rollouts, each after
    `heat` has brought the clock to its sustained level."""
    C, D, ft = wl.chunk, wl.n_denoise, wl.ft
    R = wl.n_sink + wl.window
    times, flops = [], 0.0
    for _ in range(reps):
        ring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                         wl.n_sink, wl.window, C, device=dev, n_views=wl.n_views)
        ws_bytes = ring.workspace_bytes(C)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        views = {c: ([q[:, :c * ft] for q in qs], [k[:, :c * ft] for k in ks], [v[:, :c * ft] for v in vs],
                     [o[:, :c * ft] for o in outs], q_rot[:, :c * ft], k_rot[:, :c * ft])
                 for c in set(wl.chunks())}
        heat()
        t0 = time.perf_counter()
        committed, flops = 0, 0.0
        if wl.prefill:
            ring.append_evict(ks[-1][:, :wl.prefill * ft], vs[-1][:, :wl.prefill * ft], wl.prefill)
            committed = wl.prefill
        for c in wl.chunks():
            q, k, v, o, qr, kr = views[c]
            ring.rollout_step(q, k, v, c, outs=o, q_rot_scratch=qr, k_rot_scratch=kr, workspace=ws)
            flops += D * wl.attn_flops(n_q=c * ft, n_k=(min(committed, R) + c) * ft)
            committed += c
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        ring.close()
    t = sorted(times)[len(times) // 2]
    return {"frames": wl.prefill + wl.n_gen, "chunks": len(wl.chunks()), "ms": round(t * 1e3, 3),
            "attn_tflops": round(flops / t / 1e12, 2)}


def rollout_modes(torch, wm, wl, randn, dev, steps, warmup, ring=None):
    """ms per steady-state rollout step, launched three ways: every launch
    from the host on one stream; the append on a second (finalize) stream;
    the step's launches replayed from a HIP graph."""
    own = ring is None
    if own:
        ring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                         wl.n_sink, wl.window, wl.chunk, device=dev, n_views=wl.n_views)
        for _ in range(wl.n_sink + wl.window):
            ring.append_evict(randn(1, wl.ft, wl.n_kv_heads, wl.head_dim),
                              randn(1, wl.ft, wl.n_kv_heads, wl.head_dim), 1)
    C, D, ft = wl.chunk, wl.n_denoise, wl.ft
    qs = [randn(1, C * ft, wl.n_q_heads, wl.head_dim) for _ in range(D)]
    ks = [randn(1, C * ft, wl.n_kv_heads, wl.head_dim) for _ in range(D)]
    vs = [randn(1, C * ft, wl.n_kv_heads, wl.head_dim) for _ in range(D)]
    outs = [torch.empty_like(q) for q in qs]
    q_rot, k_rot = torch.empty_like(qs[0]), torch.empty_like(ks[0])
    ws_bytes = ring.workspace_bytes(C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    fin = torch.cuda.Stream()
    graph = ring.rollout_graph(qs, ks, vs, C, outs=outs, q_rot_scratch=q_rot, k_rot_scratch=k_rot,
                               workspace=ws)
    kw = dict(outs=outs, q_rot_scratch=q_rot, k_rot_scratch=k_rot, workspace=ws)
    modes = {"eager": lambda: ring.rollout_step(qs, ks, vs, C, **kw),
             "finalize_stream": lambda: ring.rollout_step(qs, ks, vs, C, finalize_stream=fin, **kw),
             "graph": graph.launch}
    res = {}
    for name, fn in modes.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res[name + "_ms_per_step"] = round((time.perf_counter() - t0) / steps * 1e3, 4)
    res["graph_rebuilt_in_steady_state"] = bool(graph.rebuilt)
    graph.close()
    if own:
        ring.close()
    return res


def main():
    args = parse()
    if args.steady_only:
        args.layers, args.extra_workloads, args.modes_workload, args.append_sweep = 0, "0", 0, ""
    if args.gpus != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (it would shard by rollout "
              "or by kv head with no collective in the path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import autoregressive_video_world_amd as wm
    from wm_synth import WORKLOADS

    wl = WORKLOADS[args.workload]
    if wl.batch != 1:
        print("bench.py times single-rollout workloads (1-4)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + wl.cfg)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 19  # bf16 elements
        a = torch.ones(n, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)  # reads and writes exactly n*2 bytes
        torch.cuda.synchronize()
        del a, b

    ring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                     wl.n_sink, wl.window, wl.chunk, device=dev, n_views=wl.n_views)
    C, D, ft = wl.chunk, wl.n_denoise, wl.ft
    # steady state: fill sinks + window (prefill-style appends of synthetic K/V)
    filled = 0
    while filled < wl.n_sink + wl.window:
        n = min(C, wl.n_sink + wl.window - filled)
        ring.append_evict(randn(1, n * ft, wl.n_kv_heads, wl.head_dim),
                          randn(1, n * ft, wl.n_kv_heads, wl.head_dim), n)
        filled += n
    qs = [randn(1, C * ft, wl.n_q_heads, wl.head_dim) for _ in range(D)]
    ks = [randn(1, C * ft, wl.n_kv_heads, wl.head_dim) for _ in range(D)]
    vs = [randn(1, C * ft, wl.n_kv_heads, wl.head_dim) for _ in range(D)]
    outs = [torch.empty_like(q) for q in qs]
    q_rot = torch.empty_like(qs[0])
    k_rot = torch.empty_like(ks[0])
    stream = torch.cuda.current_stream()
    # key-range split workspace (non-empty only where the grid is small)
    ws_bytes = ring.workspace_bytes(C)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        ring.rollout_step(qs, ks, vs, C, outs=outs, q_rot_scratch=q_rot, k_rot_scratch=k_rot,
                          workspace=ws)

    # The first call (code-object load, first-touch of the buffers) on its own.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    first_step_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    attn_flops_step = wl.attn_flops() * D
    value = attn_flops_step * args.steps / elapsed / 1e12

    # ---- per-kernel timing with HIP events on the launch stream ------------
    # `reps` launches back to back between one pair of events: the mean
    # duration of a launch in a busy stream.  Short launches (RoPE, append)
    # are queued behind a ~1 ms spin kernel that touches no memory, so that,
    # as in a rollout, the host-side cost of each call (measured separately)
    # overlaps GPU work instead of leaving the GPU idle between launches,
    # while the caches hold what the untimed call left.  Before each loop the
    # GPU runs attention launches for about 100 ms: after an idle gap of even
    # 50 ms the clock takes tens of milliseconds to return to its sustained
    # level under load, which would otherwise inflate the first launches.
    def heat(seconds=0.1):
        t = time.perf_counter()
        while time.perf_counter() - t < seconds:
            attn()
            torch.cuda.synchronize()

    def timed(fn, reps, behind=None):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        heat()
        fn()
        torch.cuda.synchronize()
        if behind is not None:
            behind()
        a.record(stream)
        h0 = time.perf_counter()
        for _ in range(reps):
            fn()
        host_us = (time.perf_counter() - h0) / reps * 1e6
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps, host_us

    ring.rope3d(qs[0], C, y=q_rot)
    ring.rope3d(ks[0], C, y=k_rot)
    attn = lambda: ring.chunk_attn(q_rot, k_rot, vs[0], C, out=outs[0], workspace=ws)
    busy = lambda: torch.cuda._sleep(2_500_000)
    attn_mean, _ = timed(attn, args.kernel_reps)

    # Spread of single launches: an event pair around each, back to back.
    def per_launch(fn, reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        heat()
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))

    attn_each = per_launch(attn, args.kernel_reps)
    attn_p50 = attn_each[len(attn_each) // 2]
    attn_p90 = attn_each[min(len(attn_each) - 1, (9 * len(attn_each)) // 10)]
    # Power context (a diagnostic beside the metric, not part of it): under
    # this kernel the card runs at its board power limit, and the power of the
    # matrix cores depends on the operand bits.  The same launch over a ring
    # and chunk of all-zero K/V/Q, and a plain bf16 GEMM through torch (the
    # vendor library) on N(0,1) and on all-zero operands, show how much of the
    # gap to the quoted peak is the power limit on random data.
    power_ctx = None
    if not args.steady_only:
        zring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                          wl.n_sink, wl.window, wl.chunk, device=dev, n_views=wl.n_views)
        zkv = torch.zeros(1, C * ft, wl.n_kv_heads, wl.head_dim, dtype=torch.bfloat16, device=dev)
        filled = 0
        while filled < wl.n_sink + wl.window:
            n = min(C, wl.n_sink + wl.window - filled)
            zring.append_evict(zkv[:, :n * ft], zkv[:, :n * ft], n)
            filled += n
        zq = torch.zeros_like(q_rot)
        zout = torch.empty_like(q_rot)
        zattn = lambda: zring.chunk_attn(zq, zkv, zkv, C, out=zout, workspace=ws)
        zattn()
        torch.cuda.synchronize()
        z_mean, _ = timed(zattn, args.kernel_reps)
        zring.close()
        del zkv, zq, zout
        n_g = 8192
        gflop = 2.0 * n_g ** 3

        def gemm_tflops(a, b):
            c = torch.empty(n_g, n_g, dtype=torch.bfloat16, device=dev)
            t, _ = timed(lambda: torch.matmul(a, b, out=c), 40)
            return gflop / (t * 1e-3) / 1e12

        ga, gb = randn(n_g, n_g), randn(n_g, n_g)
        g_rand = gemm_tflops(ga, gb)
        ga.zero_()
        gb.zero_()
        g_zero = gemm_tflops(ga, gb)
        del ga, gb
        power_ctx = {
            "note": "diagnostic, not the metric: the board power limit and operand-dependent matrix-core power",
            "attn_zero_inputs_tflops": round(wl.attn_flops() / (z_mean * 1e-3) / 1e12, 1),
            "attn_zero_inputs_frac": round(wl.attn_flops() / (z_mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "attn_zero_inputs_launch_ms_mean": round(z_mean, 4),
            "gemm_bf16_%d_randn_tflops" % n_g: round(g_rand, 1),
            "gemm_bf16_%d_zeros_tflops" % n_g: round(g_zero, 1),
        }
    rope_mean, rope_host_us = timed(lambda: ring.rope3d_pair(qs[0], ks[0], C, y=q_rot, y2=k_rot),
                                    args.kernel_reps, busy)
    rope_q_mean, _ = timed(lambda: ring.rope3d(qs[0], C, y=q_rot), args.kernel_reps, busy)
    rope_k_mean, _ = timed(lambda: ring.rope3d(ks[0], C, y=k_rot), args.kernel_reps, busy)
    # The paired RoPE with its inputs rotated over more than twice the 256 MB
    # last-level cache (MALL), so that every read comes from HBM.
    rope_in = (qs[0].numel() + ks[0].numel()) * 2
    n_rc = max(2, -(-(512 << 20) // rope_in))
    rcold = [(randn(*qs[0].shape), randn(*ks[0].shape)) for _ in range(n_rc)]
    rc_i = [0]

    def rope_cold():
        qc, kc = rcold[rc_i[0] % n_rc]
        rc_i[0] += 1
        ring.rope3d_pair(qc, kc, C, y=q_rot, y2=k_rot)

    rope_cold_mean, _ = timed(rope_cold, max(args.kernel_reps, 2 * n_rc), busy)
    del rcold
    app_mean, app_host_us = timed(lambda: ring.append_evict(ks[-1], vs[-1], C), args.kernel_reps, busy)
    # The same append with its inputs rotated over more than twice the
    # 256 MB last-level cache (MALL), so every read comes from HBM.  In a
    # rollout the committed K and V were produced just before the commit, so
    # the figure above (inputs cache-warm) is the one a rollout sees.
    n_cold = max(2, -(-(512 << 20) // (2 * ks[-1].numel() * 2)))
    cold = [(randn(*ks[-1].shape), randn(*vs[-1].shape)) for _ in range(n_cold)]
    cold_i = [0]

    def app_cold():
        kc, vc = cold[cold_i[0] % n_cold]
        cold_i[0] += 1
        ring.append_evict(kc, vc, C)

    app_cold_mean, _ = timed(app_cold, max(args.kernel_reps, 2 * n_cold), busy)
    del cold
    # Reference: a plain elementwise copy (torch.neg) of the same bytes, its
    # inputs rotated the same way -- what HBM delivers to a transfer this short.
    copy_src = [randn(wl.append_bytes() // 4) for _ in range(n_cold)]
    copy_dst = [torch.empty_like(x) for x in copy_src]
    copy_i = [0]

    def copy_cold():
        a = copy_i[0] % n_cold
        copy_i[0] += 1
        torch.neg(copy_src[a], out=copy_dst[a])

    copy_cold_mean, _ = timed(copy_cold, max(args.kernel_reps, 2 * n_cold), busy)
    del copy_src, copy_dst

    # A whole model's commit: the same workload's ring with `--layers` layers,
    # every layer's K and V appended by one call (one launch), against the
    # same bytes committed by one one-layer append per layer.  The inputs
    # (layers x 28.8 MB at sf13b) exceed the last-level cache: HBM-bound.
    layers = None
    if args.layers > 1:
        Ln = args.layers
        mring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                          wl.n_sink, wl.window, wl.chunk, device=dev, n_layers=Ln, n_views=wl.n_views)
        lk = randn(Ln, *ks[-1].shape)
        lv = randn(Ln, *vs[-1].shape)
        lay_mean, _ = timed(lambda: mring.append_evict(lk, lv, C), max(4, args.kernel_reps // 4), busy)
        per_layer = lambda: [ring.append_evict(lk[i], lv[i], C) for i in range(Ln)]
        per_mean, _ = timed(per_layer, max(2, args.kernel_reps // 10), busy)
        lay_bytes = Ln * wl.append_bytes()
        del lk, lv
        csrc = randn(lay_bytes // 4)
        cdst = torch.empty_like(csrc)
        copy_mean, _ = timed(lambda: torch.neg(csrc, out=cdst), max(4, args.kernel_reps // 4), busy)
        del csrc, cdst
        layers = {"bound": "hbm", "layers": Ln, "bytes_per_launch": lay_bytes,
                  "achieved": round(lay_bytes / (lay_mean * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": round(lay_bytes / (lay_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "launch_ms_mean": round(lay_mean, 4),
                  "one_append_per_layer_gbs": round(lay_bytes / (per_mean * 1e-3) / 1e9, 1),
                  "copy_same_bytes_gbs": round(lay_bytes / (copy_mean * 1e-3) / 1e9, 1),
                  "pool_bytes": mring.pool_bytes}
        mring.close()
    torch.cuda.synchronize()

    # Append transfer-size sweep: one append of L layers per launch (L x the
    # workload's per-chunk bytes), inputs rotated over more than twice the
    # 256 MB last-level cache so that they come from HBM, beside a plain
    # elementwise copy (torch.neg) of exactly the same bytes rotated the same
    # way -- where one transfer of this size tops out on this chip.
    sweep = []
    for Ln in [int(x) for x in args.append_sweep.split(",") if x.strip()]:
        sring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                          wl.n_sink, wl.window, wl.chunk, device=dev, n_layers=Ln, n_views=wl.n_views)
        nbytes = Ln * wl.append_bytes()
        nrot = max(2, -(-(512 << 20) // (nbytes // 2)))
        sin = [(randn(Ln, *ks[-1].shape), randn(Ln, *vs[-1].shape)) for _ in range(nrot)]
        si = [0]

        def sweep_app():
            kc, vc = sin[si[0] % nrot]
            si[0] += 1
            sring.append_evict(kc, vc, C)

        reps = max(2 * nrot, 8)
        a_mean, _ = timed(sweep_app, reps, busy)
        del sin
        csrc = [randn(nbytes // 4) for _ in range(nrot)]
        cdst = [torch.empty_like(x) for x in csrc]
        ci = [0]

        def sweep_copy():
            a = ci[0] % nrot
            ci[0] += 1
            torch.neg(csrc[a], out=cdst[a])

        c_mean, _ = timed(sweep_copy, reps, busy)
        del csrc, cdst
        sring.close()
        sweep.append({"layers": Ln, "bytes_per_launch": nbytes,
                      "append_gbs": round(nbytes / (a_mean * 1e-3) / 1e9, 1),
                      "append_frac": round(nbytes / (a_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "append_us": round(a_mean * 1e3, 2),
                      "copy_gbs": round(nbytes / (c_mean * 1e-3) / 1e9, 1),
                      "copy_us": round(c_mean * 1e3, 2)})
    torch.cuda.synchronize()

    # Steady-state attention of other workloads: the same kernel at other
    # shapes, the key-range split and its merge where the grid is small (the
    # merge runs inside the attention launch), several camera views per frame.
    extras = []
    for wid in [int(x) for x in args.extra_workloads.split(",") if x.strip()]:
        if wid in (0, args.workload):
            continue
        vw = WORKLOADS[wid]
        nb = vw.batch   # every rollout at steady state (window full), one call for all
        vring = wm.KVRing(nb, vw.n_q_heads, vw.n_kv_heads, vw.head_dim, vw.frame_h, vw.frame_w,
                          vw.n_sink, vw.window, vw.chunk, device=dev, n_views=vw.n_views)
        for _ in range(vw.n_sink + vw.window):
            vring.append_evict(randn(nb, vw.ft, vw.n_kv_heads, vw.head_dim),
                               randn(nb, vw.ft, vw.n_kv_heads, vw.head_dim), 1)
        vq, vk = vring.rope3d_pair(randn(nb, vw.nq, vw.n_q_heads, vw.head_dim),
                                   randn(nb, vw.nq, vw.n_kv_heads, vw.head_dim), vw.chunk)
        vv = randn(nb, vw.nq, vw.n_kv_heads, vw.head_dim)
        vo = torch.empty_like(vq)
        vws_bytes = vring.workspace_bytes(vw.chunk)
        vws = torch.empty(vws_bytes, dtype=torch.uint8, device=dev) if vws_bytes else None
        flops = nb * vw.attn_flops()
        reps = max(3, int(round(20 * 1e12 / flops)))   # about 20 ms of work
        v_mean, _ = timed(lambda: vring.chunk_attn(vq, vk, vv, vw.chunk, out=vo, workspace=vws), reps)
        tf = flops / (v_mean * 1e-3) / 1e12
        extras.append({"workload": "%s: %s%d q/%d kv heads, d %d, %s%dx%d tokens/frame (Nq %d, Nk %d)"
                                   % (vw.name, "%d rollouts, " % nb if nb > 1 else "", vw.n_q_heads,
                                      vw.n_kv_heads, vw.head_dim,
                                      "%d views of " % vw.n_views if vw.n_views > 1 else "", vw.frame_h,
                                      vw.frame_w, vw.nq, vw.steady_keys()),
                       "attn_tflops": round(tf, 2), "attn_pct_mfma_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                       "launch_ms_mean": round(v_mean, 4), "split_workspace_bytes": vws_bytes})
        vring.close()
        del vq, vk, vv, vo, vws

    # Whole-rollout average beside the steady state.
    rollout = None if args.steady_only else whole_rollout(torch, wm, wl, dev, qs, ks, vs, outs,
                                                            q_rot, k_rot, heat)

    # The same step launched from the finalize stream and from a HIP graph,
    # here and on a workload small enough that launch costs show.
    modes = None if args.steady_only else {
        "workload": wl.name, **rollout_modes(torch, wm, wl, randn, dev, args.steps, args.warmup, ring)}
    modes_small = None
    if args.modes_workload and args.modes_workload != args.workload:
        mw = WORKLOADS[args.modes_workload]
        modes_small = {"workload": "%s: %d q/%d kv heads, d %d, %dx%d tokens/frame, chunk %d, "
                                   "%d sink + %d window frames, %d denoise steps"
                                   % (mw.name, mw.n_q_heads, mw.n_kv_heads, mw.head_dim, mw.frame_h,
                                      mw.frame_w, mw.chunk, mw.n_sink, mw.window, mw.n_denoise),
                       **rollout_modes(torch, wm, mw, randn, dev, max(args.steps, 200), args.warmup)}

    attn_tflops = wl.attn_flops() / (attn_mean * 1e-3) / 1e12
    app_bytes = wl.append_bytes()
    app_gbs = app_bytes / (app_mean * 1e-3) / 1e9
    app_cold_gbs = app_bytes / (app_cold_mean * 1e-3) / 1e9
    copy_cold_gbs = app_bytes / (copy_cold_mean * 1e-3) / 1e9
    rope_bytes = 2 * wl.nq * wl.head_dim * 2 * (wl.n_q_heads + wl.n_kv_heads)
    rope_gbs = rope_bytes / (rope_mean * 1e-3) / 1e9
    rope_cold_gbs = rope_bytes / (rope_cold_mean * 1e-3) / 1e9
    prof_traffic = profiled_traffic(wl.name)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %d q/%d kv heads, d %d, %s%dx%d tokens/frame, chunk %d frames "
                               "(Nq %d), %d sink + %d window frames (Nk %d), %d denoise steps, steady state"
                               % (wl.name, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                  "%d views of " % wl.n_views if wl.n_views > 1 else "", wl.frame_h,
                                  wl.frame_w, C, wl.nq, wl.n_sink, wl.window, wl.steady_keys(), D),
                   "batch": 1, "n_q": wl.nq, "n_k": wl.steady_keys(), "denoise_steps": D},
        "denoise_steps_per_s_per_chunk": round(1e3 / (attn_mean + rope_mean), 2),
        "chunks_per_s": round(1e3 / ms_per_step, 3),
        "first_step_ms": round(first_step_ms, 3),
        "whole_rollout": rollout,
        "attn_pct_mfma_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": attn_kernel_name(wl.head_dim),
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": prof_traffic,
                     "launch_ms_mean": round(attn_mean, 4), "launch_ms_p50": round(attn_p50, 4),
                     "launch_ms_p90": round(attn_p90, 4),
                     "flops_per_launch": wl.attn_flops(), "split_workspace_bytes": ws_bytes},
        "append": {"bound": "hbm", "inputs": "from HBM (rotated over 512 MB, twice the last-level cache)",
                   "achieved": round(app_cold_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(app_cold_gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": app_bytes,
                   "traffic": profiled_traffic(wl.name, "append_traffic_bytes_per_launch"),
                   "launch_ms_mean": round(app_cold_mean, 5), "host_us_per_call": round(app_host_us, 1),
                   "copy_same_bytes_from_hbm": round(copy_cold_gbs, 1),
                   "frac_of_copy": round(app_cold_gbs / copy_cold_gbs, 4),
                   "achieved_mall_warm": round(app_gbs, 1),
                   "frac_mall_warm": round(app_gbs / PEAK_HBM_GBS, 4),
                   "launch_ms_mean_mall_warm": round(app_mean, 5)},
        "power_context": power_ctx,
        "append_size_sweep": sweep,
        "rollout_modes": ([modes] if modes else []) + ([modes_small] if modes_small else []),
        "append_layers": layers,
        "other_workloads": extras,
        "rope": {"bound": "hbm", "inputs": "from HBM (rotated over 512 MB, twice the last-level cache)",
                 "achieved": round(rope_cold_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(rope_cold_gbs / PEAK_HBM_GBS, 4),
                 "launch_ms_mean": round(rope_cold_mean, 5), "host_us_per_call": round(rope_host_us, 1),
                 "achieved_mall_warm": round(rope_gbs, 1),
                 "frac_mall_warm": round(rope_gbs / PEAK_HBM_GBS, 4),
                 "launch_ms_mean_mall_warm": round(rope_mean, 5),
                 "q_and_k_as_two_launches_gbs_mall_warm":
                     round(rope_bytes / ((rope_q_mean + rope_k_mean) * 1e-3) / 1e9, 1)},
        "cpu_baseline": None,
    }
    ring.close()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads)
        if not args.steady_only:
            result["cpu_baseline"]["other_workloads"] = cpu_baseline_others()
    try:
        result["git"] = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"],
                                       capture_output=True, text=True).stdout.strip() or None
    except Exception:
        pass
    result["versions"] = {"torch": torch.__version__, "hip": torch.version.hip}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
