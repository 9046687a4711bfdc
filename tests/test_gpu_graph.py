"""GPU: a rollout step as a HIP graph, and the append on a finalize stream.

Three rings start identical and run the same chunks: one through
wm_rollout_step on one stream (eager), one through wm_rollout_graph_launch
(the graph's buffers are refilled with each chunk's inputs), one through
wm_rollout_step with a separate finalize stream.  Every chunk's outputs,
append reports and pool bytes must be identical bit for bit, through the
window filling (where the launch shapes may change and the graph is
rebuilt) and steady state (where only its node parameters are refreshed).  Between
graph launches the test does unrelated eager work and synchronizes, and the
first steady-state chunk is also checked against the fp64 oracle.
"""

import os
import time

import numpy as np
import pytest
import torch

import autoregressive_video_world_amd as wm
from oracle.rollout import Rollout
from wm_synth import Source, Workload
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

CASES = {
    "mha_c2": Workload(401, "graph_mha", 1, 4, 4, 128, 10, 10, 2, 1, 3, 0, 14, 2),
    "gqa_batch2": Workload(402, "graph_gqa", 2, 8, 2, 128, 7, 9, 1, 1, 2, 0, 8, 2),
    "d64_c3": Workload(403, "graph_d64", 1, 2, 2, 64, 5, 10, 3, 1, 4, 0, 15, 1),
    # a step of ~0.6 ms on the GPU against ~40 us of host time per launch:
    # the host queues replays and refreshes parameters while earlier replays run
    "long_steps": Workload(404, "graph_long", 1, 12, 12, 128, 30, 52, 1, 1, 18, 0, 40, 2),
}


def new_ring(wl):
    """A ring over a zero-filled pool (filled before create: the RoPE tables live in the pool)."""
    meta = wm.KVRing(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                     wl.n_sink, wl.window, wl.chunk, meta_only=True)
    pool = torch.zeros(meta.pool_bytes, dtype=torch.uint8, device="cuda")
    meta.close()
    return wm.KVRing(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                     wl.n_sink, wl.window, wl.chunk, pool=pool)


@pytest.mark.parametrize("name,split", [("mha_c2", False), ("gqa_batch2", False), ("gqa_batch2", True),
                                        ("d64_c3", False)])
def test_graph_and_finalize_stream_match_eager(name, split):
    wl = CASES[name]
    print("case", name, "split", split, flush=True)
    old = os.environ.get("WM_ATTN_SPLIT")
    if split:
        os.environ["WM_ATTN_SPLIT"] = "3"
    try:
        _run(wl, split)
    finally:
        if old is None:
            os.environ.pop("WM_ATTN_SPLIT", None)
        else:
            os.environ["WM_ATTN_SPLIT"] = old


def _run(wl, split):
    B, C, D = wl.batch, wl.chunk, wl.n_denoise
    src = Source(wl)
    eager, graphed, overl = new_ring(wl), new_ring(wl), new_ring(wl)
    ws_bytes = eager.workspace_bytes(C)
    if split:
        assert ws_bytes > 0
    wss = [torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda") if ws_bytes else None
           for _ in range(3)]
    shape_q = (B, C * wl.ft, wl.n_q_heads, wl.head_dim)
    shape_k = (B, C * wl.ft, wl.n_kv_heads, wl.head_dim)
    gq = [torch.empty(shape_q, dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    gk = [torch.empty(shape_k, dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    gv = [torch.empty(shape_k, dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    graph = graphed.rollout_graph(gq, gk, gv, C, workspace=wss[1])
    fin_stream = torch.cuda.Stream()
    used = []
    junk = torch.randn(1 << 20, device="cuda")
    checked_oracle = False
    for ci in range(wl.n_gen // C):
        n0 = ci * C
        qs = [dev(src.batch_chunk([n0] * B, C, s, "q")) for s in range(D)]
        ks = [dev(src.batch_chunk([n0] * B, C, s, "k")) for s in range(D)]
        vs = [dev(src.batch_chunk([n0] * B, C, s, "v")) for s in range(D)]
        out_e, rep_e = eager.rollout_step(qs, ks, vs, C, workspace=wss[0])
        out_e = [host(o) for o in out_e]
        for s in range(D):
            gq[s].copy_(qs[s])
            gk[s].copy_(ks[s])
            gv[s].copy_(vs[s])
        out_g, rep_g = graph.launch()
        used.append(graph.rebuilt)
        out_g = [host(o) for o in out_g]
        # unrelated eager work and a synchronization between graph launches
        junk.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        out_o, rep_o = overl.rollout_step(qs, ks, vs, C, workspace=wss[2], finalize_stream=fin_stream)
        out_o = [host(o) for o in out_o]
        assert rep_g == rep_e and rep_o == rep_e, ci
        for s in range(D):
            assert np.array_equal(out_g[s], out_e[s]), ("graph", ci, s)
            assert np.array_equal(out_o[s], out_e[s]), ("finalize stream", ci, s)
        torch.cuda.synchronize()
        for r in (graphed, overl):
            assert torch.equal(r.pool_k(), eager.pool_k()) and torch.equal(r.pool_v(), eager.pool_v()), ci
        # the oracle, once the window is full
        if not checked_oracle and n0 >= wl.n_sink + wl.window:
            ro = Rollout(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                         wl.n_sink, wl.window)
            for cj in range(ci):
                m0 = cj * C
                ro.commit(src.batch_chunk([m0] * B, C, D - 1, "k")[0],
                          src.batch_chunk([m0] * B, C, D - 1, "v")[0], C)
            _, _, ref = ro.denoise_step(src.batch_chunk([n0] * B, C, 0, "q")[0],
                                        src.batch_chunk([n0] * B, C, 0, "k")[0],
                                        src.batch_chunk([n0] * B, C, 0, "v")[0], C)
            assert_close(out_e[0][0], ref, "oracle chunk %d" % ci)
            checked_oracle = True
    assert checked_oracle
    assert not used[-1] and not used[-2], used  # steady state: parameters refreshed, no rebuild
    graph.close()
    for r in (eager, graphed, overl):
        r.close()


def test_graph_of_a_destroyed_ring_is_refused():
    """A graph whose ring was destroyed must not launch, also when a new ring
    happens to be created at the same host address."""
    wl = CASES["mha_c2"]
    C, D = wl.chunk, wl.n_denoise
    ring = new_ring(wl)
    shape_q = (1, C * wl.ft, wl.n_q_heads, wl.head_dim)
    shape_k = (1, C * wl.ft, wl.n_kv_heads, wl.head_dim)
    gq = [torch.zeros(shape_q, dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    gk = [torch.zeros(shape_k, dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    gv = [torch.zeros(shape_k, dtype=torch.bfloat16, device="cuda") for _ in range(D)]
    graph = ring.rollout_graph(gq, gk, gv, C)
    graph.launch()
    torch.cuda.synchronize()
    ring.close()
    others = [new_ring(wl) for _ in range(4)]   # one may reuse the freed address
    with pytest.raises(wm.WMError) as e:
        graph.launch()
    assert e.value.name == "WM_E_STATE"
    graph.close()
    for r in others:
        r.close()


@pytest.mark.parametrize("name", ["mha_c2", "gqa_batch2", "long_steps"])
def test_back_to_back_graph_launches_match_eager(name):
    """Graph launches queued back to back with no synchronization between
    them (each refreshes its node parameters while the previous replay may
    still run), and steps whose appends go to a finalize stream -- on torch's
    default stream, which reaches the library as the null stream -- give the
    same pool bytes and last outputs as eager steps; so does a plain step
    queued right after a finalize-stream step."""
    wl = CASES[name]
    B, C, D = wl.batch, wl.chunk, wl.n_denoise
    src = Source(wl)
    eager, graphed, overl = new_ring(wl), new_ring(wl), new_ring(wl)
    fin = torch.cuda.Stream()
    shape_q = (B, C * wl.ft, wl.n_q_heads, wl.head_dim)
    shape_k = (B, C * wl.ft, wl.n_kv_heads, wl.head_dim)
    qs = [dev(src.batch_chunk([0] * B, C, s, "q")) for s in range(D)]
    ks = [dev(src.batch_chunk([0] * B, C, s, "k")) for s in range(D)]
    vs = [dev(src.batch_chunk([0] * B, C, s, "v")) for s in range(D)]
    assert qs[0].shape == shape_q and ks[0].shape == shape_k
    # fill the window first (shapes settle), then many steps without a sync
    graph = graphed.rollout_graph(qs, ks, vs, C)
    n_fill = -(-(wl.n_sink + wl.window) // C)
    for _ in range(n_fill):
        eager.rollout_step(qs, ks, vs, C)
        graph.launch()
        overl.rollout_step(qs, ks, vs, C, finalize_stream=fin)
    torch.cuda.synchronize()
    outs_e = outs_o = None
    for _ in range(12):
        outs_e, _ = eager.rollout_step(qs, ks, vs, C)
    plain_e, _ = eager.rollout_step(qs, ks, vs, C)
    for _ in range(12):
        outs_o, _ = overl.rollout_step(qs, ks, vs, C, finalize_stream=fin)
    plain_o, _ = overl.rollout_step(qs, ks, vs, C)   # must wait for the last pending append
    t0 = time.perf_counter()
    for _ in range(13):
        graph.launch()
        assert not graph.rebuilt
    queued = time.perf_counter() - t0
    torch.cuda.synchronize()
    print("13 graph launches queued in %.2f ms, ran in %.2f ms" % (queued * 1e3, (time.perf_counter() - t0) * 1e3))
    for r in (graphed, overl):
        assert torch.equal(r.pool_k(), eager.pool_k()) and torch.equal(r.pool_v(), eager.pool_v())
        for b in range(B):
            assert r.view(b) == eager.view(b)
    for s in range(D):
        assert torch.equal(graph.outs[s], plain_e[s]), s
        assert torch.equal(outs_o[s], outs_e[s]), s
        assert torch.equal(plain_o[s], plain_e[s]), s
    graph.close()
    for r in (eager, graphed, overl):
        r.close()


def test_graph_and_eager_steps_interleave_on_one_ring():
    """Graph replays, eager steps and finalize-stream steps alternate on one
    ring with no synchronization; every step's outputs and the final pool
    equal those of eager steps only."""
    wl = CASES["gqa_batch2"]
    B, C, D = wl.batch, wl.chunk, wl.n_denoise
    src = Source(wl)
    ref, mixed = new_ring(wl), new_ring(wl)
    fin = torch.cuda.Stream()
    qs = [dev(src.batch_chunk([0] * B, C, s, "q")) for s in range(D)]
    ks = [dev(src.batch_chunk([0] * B, C, s, "k")) for s in range(D)]
    vs = [dev(src.batch_chunk([0] * B, C, s, "v")) for s in range(D)]
    graph = mixed.rollout_graph(qs, ks, vs, C)
    want, got = [], []
    for i in range(15):
        o, _ = ref.rollout_step(qs, ks, vs, C)
        want.append([x.clone() for x in o])
        kind = i % 3
        if kind == 0:
            graph.launch()
            o = graph.outs
        elif kind == 1:
            o, _ = mixed.rollout_step(qs, ks, vs, C)
        else:
            o, _ = mixed.rollout_step(qs, ks, vs, C, finalize_stream=fin)
        got.append([x.clone() for x in o])
    torch.cuda.synchronize()
    for i in range(15):
        for s in range(D):
            assert torch.equal(got[i][s], want[i][s]), (i, s)
    assert torch.equal(mixed.pool_k(), ref.pool_k()) and torch.equal(mixed.pool_v(), ref.pool_v())
    graph.close()
    ref.close()
    mixed.close()


def test_created_stream_and_graph_with_active_mask():
    """A rollout on a created (non-default) stream, and a graph built with an
    active mask (rollout 1 idle), against eager steps on the default stream
    with the same mask: outputs of the active rollout, reports and pools are
    identical, and the idle rollout's slots stay as they were."""
    wl = CASES["gqa_batch2"]
    B, C, D = wl.batch, wl.chunk, wl.n_denoise
    src = Source(wl)
    ref, on_stream, graphed = new_ring(wl), new_ring(wl), new_ring(wl)
    qs = [dev(src.batch_chunk([0] * B, C, s, "q")) for s in range(D)]
    ks = [dev(src.batch_chunk([0] * B, C, s, "k")) for s in range(D)]
    vs = [dev(src.batch_chunk([0] * B, C, s, "v")) for s in range(D)]
    active = [1, 0]
    graph = graphed.rollout_graph(qs, ks, vs, C, active=active)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())   # the inputs were made on the default stream
    for i in range(9):
        o_ref, rep_ref = ref.rollout_step(qs, ks, vs, C, active=active)
        with torch.cuda.stream(side):
            o_side, rep_side = on_stream.rollout_step(qs, ks, vs, C, active=active, stream=side)
            o_side = [x.clone() for x in o_side]
        o_g, rep_g = graph.launch()
        assert rep_side == rep_ref and rep_g == rep_ref, i
        torch.cuda.current_stream().wait_stream(side)
        for s in range(D):
            assert torch.equal(o_side[s][0], o_ref[s][0]), (i, s)
            assert torch.equal(o_g[s][0], o_ref[s][0]), (i, s)
    torch.cuda.synchronize()
    for r in (on_stream, graphed):
        assert torch.equal(r.pool_k(), ref.pool_k()) and torch.equal(r.pool_v(), ref.pool_v())
        assert r.view(1)["n_committed"] == 0
    assert torch.count_nonzero(ref.pool_k()[1]) == 0   # the idle rollout's slots: still the zero fill
    graph.close()
    for r in (ref, on_stream, graphed):
        r.close()


def test_steps_with_no_active_rollout_change_nothing():
    """Calls whose active mask names no rollout enqueue nothing: RoPE and
    attention outputs keep their fill, every report is empty, pools and
    bookkeeping are unchanged (eager, finalize stream, and a graph, which
    then has no kernel node); the next active step matches a ring that never
    saw those calls."""
    wl = CASES["gqa_batch2"]
    B, C, D = wl.batch, wl.chunk, wl.n_denoise
    src = Source(wl)
    ring, ref = new_ring(wl), new_ring(wl)
    qs = [dev(src.batch_chunk([0] * B, C, s, "q")) for s in range(D)]
    ks = [dev(src.batch_chunk([0] * B, C, s, "k")) for s in range(D)]
    vs = [dev(src.batch_chunk([0] * B, C, s, "v")) for s in range(D)]
    for r in (ring, ref):
        r.rollout_step(qs, ks, vs, C)
    torch.cuda.synchronize()
    none = [0] * B
    pool_k, pool_v = ring.pool_k().clone(), ring.pool_v().clone()
    views = [ring.view(b) for b in range(B)]
    fill = torch.full_like(qs[0], 7.0)
    empty = [{"written": [], "evicted": []}] * B

    y = ring.rope3d(qs[0], C, y=fill.clone(), active=none)
    y2, y3 = ring.rope3d_pair(qs[0], ks[0], C, y=fill.clone(), y2=torch.full_like(ks[0], 7.0), active=none)
    o = ring.chunk_attn(qs[0], ks[0], vs[0], C, out=fill.clone(), active=none)
    assert torch.equal(y, fill) and torch.equal(y2, fill) and torch.equal(o, fill)
    assert torch.count_nonzero(y3 != 7.0) == 0
    assert ring.append_evict(ks[-1], vs[-1], C, active=none) == empty
    outs = [fill.clone() for _ in range(D)]
    _, reps = ring.rollout_step(qs, ks, vs, C, outs=outs, active=none)
    assert reps == empty and all(torch.equal(x, fill) for x in outs)
    fin = torch.cuda.Stream()
    _, reps = ring.rollout_step(qs, ks, vs, C, outs=outs, active=none, finalize_stream=fin)
    assert reps == empty
    g_outs = [fill.clone() for _ in range(D)]
    graph = ring.rollout_graph(qs, ks, vs, C, outs=g_outs, active=none)
    for _ in range(3):
        _, reps = graph.launch()
        assert reps == empty
        torch.cuda.synchronize()
    graph.close()
    torch.cuda.current_stream().wait_stream(fin)
    torch.cuda.synchronize()
    assert all(torch.equal(x, fill) for x in outs + g_outs)
    assert torch.equal(ring.pool_k(), pool_k) and torch.equal(ring.pool_v(), pool_v)
    assert [ring.view(b) for b in range(B)] == views

    qs2 = [dev(src.batch_chunk([C] * B, C, s, "q")) for s in range(D)]
    ks2 = [dev(src.batch_chunk([C] * B, C, s, "k")) for s in range(D)]
    vs2 = [dev(src.batch_chunk([C] * B, C, s, "v")) for s in range(D)]
    o_a, rep_a = ring.rollout_step(qs2, ks2, vs2, C)
    o_b, rep_b = ref.rollout_step(qs2, ks2, vs2, C)
    torch.cuda.synchronize()
    assert rep_a == rep_b
    assert all(torch.equal(a, b) for a, b in zip(o_a, o_b))
    assert torch.equal(ring.pool_k(), ref.pool_k()) and torch.equal(ring.pool_v(), ref.pool_v())
    ring.close()
    ref.close()
