"""GPU: the reset-at-window-boundary policy with a classifier-free-guidance
pair (DreamZero single-GPU page, "Sequential requests": at the
local-attention window boundary the old KV is released, the frame position
reset and a new window started; the scheduler runs CFG branches).

Two rollouts (the conditional and unconditional branch, each with its own
seeded data and cache) go through three windows: prefill of the
conditioning frame, generated frames until the window is full, then a
refused append (WM_E_CAPACITY, pool bytes unchanged), wm_kvring_reset at
origin 0 and a fresh conditioning prefill.  RoPE and pool bytes are
compared bit-exact and attention within tolerance against two fp64 oracles
that do the same resets.
"""

import numpy as np
import pytest
import torch

import autoregressive_video_world_amd as wm
from oracle.rollout import Rollout
from wm_synth import Source, Workload
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [1, 2])
def test_reset_window_cfg_pair(chunk):
    wl = Workload(301 + chunk, "reset_cfg", 2, 4, 2, 128, 6, 9, chunk, 1, 4, 1, 0, 2)
    src = Source(wl)
    B, S, W = 2, wl.n_sink, wl.window
    meta = wm.KVRing(B, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, S, W, chunk,
                     meta_only=True, evict_policy=wm.EVICT_RESET)
    pool = torch.zeros(meta.pool_bytes, dtype=torch.uint8, device="cuda")   # before create: the
    meta.close()                                                            # tables live in the pool
    ring = wm.KVRing(B, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, S, W, chunk,
                     evict_policy=wm.EVICT_RESET, pool=pool)
    oracles = [Rollout(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, S, W)
               for _ in range(B)]
    seq = 0   # data of each window differs: the frame index fed to the source keeps counting

    def commit(k_np, v_np, n):
        reps = ring.append_evict(dev(k_np), dev(v_np), n)
        for b in range(B):
            written, evicted = oracles[b].commit(k_np[b], v_np[b], n)
            assert reps[b] == {"written": written, "evicted": evicted}
            assert evicted == []

    def check_pool():
        pk, pv = host(ring.pool_k()), host(ring.pool_v())
        for b in range(B):
            for f, slot, t in oracles[b].retained():
                kb, vb = oracles[b].cache[f]
                assert np.array_equal(pk[b, slot], kb.transpose(1, 0, 2)), (b, f)
                assert np.array_equal(pv[b, slot], vb.transpose(1, 0, 2)), (b, f)

    for window in range(3):
        # conditioning frame(s): prefill, no attention
        n0s = [seq] * B
        commit(src.batch_chunk(n0s, 1, -1, "k"), src.batch_chunk(n0s, 1, -1, "v"), 1)
        seq += 1
        while oracles[0].n_committed + chunk <= S + W:
            n0s = [seq] * B
            for s in range(wl.n_denoise):
                q_np = src.batch_chunk(n0s, chunk, s, "q")
                k_np = src.batch_chunk(n0s, chunk, s, "k")
                v_np = src.batch_chunk(n0s, chunk, s, "v")
                q_rot = ring.rope3d(dev(q_np), chunk)
                k_rot = ring.rope3d(dev(k_np), chunk)
                out = host(ring.chunk_attn(q_rot, k_rot, dev(v_np), chunk))
                qr, kr = host(q_rot), host(k_rot)
                for b in range(B):
                    ref_q, ref_k, ref_o = oracles[b].denoise_step(q_np[b], k_np[b], v_np[b], chunk)
                    assert np.array_equal(qr[b], ref_q) and np.array_equal(kr[b], ref_k)
                    assert_close(out[b], ref_o, "window %d frame %d b %d s %d" % (window, seq, b, s))
            commit(k_np, v_np, chunk)
            check_pool()
            seq += chunk
        # the window is full: an append is refused and leaves every byte as it was
        before = ring.pool.clone()
        with pytest.raises(wm.WMError) as e:
            ring.append_evict(dev(src.batch_chunk([seq] * B, chunk, -1, "k")),
                              dev(src.batch_chunk([seq] * B, chunk, -1, "v")), chunk)
        assert e.value.name == "WM_E_CAPACITY"
        torch.cuda.synchronize()
        assert torch.equal(before, ring.pool)
        # new window: release, positions restart
        for b in range(B):
            ring.reset(b, 0)
            oracles[b].reset(0)
        assert ring.view(0)["retained"] == []
    ring.close()


@pytest.mark.parametrize("kind", ["launch", "attn", "append"])
def test_refused_launch_mid_step_then_reset(kind, monkeypatch):
    """A launch the runtime refuses (forced with WM_FAULT_INJECT) inside a
    rollout step whose append would evict: the step fails with WM_E_HIP, the
    bookkeeping and the pool bytes are unchanged (the append is the only
    launch that writes the pool), and after wm_kvring_reset the rollouts
    continue exactly as fresh oracle sequences."""
    wl = Workload(311, "fault", 2, 4, 2, 64, 5, 7, 2, 1, 3, 0, 0, 2)
    src = Source(wl)
    B, S, W, C, D = 2, wl.n_sink, wl.window, wl.chunk, wl.n_denoise
    ring = wm.KVRing(B, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, S, W, C)
    oracles = [Rollout(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, S, W)
               for _ in range(B)]
    seq = 0
    while seq < S + W:   # fill sinks and window
        n = min(C, S + W - seq)
        ring.append_evict(dev(src.batch_chunk([seq] * B, n, -1, "k")),
                          dev(src.batch_chunk([seq] * B, n, -1, "v")), n)
        seq += n

    def step_inputs(n0):
        return [[dev(src.batch_chunk([n0] * B, C, s, x)) for s in range(D)] for x in "qkv"]

    views = [ring.view(b) for b in range(B)]
    torch.cuda.synchronize()
    pool = ring.pool.clone()
    qs, ks, vs = step_inputs(seq)
    monkeypatch.setenv("WM_FAULT_INJECT", kind)
    with pytest.raises(wm.WMError) as e:
        ring.rollout_step(qs, ks, vs, C)
    monkeypatch.delenv("WM_FAULT_INJECT")
    assert e.value.name == "WM_E_HIP"
    assert [ring.view(b) for b in range(B)] == views
    torch.cuda.synchronize()
    assert torch.equal(pool, ring.pool)

    # recovery: new sequences at new origins, one conditioning frame, two steps
    for b in range(B):
        ring.reset(b, 1000 + 7 * b)
        oracles[b].reset(1000 + 7 * b)
    k_np, v_np = src.batch_chunk([seq] * B, 1, -1, "k"), src.batch_chunk([seq] * B, 1, -1, "v")
    ring.append_evict(dev(k_np), dev(v_np), 1)
    for b in range(B):
        oracles[b].commit(k_np[b], v_np[b], 1)
    seq += 1
    for _ in range(2):
        qs, ks, vs = step_inputs(seq)
        outs, reps = ring.rollout_step(qs, ks, vs, C)
        for s in range(D):
            got = host(outs[s])
            for b in range(B):
                _, _, ref = oracles[b].denoise_step(host(qs[s])[b], host(ks[s])[b], host(vs[s])[b], C)
                assert_close(got[b], ref, "%s: recovered step at frame %d, b %d, s %d" % (kind, seq, b, s))
        for b in range(B):
            written, evicted = oracles[b].commit(host(ks[-1])[b], host(vs[-1])[b], C)
            assert reps[b] == {"written": written, "evicted": evicted}
        seq += C
    ring.close()


def test_rope_tensor_size_limit_on_a_device_ring():
    """wm_rope3d takes its own head count: a tensor of 2^31 elements or more
    per rollout (32-bit offsets in the kernel) is refused before any launch."""
    import ctypes
    ring = wm.KVRing(1, 8, 8, 128, 256, 256, 1, 1, 1)   # Ft = 2^16
    L = wm.lib()
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    assert L.wm_rope3d(ring._h, p, p, 256, 1, None, None, None) == 2    # 2^16 * 256 * 128 = 2^31
    assert b"2^31" in L.wm_last_error()
    assert L.wm_rope3d_pair(ring._h, p, p, 8, p, p, 256, 1, None, None, None) == 2
    torch.cuda.synchronize()
    ring.close()


def test_reset_policy_refuses_whole_steps_before_any_launch():
    """With WM_EVICT_RESET and the window full, wm_rollout_step and a graph
    launch fail with WM_E_CAPACITY before anything is enqueued: outputs keep
    their fill, bookkeeping and pool bytes are unchanged; after a reset both
    run again."""
    wl = Workload(320, "reset_step", 1, 4, 2, 128, 5, 6, 1, 1, 2, 0, 0, 2)
    src = Source(wl)
    B, C, D = 1, wl.chunk, wl.n_denoise
    ring = wm.KVRing(B, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, wl.n_sink,
                     wl.window, C, evict_policy=wm.EVICT_RESET)
    qs = [dev(src.batch_chunk([0], C, s, "q")) for s in range(D)]
    ks = [dev(src.batch_chunk([0], C, s, "k")) for s in range(D)]
    vs = [dev(src.batch_chunk([0], C, s, "v")) for s in range(D)]
    outs = [torch.full_like(q, 5.0) for q in qs]
    graph_outs = [torch.full_like(q, 5.0) for q in qs]
    graph = ring.rollout_graph(qs, ks, vs, C, outs=graph_outs)
    for _ in range(wl.n_sink + wl.window):        # fill sinks and window exactly
        ring.rollout_step(qs, ks, vs, C)
    torch.cuda.synchronize()
    view, pool = ring.view(0), ring.pool.clone()
    with pytest.raises(wm.WMError) as e1:
        ring.rollout_step(qs, ks, vs, C, outs=outs)
    with pytest.raises(wm.WMError) as e2:
        graph.launch()
    assert e1.value.name == "WM_E_CAPACITY" and e2.value.name == "WM_E_CAPACITY"
    torch.cuda.synchronize()
    assert ring.view(0) == view and torch.equal(ring.pool, pool)
    five = torch.full_like(qs[0], 5.0)
    assert all(torch.equal(o, five) for o in outs + graph_outs)
    ring.reset(0, 0)
    out_step, _ = ring.rollout_step(qs, ks, vs, C, outs=outs)
    graph.launch()
    torch.cuda.synchronize()
    assert ring.view(0)["n_committed"] == 2
    assert not any(torch.equal(o, five) for o in outs + graph_outs)
    graph.close()
    ring.close()
