"""GPU: the long bounded rollout -- 8 rollouts x 10,000 frames through the ring.

Rollout b is admitted at global step 7b, prefills frame 0 (the sink) and then
generates frames 1..10,000 one per step (positions reach t = 10,000).  Frames
come from a pool of 17 seeded draws per tensor kind (entry (7919 b + 31 n + s)
mod 17), so the oracle can rebuild any frame.  Checked:
* every append report (written frame, slot, t; evicted ids) bit-exact against
  the oracle deque, for every rollout and step, and the final ring views;
* device memory is flat: allocated and free bytes after the window first
  fills equal those after the last step (the library allocates nothing);
* at sampled frames (1, 2, 5, 5000, 9999, 10000) of rollouts 0, 3 and 7:
  RoPE output bit-exact and attention within tolerance on 256 query rows of
  q heads 0 and 15, from full-batch calls (rollouts at different fill levels
  in one launch);
* at the end, stored K (rotated at t up to 10,000) and V bytes of every
  retained frame of every rollout, for kv heads 0, 7 and 15.
"""

import gc

import numpy as np
import pytest
import torch

import autoregressive_video_world_amd as wm
from oracle import attention as oatt
from oracle import bf16 as obf16
from oracle import rope as orope
from oracle.ring import DequeRing
from wm_synth import POOL_ENTRIES, WORKLOADS, Source
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu

CHECK_FRAMES = (1, 2, 5, 5000, 9999, 10000)
CHECK_ROLLOUTS = (0, 3, 7)
ATTN_HEADS = [0, 15]
KV_HEADS = [0, 7, 15]
N_ROWS = 256


def test_long_rollout_10000_frames_bounded_and_exact():
    wl = WORKLOADS[5]
    B, ft, H, d = wl.batch, wl.ft, wl.n_q_heads, wl.head_dim
    S, W, P, N, D, stagger = wl.n_sink, wl.window, wl.prefill, wl.n_gen, wl.n_denoise, wl.stagger
    assert wl.n_kv_heads == H and wl.chunk == 1
    src = Source(wl)
    pools = {kind: torch.stack([dev(src.pool_entry(e, kind)) for e in range(POOL_ENTRIES)])
             for kind in "qkv"}

    meta = wm.KVRing(B, H, H, d, wl.frame_h, wl.frame_w, S, W, 1, meta_only=True)
    pool = torch.full((meta.pool_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    meta.close()
    ring = wm.KVRing(B, H, H, d, wl.frame_h, wl.frame_w, S, W, 1, pool=pool)
    oracle_rings = [DequeRing(S, W) for _ in range(B)]

    bufs = {kind: torch.empty(B, ft, H, d, dtype=torch.bfloat16, device="cuda") for kind in "qkv"}
    q_rot = torch.empty_like(bufs["q"])
    k_rot = torch.empty_like(bufs["k"])
    out = torch.empty_like(bufs["q"])
    rows = np.sort(np.random.default_rng(5).choice(ft, N_ROWS, replace=False))

    def gather(entries, kinds="qkv"):
        for kind in kinds:
            idx = torch.tensor(entries, dtype=torch.long, device="cuda")
            torch.index_select(pools[kind], 0, idx, out=bufs[kind])

    rot_cache = {}

    def k_rot_oracle(e, f, heads):
        key = (e, f, tuple(heads))
        if key not in rot_cache:
            t, hh, ww = orope.token_positions(1, wl.frame_h, wl.frame_w, f)
            rot_cache[key] = orope.rotate(src.pool_entry(e, "k")[:, heads, :], t, hh, ww)
        return rot_cache[key]

    def committed_step(f):
        return -1 if f < P else D - 1

    def check_attention(b, n, s, got_q, got_k, got_o):
        vis = oatt.visible_frames(n, 1, S, W)
        assert vis[:-1] == oracle_rings[b].retained_frames(), (b, n)
        ks, vs = [], []
        for f in vis:
            e = src.pool_index(b, f, s if f == n else committed_step(f))
            ks.append(k_rot_oracle(e, f, ATTN_HEADS))
            vs.append(src.pool_entry(e, "v")[:, ATTN_HEADS, :])
        e = src.pool_index(b, n, s)
        q_want = orope.rotate(src.pool_entry(e, "q")[rows][:, ATTN_HEADS, :],
                              np.full(N_ROWS, n), rows // wl.frame_w, rows % wl.frame_w)
        assert np.array_equal(got_q[b][rows][:, ATTN_HEADS, :], q_want), ("q_rot", b, n, s)
        assert np.array_equal(got_k[b][:, ATTN_HEADS, :], ks[-1]), ("k_rot", b, n, s)
        want = oatt.attend(obf16.bits_to_f64(q_want), obf16.bits_to_f64(np.concatenate(ks)),
                           obf16.bits_to_f64(np.concatenate(vs)))
        assert_close(got_o[b][rows][:, ATTN_HEADS, :], want, "rollout %d frame %d step %d" % (b, n, s))

    total = P + N
    n_steps = stagger * (B - 1) + total
    mem_mark = None
    mark_step = stagger * (B - 1) + S + W + 1
    n_checked = 0
    for g in range(n_steps):
        n = [g - stagger * b for b in range(B)]
        active = [0 <= n[b] < total for b in range(B)]
        # generate(): sampled denoise steps, full batch, compared on sampled rollouts
        check = [b for b in CHECK_ROLLOUTS if active[b] and n[b] in CHECK_FRAMES]
        if check:
            for s in range(D):
                gather([src.pool_index(b, n[b], s) if active[b] else 0 for b in range(B)])
                ring.rope3d(bufs["q"], 1, y=q_rot, active=active)
                ring.rope3d(bufs["k"], 1, y=k_rot, active=active)
                ring.chunk_attn(q_rot, k_rot, bufs["v"], 1, out=out, active=active)
                got_q, got_k, got_o = host(q_rot), host(k_rot), host(out)
                for b in check:
                    check_attention(b, n[b], s, got_q, got_k, got_o)
                    n_checked += 1
        # finalize(): commit frame n[b] of every active rollout
        gather([src.pool_index(b, n[b], committed_step(n[b])) if active[b] else 0 for b in range(B)], "kv")
        reps = ring.append_evict(bufs["k"], bufs["v"], 1, active=active)
        for b in range(B):
            if active[b]:
                frame, slot, ev = oracle_rings[b].commit()
                assert frame == n[b]
                assert reps[b] == {"written": [(frame, slot, frame)], "evicted": ev}, (g, b)
            else:
                assert reps[b] == {"written": [], "evicted": []}, (g, b)
        if g == mark_step:
            # cyclic garbage (of this or earlier tests) is freed first, so
            # that only this rollout's own memory is compared
            gc.collect()
            torch.cuda.synchronize()
            mem_mark = (torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0])
    gc.collect()
    torch.cuda.synchronize()
    assert n_checked == len(CHECK_ROLLOUTS) * len(CHECK_FRAMES) * D
    assert (torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0]) == mem_mark

    pk, pv = host(ring.pool_k()), host(ring.pool_v())
    for b in range(B):
        view = ring.view(b)
        assert view["n_committed"] == total
        assert view["retained"] == [(f, s, f) for f, s in oracle_rings[b].retained()]
        assert oracle_rings[b].retained_frames() == [0, N - 2, N - 1, N]
        for f, slot in oracle_rings[b].retained():
            e = src.pool_index(b, f, committed_step(f))
            assert np.array_equal(pk[b, slot][KV_HEADS], k_rot_oracle(e, f, KV_HEADS).transpose(1, 0, 2)), (b, f)
            assert np.array_equal(pv[b, slot][KV_HEADS],
                                  src.pool_entry(e, "v")[:, KV_HEADS, :].transpose(1, 0, 2)), (b, f)
    ring.close()
