"""Whole rollouts at full shape on the GPU: the Self-Forcing 1.3B (sf13b),
driving (drive) and 15B MoT (mot15) workloads from an empty ring.

Each rollout runs through ``wm_rollout_step`` chunk by chunk -- the window
filling, the first evictions and steady state, the conditioning prefill of
the drive and mot15 workloads (Cosmos3-H-Dreams model card, "Model
Architecture" / "Inference"; AlpaDreams write-up, VIII), and sf13b's short
last chunk of 2 frames (3120 queries) -- so every launch shape the library
picks on the way (grid, key-range split) is exercised at its real size.

The oracle follows three kv heads and one q head of each (attention and RoPE
act on every head alone, so a head subset of the inputs is an exact smaller
rollout): on every denoise step it gives 256 query rows (first 64, last 64,
128 seeded random) of those heads, compared with the library's output under
the stated tolerance; after every append the report (frames, slots,
positions, evictions) is compared bit for bit, and so are the pool bytes of
every slot written, on the followed kv heads; at the end every retained slot
is compared again.  The pool starts filled with 0xFF.
"""

import numpy as np
import pytest
import torch

import autoregressive_video_world_amd as wm
from oracle.rollout import Rollout
from wm_synth import WORKLOADS, Source
from gpu_util import assert_close, dev, host

pytestmark = pytest.mark.gpu


def sample_rows(nq, seed):
    rng = np.random.default_rng(seed)
    mid = np.arange(64, nq - 64)
    return np.concatenate([np.arange(64), rng.choice(mid, 128, replace=False), np.arange(nq - 64, nq)])


@pytest.mark.timeout(400)
@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_whole_rollout_at_full_shape(cfg):
    wl = WORKLOADS[cfg]
    src = Source(wl)
    group = wl.n_q_heads // wl.n_kv_heads
    gsel = [0, wl.n_kv_heads // 2 - 1, wl.n_kv_heads - 1]
    hsel = [g * group + g % group for g in gsel]
    ft, D = wl.ft, wl.n_denoise

    pool_bytes = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                           wl.n_sink, wl.window, wl.chunk, meta_only=True).pool_bytes
    pool = torch.full((pool_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ring = wm.KVRing(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w,
                     wl.n_sink, wl.window, wl.chunk, pool=pool)
    ro = Rollout(len(hsel), len(gsel), wl.head_dim, wl.frame_h, wl.frame_w, wl.n_sink, wl.window)
    ws_bytes = ring.workspace_bytes(wl.chunk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    print("%s: %d chunks, split workspace %d B" % (wl.name, len(wl.chunks()), ws_bytes), flush=True)

    def check_written(rep, written):
        pk, pv = ring.pool_k(), ring.pool_v()
        for frame, slot, t in written:
            if slot < 0:
                continue
            kb, vb = ro.cache[frame]
            assert np.array_equal(host(pk[0, slot, gsel]), kb.transpose(1, 0, 2)), ("K", frame, slot)
            assert np.array_equal(host(pv[0, slot, gsel]), vb.transpose(1, 0, 2)), ("V", frame, slot)

    if wl.prefill:
        k = src.chunk(0, 0, wl.prefill, -1, "k")
        v = src.chunk(0, 0, wl.prefill, -1, "v")
        rep = ring.append_evict(dev(k[None]), dev(v[None]), wl.prefill)
        written, evicted = ro.commit(k[:, gsel], v[:, gsel], wl.prefill)
        assert rep[0] == {"written": written, "evicted": evicted}
        check_written(rep, written)

    worst = 0.0
    for ci, c in enumerate(wl.chunks()):
        n0 = ro.n_committed
        nq = c * ft
        draws = [{kind: src.chunk(0, n0, c, s, kind) for kind in "qkv"} for s in range(D)]
        outs, reps = ring.rollout_step([dev(d["q"][None]) for d in draws], [dev(d["k"][None]) for d in draws],
                                       [dev(d["v"][None]) for d in draws], c, workspace=ws)
        rows = sample_rows(nq, 1000 * cfg + ci)
        for s, d in enumerate(draws):
            _, _, ref = ro.denoise_step(d["q"][:, hsel], d["k"][:, gsel], d["v"][:, gsel], c, rows=rows)
            got = host(outs[s][0])[rows][:, hsel]
            mx, _, _ = assert_close(got, ref, "%s chunk %d (frames %d..%d) step %d"
                                    % (wl.name, ci, n0, n0 + c - 1, s))
            worst = max(worst, mx)
        written, evicted = ro.commit(draws[-1]["k"][:, gsel], draws[-1]["v"][:, gsel], c)
        assert reps[0] == {"written": written, "evicted": evicted}, (ci, reps[0], written, evicted)
        check_written(reps, written)
    # every retained slot once more, and nothing written outside them
    assert ring.view(0)["retained"] == ro.retained()
    check_written(None, ro.retained())
    used = {slot for _, slot, _ in ro.retained()}
    pk = host(ring.pool_k())
    for slot in range(ring.slots):
        if slot not in used:
            assert np.all(pk[0, slot] == 0xFFFF), slot
    print("%s: every step of %d chunks checked, worst max |O - oracle| %.3g"
          % (wl.name, len(wl.chunks()), worst), flush=True)
    ring.close()
