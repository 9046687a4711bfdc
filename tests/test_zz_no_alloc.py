"""The allocation-free attention entry point (wm_chunk_attn_noalloc) on the GPU.

It must give exactly what wm_chunk_attn gives with a large enough
workspace -- same launches, same key-range split, same output bits -- while
its split partials live in the library's static per-GPU scratch.  Two calls
in a row, the second smaller, show that one call's leftovers do not leak into
the next; a call whose split would need more than the scratch holds is
refused before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import autoregressive_video_world_amd as wm
from autoregressive_video_world_amd.binding import WMError
from gpu_util import host

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20


def filled_ring(hq, hkv, d, fh, fw, n_sink, window, n_fill, seed):
    ring = wm.KVRing(1, hq, hkv, d, fh, fw, n_sink, window, 1, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed)
    ft = fh * fw
    for _ in range(n_fill):
        k = torch.randn(1, ft, hkv, d, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(1, ft, hkv, d, device="cuda", generator=g).to(torch.bfloat16)
        ring.append_evict(k, v, 1)
    q = torch.randn(1, ft, hq, d, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(1, ft, hkv, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(1, ft, hkv, d, device="cuda", generator=g).to(torch.bfloat16)
    return ring, q, k, v


def reference(ring, q, k, v):
    ws_bytes = ring.workspace_bytes(1)
    assert 0 < ws_bytes <= SCRATCH_BYTES, ws_bytes   # the case splits its key range
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    return ring.chunk_attn(q, k, v, 1, workspace=ws)


def test_noalloc_equals_chunk_attn_on_two_calls_in_a_row():
    # a 4/1-head GQA group over a full 1 + 6-frame window: 5 workgroups for
    # 2560 keys, so the launch splits its key range (partials in scratch)
    big = filled_ring(4, 1, 128, 16, 20, 1, 6, 9, seed=1)
    # then a smaller call: fewer queries, heads and keys (2080), d = 64 and
    # another split count
    small = filled_ring(2, 1, 64, 8, 10, 1, 24, 30, seed=2)
    outs = []
    for ring, q, k, v in (big, small):
        print("noalloc call: Hq %d, Hkv %d, d %d, %d tokens/frame, split workspace %d B"
              % (ring.hq, ring.hkv, ring.d, ring.ft, ring.workspace_bytes(1)), flush=True)
        got = ring.chunk_attn_noalloc(q, k, v, 1)
        torch.cuda.synchronize()
        ref = reference(ring, q, k, v)
        torch.cuda.synchronize()
        assert np.array_equal(host(got), host(ref)), "noalloc output differs from wm_chunk_attn"
        outs.append(got)
    # the first call again after the second: still the same bits
    ring, q, k, v = big
    again = ring.chunk_attn_noalloc(q, k, v, 1)
    torch.cuda.synchronize()
    assert np.array_equal(host(again), host(outs[0]))
    for ring, *_ in (big, small):
        ring.close()


def test_noalloc_refuses_a_split_larger_than_its_scratch(monkeypatch):
    # 16 heads x 3520 queries split 8 ways: 8 x 3520 x 16 x 128 fp32 partials
    # (230 MB) do not fit the 128 MiB scratch
    monkeypatch.setenv("WM_ATTN_SPLIT", "8")
    ring = wm.KVRing(1, 16, 16, 128, 44, 80, 1, 3, 1, device="cuda")
    assert ring.workspace_bytes(1) > SCRATCH_BYTES
    q = torch.zeros(1, 3520, 16, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(WMError) as e:
        ring.chunk_attn_noalloc(q, q, q, 1, out=out)
    assert e.value.name == "WM_E_CAPACITY"
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0)), "a refused call wrote its output"
    ring.close()
