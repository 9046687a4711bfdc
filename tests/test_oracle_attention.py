"""Pins for the oracle's chunk attention and rollout (CPU).

Special cases that reduce to PyTorch's scaled_dot_product_attention (CPU,
float64), brute-force loops, the masked full-sequence formulation, and
invariants (key-order, GQA, Q = 0, single key, linearity in V).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, bf16
from oracle.rollout import Rollout
from wm_synth import WORKLOADS, Source, to_bf16_bits


def sdpa(q, k, v, mask=None):
    """PyTorch reference on (N, H, d) float64 arrays."""
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    if kt.shape[0] != qt.shape[0]:
        rep = qt.shape[0] // kt.shape[0]
        kt = kt.repeat_interleave(rep, dim=0)
        vt = vt.repeat_interleave(rep, dim=0)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    return o.permute(1, 0, 2).numpy()


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, k, v, scale):
    Nq, Hq, d = q.shape
    Nk, Hkv, _ = k.shape
    out = np.zeros_like(q)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(Nq):
            sc = [sum(q[i, h, e] * k[j, g, e] for e in range(d)) * scale for j in range(Nk)]
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            z = sum(ex)
            for e in range(d):
                out[i, h, e] = sum(ex[j] * v[j, g, e] for j in range(Nk)) / z
    return out


def test_plain_attention_equals_sdpa():
    q, k, v = rand((40, 4, 64), 0), rand((70, 4, 64), 1), rand((70, 4, 64), 2)
    assert np.allclose(attention.attend(q, k, v), sdpa(q, k, v), atol=1e-13, rtol=0)


def test_gqa_equals_repeated_heads():
    q, k, v = rand((30, 8, 32), 3), rand((50, 2, 32), 4), rand((50, 2, 32), 5)
    kr = np.repeat(k, 4, axis=1)
    vr = np.repeat(v, 4, axis=1)
    assert np.allclose(attention.attend(q, k, v), attention.attend(q, kr, vr), atol=1e-14, rtol=0)
    assert np.allclose(attention.attend(q, k, v), sdpa(q, k, v), atol=1e-13, rtol=0)


def test_brute_force_tiny():
    q, k, v = rand((5, 2, 8), 6), rand((9, 2, 8), 7), rand((9, 2, 8), 8)
    sc = 1 / math.sqrt(8)
    assert np.allclose(attention.attend(q, k, v), brute_force(q, k, v, sc), atol=1e-13, rtol=0)


def test_key_permutation_invariance():
    q, k, v = rand((20, 2, 64), 9), rand((80, 2, 64), 10), rand((80, 2, 64), 11)
    perm = np.random.default_rng(12).permutation(80)
    a = attention.attend(q, k, v)
    b = attention.attend(q, k[perm], v[perm])
    assert np.allclose(a, b, atol=1e-12, rtol=0)


def test_zero_query_gives_mean_of_values():
    k, v = rand((33, 2, 16), 13), rand((33, 2, 16), 14)
    q = np.zeros((4, 2, 16))
    o = attention.attend(q, k, v)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14, rtol=0)


def test_single_key_gives_value_exactly():
    q, k, v = rand((3, 2, 16), 15), rand((1, 2, 16), 16), rand((1, 2, 16), 17)
    o = attention.attend(q, k, v)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))


def test_linear_in_values():
    q, k = rand((10, 2, 16), 18), rand((25, 2, 16), 19)
    v1, v2 = rand((25, 2, 16), 20), rand((25, 2, 16), 21)
    a = attention.attend(q, k, 2.5 * v1 - v2)
    b = 2.5 * attention.attend(q, k, v1) - attention.attend(q, k, v2)
    assert np.allclose(a, b, atol=1e-13, rtol=0)


def test_masked_formulation_equals_sdpa_with_mask():
    q, k, v = rand((12, 2, 16), 22), rand((30, 2, 16), 23), rand((30, 2, 16), 24)
    mask = np.random.default_rng(25).random((12, 30)) < 0.5
    mask[:, 0] = True
    assert np.allclose(attention.attend_masked(q, k, v, mask), sdpa(q, k, v, mask), atol=1e-13, rtol=0)


def run_rollout(S, W, C, P, N, D, Hq=2, Hkv=2, d=32, fh=2, fw=3, seed=0, t0=0):
    """Drive the oracle rollout; also keep every frame's committed K/V and the
    per-chunk step inputs so the full-sequence formulation can be rebuilt."""
    rng = np.random.default_rng(seed)
    ft = fh * fw

    def draw(n, H):
        return to_bf16_bits(rng.standard_normal((n * ft, H, d)).astype(np.float32))

    ro = Rollout(Hq, Hkv, d, fh, fw, S, W, t0=t0)
    committed_k, committed_v = {}, {}
    records = []
    if P:
        kp, vp = draw(P, Hkv), draw(P, Hkv)
        kr = ro.rope(kp, P)
        ro.commit(kp, vp, P)
        for j in range(P):
            committed_k[j] = kr[j * ft:(j + 1) * ft]
            committed_v[j] = vp[j * ft:(j + 1) * ft]
    left = N
    while left > 0:
        c = min(C, left)
        n0 = ro.n_committed
        for s in range(D):
            q, k, v = draw(c, Hq), draw(c, Hkv), draw(c, Hkv)
            q_rot, k_rot, o = ro.denoise_step(q, k, v, c)
            records.append((n0, c, q_rot, k_rot, v, o))
        kr = k_rot
        ro.commit(k, v, c)
        for j in range(c):
            committed_k[n0 + j] = kr[j * ft:(j + 1) * ft]
            committed_v[n0 + j] = v[j * ft:(j + 1) * ft]
        left -= c
    return ro, records, committed_k, committed_v


def full_sequence_output(n0, c, q_rot, k_rot, v, committed_k, committed_v, S, W, ft):
    """Masked attention over every frame committed so far + the current chunk."""
    frames = list(range(n0 + c))
    ks, vs, fr = [], [], []
    for f in frames:
        if f >= n0:
            j = f - n0
            ks.append(k_rot[j * ft:(j + 1) * ft])
            vs.append(v[j * ft:(j + 1) * ft])
        else:
            ks.append(committed_k[f])
            vs.append(committed_v[f])
        fr += [f] * ft
    mask = np.array([[attention.frame_visible(f, n0, c, S, W) for f in fr]] * (c * ft))
    return attention.attend_masked(bf16.bits_to_f64(q_rot), bf16.bits_to_f64(np.concatenate(ks)),
                                   bf16.bits_to_f64(np.concatenate(vs)), mask)


@pytest.mark.parametrize("S,W,C,P,N,D", [(1, 3, 1, 0, 9, 2), (1, 2, 2, 1, 9, 2), (2, 3, 3, 1, 11, 1),
                                         (0, 2, 1, 0, 6, 1), (1, 0, 2, 0, 5, 1)])
def test_streaming_equals_full_sequence_masked(S, W, C, P, N, D):
    ro, records, ck, cv = run_rollout(S, W, C, P, N, D)
    for n0, c, q_rot, k_rot, v, o in records:
        ref = full_sequence_output(n0, c, q_rot, k_rot, v, ck, cv, S, W, ro.ft)
        assert np.allclose(o, ref, atol=1e-12, rtol=0)


def test_no_eviction_equals_block_causal_sdpa():
    """Rollout no longer than sinks + window: plain block-causal attention."""
    S, W, C, N = 1, 6, 2, 6
    ro, records, ck, cv = run_rollout(S, W, C, 0, N, 1, Hq=4, Hkv=2)
    ft = ro.ft
    for n0, c, q_rot, k_rot, v, o in records:
        ks = [ck[f] for f in range(n0)] + [k_rot]
        vs = [cv[f] for f in range(n0)] + [v]
        kk = bf16.bits_to_f64(np.concatenate(ks))
        vv = bf16.bits_to_f64(np.concatenate(vs))
        ref = sdpa(bf16.bits_to_f64(q_rot), kk, vv)
        assert kk.shape[0] == (n0 + c) * ft
        assert np.allclose(o, ref, atol=1e-13, rtol=0)


def test_no_cache_equals_plain_bidirectional():
    ro, records, _, _ = run_rollout(0, 0, 2, 0, 4, 1)
    for n0, c, q_rot, k_rot, v, o in records:
        ref = sdpa(bf16.bits_to_f64(q_rot), bf16.bits_to_f64(k_rot), bf16.bits_to_f64(v))
        assert np.allclose(o, ref, atol=1e-13, rtol=0)


def test_tiny_workload_brute_force():
    """The whole tiny rollout, attention recomputed with Python loops."""
    wl = WORKLOADS[1]
    src = Source(wl)
    ro = Rollout(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.frame_h, wl.frame_w, wl.n_sink, wl.window)
    sc = 1 / math.sqrt(wl.head_dim)
    for n0 in range(4):                   # first 4 frames keep the brute force quick
        for s in range(wl.n_denoise):
            q, k, v = (src.chunk(0, n0, 1, s, kind) for kind in "qkv")
            q_rot, k_rot, o = ro.denoise_step(q, k, v, 1)
            kb, vb = ro.keys_values(k_rot, v, 1)
            ref = brute_force(bf16.bits_to_f64(q_rot)[:4], bf16.bits_to_f64(kb), bf16.bits_to_f64(vb), sc)
            assert np.allclose(o[:4], ref, atol=1e-13, rtol=0)
        ro.commit(k, v, 1)


def test_commit_stores_final_step_keys_rotated_at_absolute_t():
    ro, records, ck, cv = run_rollout(1, 2, 1, 0, 6, 2, t0=100)
    for f, slot, t in ro.retained():
        assert t == 100 + f
        kb, vb = ro.cache[f]
        assert np.array_equal(kb, ck[f]) and np.array_equal(vb, cv[f])
    assert [f for f, _, _ in ro.retained()] == [0, 4, 5]


def test_shift_of_all_positions_changes_little():
    """A constant shift of t changes O only through fp32 table rounding."""
    _, r0, _, _ = run_rollout(1, 2, 1, 0, 4, 1, seed=3, t0=0)
    _, r1, _, _ = run_rollout(1, 2, 1, 0, 4, 1, seed=3, t0=37)
    for a, b in zip(r0, r1):
        assert np.max(np.abs(a[5] - b[5])) < 5e-2


def test_reset_starts_a_fresh_sequence_at_new_origin():
    """DreamZero page, "Sequential requests": a new request resets the cache
    and the start frame.  After a reset to origin t0, the rollout is the one a
    new rollout at t0 produces from the same inputs (RoPE bits, keys, O bit
    for bit); its outputs equal block-causal attention over the post-reset
    frames alone; committed frames carry t = t0 + frame; and the cache holds
    exactly the retained frames (nothing of the old sequence)."""
    S, W, C, D = 1, 2, 1, 2
    Hq = Hkv = 2
    d, fh, fw = 32, 2, 3
    ft = fh * fw
    rng = np.random.default_rng(41)

    def draw(n, H):
        return to_bf16_bits(rng.standard_normal((n * ft, H, d)).astype(np.float32))

    used = Rollout(Hq, Hkv, d, fh, fw, S, W, t0=5)
    for _ in range(6):                    # an old sequence, past eviction
        used.denoise_step(draw(1, Hq), draw(1, Hkv), draw(1, Hkv), 1)
        used.commit(draw(1, Hkv), draw(1, Hkv), 1)
    t0 = 1000
    used.reset(t0)
    fresh = Rollout(Hq, Hkv, d, fh, fw, S, W, t0=t0)
    assert used.n_committed == 0 and used.retained() == [] and used.cache == {}
    committed_k, committed_v = {}, {}
    for n0 in range(4):                   # sink + window fill + first eviction
        step_in = [(draw(C, Hq), draw(C, Hkv), draw(C, Hkv)) for _ in range(D)]
        for q, k, v in step_in:
            qa, ka, oa = used.denoise_step(q, k, v, C)
            qb, kb, ob = fresh.denoise_step(q, k, v, C)
            assert np.array_equal(qa, qb) and np.array_equal(ka, kb)
            assert np.array_equal(oa, ob)
            ks_a, vs_a = used.keys_values(ka, v, C)
            ks_b, vs_b = fresh.keys_values(kb, v, C)
            assert np.array_equal(ks_a, ks_b) and np.array_equal(vs_a, vs_b)
            # block-causal attention over the new sequence's frames only
            ref = full_sequence_output(n0, C, qa, ka, v, committed_k, committed_v, S, W, ft)
            assert np.allclose(oa, ref, atol=1e-12, rtol=0)
        assert used.commit(k, v, C) == fresh.commit(k, v, C)
        committed_k[n0], committed_v[n0] = ka, v
        assert used.retained() == fresh.retained()
        assert all(t == t0 + f for f, _, t in used.retained())
        assert sorted(used.cache) == [f for f, _, _ in used.retained()]
