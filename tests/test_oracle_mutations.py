"""Mutation test of the oracle's pins (CPU).

Each case plants one plausible mistake in the oracle -- a wrong sign, a
swapped index or operand, an off-by-one, a dropped term, another RoPE or
rounding convention -- and runs the oracle's own pin tests (tests/
test_oracle_*.py) against the mutated oracle: at least one pin must fail.
Without a mutation every pin passes.  A mistake the pins could not see would
leave the oracle unpinned there.
"""

import math
from collections import deque

import numpy as np
import pytest

import test_oracle_attention as pins_attention
import test_oracle_ring as pins_ring
import test_oracle_rope as pins_rope
from oracle import attention, bf16, ring, rope
from oracle.rollout import Rollout


def _param_sets(f):
    """Keyword sets of a test function's stacked parametrize marks."""
    sets = [{}]
    for m in getattr(f, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names, values = m.args[0], m.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        sets = [dict(s, **dict(zip(names, v if len(names) > 1 else (v,)))) for s in sets for v in values]
    return sets


def first_failing_pin(modules):
    """Name of the first pin test that fails, or None when all pass."""
    for mod in modules:
        for name in sorted(n for n in dir(mod) if n.startswith("test_")):
            f = getattr(mod, name)
            for kw in _param_sets(f):
                try:
                    with np.errstate(all="ignore"):
                        f(**kw)
                except Exception:
                    return "%s.%s%s" % (mod.__name__, name, kw or "")
    return None


# ---- mutated copies of oracle functions (one mistake each) -----------------
def _rotate_f64(sign=1.0, swap_outputs=False, halves=False):
    def rotate_f64(x, t, h, w, theta=10000.0, rope_dims=None, round_fp32=True):
        T, H, d = x.shape
        cos, sin = rope.per_token_tables(t, h, w, d, theta, rope_dims, round_fp32)
        x0, x1 = (x[..., : d // 2], x[..., d // 2:]) if halves else (x[..., 0::2], x[..., 1::2])
        c, s = cos[:, None, :], sin[:, None, :]
        y0, y1 = x0 * c - sign * x1 * s, x0 * s + x1 * c
        if swap_outputs:
            y0, y1 = y1, y0
        y = np.empty_like(x)
        if halves:
            y[..., : d // 2], y[..., d // 2:] = y0, y1
        else:
            y[..., 0::2], y[..., 1::2] = y0, y1
        return y
    return rotate_f64


def _inv_freqs_wrong_width(theta, d_a):
    return [math.pow(theta, -(2.0 * j) / (d_a + 2)) for j in range(d_a // 2)]


def _token_positions(swap_hw=False, t_shift=0, one_grid=False):
    def token_positions(n_frames, frame_h, frame_w, t_first, n_views=1):
        fv = frame_h * frame_w
        ft = n_views * fv
        r = np.arange(n_frames * ft)
        t = t_first + t_shift + r // ft
        hw = (r % ft) if one_grid else (r % ft) % fv
        h, w = hw // frame_w, hw % frame_w
        if swap_hw:
            h, w = w, h
        return t.astype(np.int64), h.astype(np.int64), w.astype(np.int64)
    return token_positions


def _table_row_sin_is_cos(pos, theta, d_a, round_fp32=True):
    c = np.empty(d_a // 2)
    for j, f in enumerate(rope.inv_freqs(theta, d_a)):
        cv = math.cos(float(pos) * f)
        c[j] = float(np.float32(cv)) if round_fp32 else cv
    return c, c.copy()


def _per_token_tables_bands_twh(t, h, w, d, theta=10000.0, rope_dims=None, round_fp32=True):
    dt, dh, dw = rope.band_sizes(d, rope_dims)
    cos, sin = np.empty((len(t), d // 2)), np.empty((len(t), d // 2))
    col = 0
    for pos_arr, d_a in ((t, dt), (w, dw), (h, dh)):
        for i, p in enumerate(pos_arr):
            c, s = rope.table_row(int(p), theta, d_a, round_fp32)
            cos[i, col:col + d_a // 2], sin[i, col:col + d_a // 2] = c, s
        col += d_a // 2
    return cos, sin


def _table_row_fp64(pos, theta, d_a, round_fp32=True):
    c = np.empty(d_a // 2)
    s = np.empty(d_a // 2)
    for j, f in enumerate(rope.inv_freqs(theta, d_a)):
        c[j], s[j] = math.cos(float(pos) * f), math.sin(float(pos) * f)
    return c, s


_F64_TO_BITS = bf16.f64_to_bits


def _f64_to_bits_via_fp32(x):
    with np.errstate(over="ignore"):
        x32 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    return _F64_TO_BITS(x32)


def _commit_unrotated(self, k_raw_bits, v_bits, n_frames):
    written, evicted = [], []
    for j in range(n_frames):
        frame, slot, ev = self.ring.commit()
        for e in ev:
            del self.cache[e]
        evicted.extend(ev)
        written.append((frame, slot, self.t_of(frame)))
        if slot >= 0:
            sl = slice(j * self.ft, (j + 1) * self.ft)
            self.cache[frame] = (np.asarray(k_raw_bits[sl]).copy(), np.asarray(v_bits[sl]).copy())
    return written, evicted


def _bits_to_f64_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _attend_masked_inverted(q, k, v, mask, scale=None, heads=None):
    return _ATTEND_MASKED(q, k, v, ~np.asarray(mask), scale, heads)


_ATTEND_MASKED = attention.attend_masked


def _frame_visible_window_long(f, n0, n_frames, n_sink, window):
    in_chunk = n0 <= f < n0 + n_frames
    is_sink = f < n_sink and f < n0 + n_frames
    in_window = window > 0 and max(n_sink, n0 - window - 1) <= f < n0
    return in_chunk or is_sink or in_window


def _t_of_plus_one(self, frame):
    return self.t0 + frame + 1


def _keys_values_own_chunk_first(self, k_rot_chunk, v_chunk, n_frames):
    n0 = self.n_committed
    frames = attention.visible_frames(n0, n_frames, self.S, self.W)
    ks, vs = [], []
    for f in frames:
        if f >= n0:
            continue
        kb, vb = self.cache[f]
        ks.append(kb)
        vs.append(vb)
    # the chunk's keys paired with the values of the frame before them
    ks.append(k_rot_chunk)
    vs.append(np.roll(np.asarray(v_chunk), self.ft, axis=0))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def _f64_to_bits(mode):
    def f64_to_bits(x):
        x = np.asarray(x, dtype=np.float64)
        ax = np.abs(x)
        axf = np.where(np.isfinite(ax), ax, 0.0)
        _, e = np.frexp(axf)
        qexp = np.maximum(e - 8, -133)
        scaled = np.ldexp(axf, -qexp)
        n = np.trunc(scaled) if mode == "truncate" else np.floor(scaled + 0.5)
        y = np.ldexp(n, qexp)
        y = np.where(y >= 2.0 ** 128, np.inf, y)
        y = np.where(np.isinf(ax), np.inf, y)
        with np.errstate(over="ignore"):
            y32 = y.astype(np.float32)
        bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        bits = bits | np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
        return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)
    return f64_to_bits


def _attend(no_scale=False, gqa_mod=False, axis=1, values_are_keys=False):
    def attend(q, k, v, scale=None, heads=None):
        Nq, Hq, d = q.shape
        Nk, Hkv, _ = k.shape
        if Hq % Hkv:
            raise ValueError("Hq must be a multiple of Hkv")
        group = Hq // Hkv
        if scale is None:
            scale = 1.0 if no_scale else 1.0 / math.sqrt(d)
        out = np.full((Nq, Hq, d), np.nan)
        for h in (range(Hq) if heads is None else heads):
            g = h % Hkv if gqa_mod else h // group
            s = (q[:, h, :] @ k[:, g, :].T) * scale
            s = s - s.max(axis=axis, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=axis, keepdims=True)
            out[:, h, :] = p @ (k if values_are_keys else v)[:, g, :]
        return out
    return attend


def _visible_frames(window_short=False, no_own=False, early_sinks=False):
    def visible_frames(n0, n_frames, n_sink, window):
        sinks = list(range(n_sink if early_sinks else min(n_sink, n0)))
        lo = max(n_sink, n0 - window + (1 if window_short else 0))
        win = list(range(lo, n0)) if window > 0 else []
        own = [] if no_own else list(range(n0, n0 + n_frames))
        return sinks + win + own
    return visible_frames


def _commit(evict_newest=False, highest_free=False, evict_sinks=False):
    def commit(self):
        frame = self.n_committed
        self.n_committed += 1
        evicted = []
        if len(self.sinks) < self.n_sink and not evict_sinks:
            slot = len(self.sinks)
            self.sinks.append((frame, slot))
            return frame, slot, evicted
        if evict_sinks and len(self.sinks) < self.n_sink:
            self.free.add(len(self.sinks))
            self.sinks.append((None, None))
        if self.window == 0:
            return frame, -1, evicted
        if len(self.win) == self.window:
            old_frame, slot = self.win.pop() if evict_newest else self.win.popleft()
            evicted.append(old_frame)
        else:
            slot = max(self.free) if highest_free else min(self.free)
            self.free.remove(slot)
        self.win.append((frame, slot))
        return frame, slot, evicted
    return commit


def _reset_keeps_t0(self, t0=0):
    self.ring.reset()
    self.cache = {}


def _reset_keeps_cache(self, t0=0):
    self.t0 = t0


def _reset_keeps_cache_entries(self, t0=0):
    self.ring.reset()
    self.t0 = t0


ROPE, ATT, RING = [pins_rope], [pins_attention], [pins_ring]

MUTATIONS = {
    "rotation: wrong sign of x1*s": (ROPE, [(rope, "rotate_f64", _rotate_f64(sign=-1.0))]),
    "rotation: outputs of a pair swapped": (ROPE, [(rope, "rotate_f64", _rotate_f64(swap_outputs=True))]),
    "rotation: pairs as (j, j + d/2) halves": (ROPE, [(rope, "rotate_f64", _rotate_f64(halves=True))]),
    "frequencies: band width off by one pair": (ROPE, [(rope, "inv_freqs", _inv_freqs_wrong_width)]),
    "positions: h and w swapped": (ROPE, [(rope, "token_positions", _token_positions(swap_hw=True))]),
    "positions: t off by one": (ROPE, [(rope, "token_positions", _token_positions(t_shift=1))]),
    "positions: views on one grid": (ROPE, [(rope, "token_positions", _token_positions(one_grid=True))]),
    "tables: sin replaced by cos": (ROPE, [(rope, "table_row", _table_row_sin_is_cos)]),
    "tables: bands in t, w, h order": (ROPE, [(rope, "per_token_tables", _per_token_tables_bands_twh)]),
    "tables: fp64 values, not rounded to fp32": (ROPE, [(rope, "table_row", _table_row_fp64)]),
    "bf16: rounded through fp32 (two roundings)": (ROPE, [(bf16, "f64_to_bits", _f64_to_bits_via_fp32)]),
    "bf16: truncation": (ROPE, [(bf16, "f64_to_bits", _f64_to_bits("truncate"))]),
    "bf16: ties away from zero": (ROPE, [(bf16, "f64_to_bits", _f64_to_bits("away"))]),
    "attention: no 1/sqrt(d)": (ATT, [(attention, "attend", _attend(no_scale=True))]),
    "attention: kv head h mod Hkv": (ATT, [(attention, "attend", _attend(gqa_mod=True))]),
    "attention: softmax over queries": (ATT, [(attention, "attend", _attend(axis=0))]),
    "attention: keys used as values": (ATT, [(attention, "attend", _attend(values_are_keys=True))]),
    "visible keys: window one frame short": (ATT + RING, [(attention, "visible_frames", _visible_frames(window_short=True)),
                                                         (pins_ring, "visible_frames", _visible_frames(window_short=True))]),
    "visible keys: own chunk left out": (ATT + RING, [(attention, "visible_frames", _visible_frames(no_own=True)),
                                                     (pins_ring, "visible_frames", _visible_frames(no_own=True))]),
    "visible keys: sinks before they exist": (ATT + RING, [(attention, "visible_frames", _visible_frames(early_sinks=True)),
                                                          (pins_ring, "visible_frames", _visible_frames(early_sinks=True))]),
    "commit: K stored unrotated": (ATT, [(Rollout, "commit", _commit_unrotated)]),
    "bf16: decoded with the wrong shift": (ROPE, [(bf16, "bits_to_f64", _bits_to_f64_shift15)]),
    "masked formulation: mask inverted": (ATT, [(attention, "attend_masked", _attend_masked_inverted)]),
    "masked formulation: window one frame long": (ATT, [(attention, "frame_visible", _frame_visible_window_long)]),
    "rollout: positions one frame late": (ATT, [(Rollout, "t_of", _t_of_plus_one)]),
    "rollout: chunk values shifted by a frame": (ATT, [(Rollout, "keys_values", _keys_values_own_chunk_first)]),
    "rollout: reset keeps the old origin t0": (ATT, [(Rollout, "reset", _reset_keeps_t0)]),
    "rollout: reset keeps the cache": (ATT, [(Rollout, "reset", _reset_keeps_cache)]),
    "rollout: reset keeps the old frames' K/V entries": (ATT, [(Rollout, "reset", _reset_keeps_cache_entries)]),
    "ring: evicts the newest frame": (RING, [(ring.DequeRing, "commit", _commit(evict_newest=True))]),
    "ring: highest free slot first": (RING, [(ring.DequeRing, "commit", _commit(highest_free=True))]),
    "ring: sinks evicted like window frames": (RING, [(ring.DequeRing, "commit", _commit(evict_sinks=True))]),
}


def test_every_pin_passes_unmutated():
    assert first_failing_pin(ROPE + ATT + RING) is None


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    modules, patches = MUTATIONS[name]
    for target, attr, value in patches:
        monkeypatch.setattr(target, attr, value)
    assert first_failing_pin(modules) is not None, "no pin fails with: " + name
