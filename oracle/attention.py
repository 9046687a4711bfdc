"""Block-causal chunk attention, fp64, by explicit concatenation (test infrastructure only).

Pages:
* Cosmos3-H-Dreams model card, "Model Architecture": the few-step student is
  block-causal and generates autoregressively with a KV cache.
* AlpaDreams write-up, section VII: the causal DiT predicts each new frame
  from the earlier, already denoised frames and the frame being denoised.
* FlashDreams blog post, "Bounded Memory for Infinite Rollouts": the cache a
  chunk attends to is bounded.

Reading taken where the pages are silent: the queries of the current chunk
attend to (a) the sink frames present, (b) the window frames present, both
as committed earlier, and (c) every frame of the chunk itself at the current
denoise step -- bidirectionally inside the chunk.  Scores are scaled by
1/sqrt(d); there is no bias, soft-cap or dropout.  Query head h reads kv head
floor(h / (Hq / Hkv)) (grouped-query attention with contiguous groups).
"""

import math

import numpy as np


def visible_frames(n0, n_frames, n_sink, window):
    """Key frame ids, in temporal order, seen by the chunk [n0, n0 + n_frames)."""
    sinks = list(range(min(n_sink, n0)))
    win = list(range(max(n_sink, n0 - window), n0)) if window > 0 else []
    own = list(range(n0, n0 + n_frames))
    return sinks + win + own


def frame_visible(f, n0, n_frames, n_sink, window):
    """Mask predicate of the full-sequence formulation: may chunk [n0, n0+C) see frame f?"""
    in_chunk = n0 <= f < n0 + n_frames
    is_sink = f < n_sink and f < n0 + n_frames
    in_window = window > 0 and max(n_sink, n0 - window) <= f < n0
    return in_chunk or is_sink or in_window


def attend(q, k, v, scale=None, heads=None):
    """Softmax attention in fp64.

    q: (Nq, Hq, d); k, v: (Nk, Hkv, d), all float64.  Returns (Nq, Hq, d)
    (only the listed ``heads`` are filled when given; the rest are NaN).
    """
    Nq, Hq, d = q.shape
    Nk, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((Nq, Hq, d), np.nan)
    for h in (range(Hq) if heads is None else heads):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def attend_masked(q, k, v, mask, scale=None, heads=None):
    """Softmax attention with a boolean (Nq, Nk) visibility mask, fp64."""
    Nq, Hq, d = q.shape
    Nk, Hkv, _ = k.shape
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((Nq, Hq, d), np.nan)
    for h in (range(Hq) if heads is None else heads):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out
