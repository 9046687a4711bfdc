"""One streaming rollout, step by step, in fp64 (test infrastructure only).

Pages:
* FlashDreams blog post, "Hot-Path Generation, Background State Updates":
  a rollout step splits into generate(), the few-step denoising whose
  latency counts, and finalize(), which brings the KV cache and the rest of
  the state up to date.
* Cosmos3-H-Dreams model card, "Model Architecture": the conditioning frame is
  prefilled into the KV cache once; then each latent frame takes 4 denoising
  steps.  The Cosmos-H-Dreams news item and the AlpaDreams write-up (section
  VII) give two steps per latent frame.
* DreamZero single-GPU page, "Sequential requests": frame positions and the
  cache carry over between requests; explicit start-frame / cache reset.

Readings taken where the pages are silent:
* the frames committed after the last denoise step carry that step's K
  (rotated at the frame's absolute t) and V;
* K is stored rotated and never re-rotated; sink frames keep their t;
* prefill frames are committed without attention.

The cache is a dict frame -> (K_rot bits, V bits); slots come from the
deque ring (``oracle.ring``).  Attention concatenates the visible frames in
temporal order and calls ``oracle.attention.attend``.
"""

import numpy as np

from . import attention, bf16, ring, rope


class Rollout:
    def __init__(self, n_q_heads, n_kv_heads, head_dim, frame_h, frame_w,
                 n_sink, window, theta=10000.0, rope_dims=None, t0=0, n_views=1):
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.fh, self.fw = frame_h, frame_w
        self.n_views = n_views
        self.ft = n_views * frame_h * frame_w
        self.S, self.W = n_sink, window
        self.theta, self.rope_dims = theta, rope_dims
        self.ring = ring.DequeRing(n_sink, window)
        self.cache = {}
        self.t0 = t0

    # -- positions ---------------------------------------------------------
    @property
    def n_committed(self):
        return self.ring.n_committed

    def t_of(self, frame):
        return self.t0 + frame

    def reset(self, t0=0):
        """Start a new sequence (DreamZero page: current_start_frame / reset_kv_cache)."""
        self.ring.reset()
        self.cache = {}
        self.t0 = t0

    # -- generate(): one denoise step of the current chunk ----------------
    def rope(self, x_bits, n_frames, t_first=None):
        if t_first is None:
            t_first = self.t_of(self.n_committed)
        return rope.rotate_frames(x_bits, self.fh, self.fw, t_first, self.theta, self.rope_dims,
                                  self.n_views)

    def keys_values(self, k_rot_chunk, v_chunk, n_frames):
        """Explicit concatenation of the visible frames' K_rot/V in temporal order."""
        n0 = self.n_committed
        ks, vs = [], []
        for f in attention.visible_frames(n0, n_frames, self.S, self.W):
            if f >= n0:
                j = f - n0
                ks.append(k_rot_chunk[j * self.ft:(j + 1) * self.ft])
                vs.append(v_chunk[j * self.ft:(j + 1) * self.ft])
            else:
                kb, vb = self.cache[f]
                ks.append(kb)
                vs.append(vb)
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)

    def attend(self, q_rot_bits, k_rot_bits, v_bits, n_frames, scale=None, heads=None, rows=None):
        """O (fp64) of the chunk's queries; ``rows``/``heads`` restrict what is computed."""
        kb, vb = self.keys_values(k_rot_bits, v_bits, n_frames)
        q = bf16.bits_to_f64(q_rot_bits if rows is None else q_rot_bits[rows])
        return attention.attend(q, bf16.bits_to_f64(kb), bf16.bits_to_f64(vb), scale, heads)

    def denoise_step(self, q_bits, k_bits, v_bits, n_frames, scale=None, heads=None, rows=None):
        """RoPE on Q and K at the chunk's absolute t, then attention."""
        q_rot = self.rope(q_bits, n_frames)
        k_rot = self.rope(k_bits, n_frames)
        return q_rot, k_rot, self.attend(q_rot, k_rot, v_bits, n_frames, scale, heads, rows)

    # -- finalize(): commit the chunk -------------------------------------
    def commit(self, k_raw_bits, v_bits, n_frames):
        """Rotate K at each frame's t, store K_rot/V, evict FIFO.

        Returns (written [(frame, slot, t)], evicted [frame]) in commit order.
        """
        n0 = self.n_committed
        k_rot = self.rope(k_raw_bits, n_frames, self.t_of(n0))
        written, evicted = [], []
        for j in range(n_frames):
            frame, slot, ev = self.ring.commit()
            for e in ev:
                del self.cache[e]
            evicted.extend(ev)
            written.append((frame, slot, self.t_of(frame)))
            if slot >= 0:
                sl = slice(j * self.ft, (j + 1) * self.ft)
                self.cache[frame] = (k_rot[sl].copy(), np.asarray(v_bits[sl]).copy())
        return written, evicted

    def retained(self):
        """[(frame, slot, t)] of stored frames in temporal order."""
        return [(f, s, self.t_of(f)) for f, s in self.ring.retained()]
