"""Seeded synthetic workloads shared by the tests and the benchmark.

This module holds shapes and random numbers only -- none of the method's
arithmetic.  The source pages measure trained models on private data, so
every input here is synthetic: standard-normal draws rounded to bf16, in the
shapes of the pages' models.

Workloads (one attention layer each):

=====  =========================================================  ==========
name   shape source                                                sizes
=====  =========================================================  ==========
tiny   CPU-checkable rollout                                       2 heads, d 64, 4x4 tokens/frame,
                                                                   chunk 1, 1 sink + 3 window, 8 frames, 2 steps
sf13b  Self-Forcing 1.3B DiT (480x832 video, 16x16 latent grid)    12 heads, d 128, 30x52 tokens/frame,
                                                                   chunk 3, 1 sink + 18 window, 32 frames, 4 steps
drive  2B driving model (AlpaDreams write-up, section VIII:        16 heads, d 128, 44x80 tokens/frame,
       704x1280, two-step)                                         chunk 1, 1 sink + 3 window, 64 frames, 2 steps
mot15  15B MoT generation expert (Cosmos3-H-Dreams model card)     32 q / 8 kv heads, d 128, 30x40 tokens/frame,
                                                                   chunk 1, 1 reference + 17 window, 36 frames, 4 steps
long   drive shapes, 8 rollouts admitted at staggered steps        10,000 frames each, 2 steps
drv4v  drive shapes with four camera views per frame (AlpaDreams   16 heads, d 128, 4 views of 44x80 tokens,
       write-up, VIII: four-view model)                            chunk 1, 1 sink + 3 window, 8 frames, 2 steps
=====  =========================================================  ==========

Draws: ``numpy.random.Generator(PCG64(SeedSequence([cfg, b, n, s + 1, kind])))``
``.standard_normal(float32)`` rounded to bf16 (round-to-nearest-even, by
PyTorch's CPU conversion).  ``s`` is the denoise step (-1 for prefill
frames), ``kind`` 0/1/2 for Q/K/V.  The long-rollout workload cannot afford
fresh draws for 8 x 10,000 frames, so it cycles a pool of 17 seeded frames
per kind: frame (b, n, s) takes entry (7919*b + 31*n + s) mod 17.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

KINDS = {"q": 0, "k": 1, "v": 2}


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    frame_h: int
    frame_w: int
    chunk: int            # frames per generated chunk
    n_sink: int
    window: int
    prefill: int          # frames committed before generation, without attention
    n_gen: int            # generated frames per rollout
    n_denoise: int
    stagger: int = 0      # rollout b is admitted at global step stagger*b
    theta: float = 10000.0
    rope_dims: tuple = field(default=(0, 0, 0))
    n_views: int = 1      # camera views per frame (each a frame_h x frame_w grid)

    @property
    def ft(self):
        return self.n_views * self.frame_h * self.frame_w

    @property
    def nq(self):
        return self.chunk * self.ft

    def chunks(self):
        """Generated-chunk sizes in order (the last one may be short)."""
        out, left = [], self.n_gen
        while left > 0:
            c = min(self.chunk, left)
            out.append(c)
            left -= c
        return out

    def steady_keys(self):
        """Visible keys of a full-window chunk of ``chunk`` frames."""
        return (self.n_sink + self.window + self.chunk) * self.ft

    def attn_flops(self, n_q=None, n_k=None):
        """4 * Nq * Nk * d * Hq per denoise step (QK^T and PV, 2 flops per MAC)."""
        n_q = self.nq if n_q is None else n_q
        n_k = self.steady_keys() if n_k is None else n_k
        return 4.0 * n_q * n_k * self.head_dim * self.n_q_heads

    def append_bytes(self, n_frames=None):
        """K and V read once and written once: 4 * C * Ft * Hkv * d * 2 bytes."""
        c = self.chunk if n_frames is None else n_frames
        return 4 * c * self.ft * self.n_kv_heads * self.head_dim * 2


WORKLOADS = {
    1: Workload(1, "tiny", 1, 2, 2, 64, 4, 4, 1, 1, 3, 0, 8, 2),
    2: Workload(2, "sf13b", 1, 12, 12, 128, 30, 52, 3, 1, 18, 0, 32, 4),
    3: Workload(3, "drive", 1, 16, 16, 128, 44, 80, 1, 1, 3, 1, 64, 2),
    4: Workload(4, "mot15", 1, 32, 8, 128, 30, 40, 1, 1, 17, 1, 36, 4),
    5: Workload(5, "long", 8, 16, 16, 128, 44, 80, 1, 1, 3, 1, 10000, 2, stagger=7),
    6: Workload(6, "drv4v", 1, 16, 16, 128, 44, 80, 1, 1, 3, 1, 8, 2, n_views=4),
}

POOL_ENTRIES = 17


def to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns (PyTorch CPU round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw(seed_words, shape, scale=1.0):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed_words)))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return to_bf16_bits(x)


class Source:
    """Seeded per-frame Q/K/V draws for one workload."""

    def __init__(self, wl: Workload, q_scale=1.0):
        self.wl = wl
        self.q_scale = q_scale
        self._pool = {}

    def shape(self, kind):
        h = self.wl.n_q_heads if kind == "q" else self.wl.n_kv_heads
        return (self.wl.ft, h, self.wl.head_dim)

    @staticmethod
    def pool_index(b, n, s):
        """Pool entry of (rollout b, frame n, denoise step s) in the long workload."""
        return (7919 * b + 31 * n + s) % POOL_ENTRIES

    def pool_entry(self, e, kind):
        """uint16 (Ft, H, d) pool entry e of the long workload (cached)."""
        key = (e, kind)
        if key not in self._pool:
            scale = self.q_scale if kind == "q" else 1.0
            self._pool[key] = _draw([self.wl.cfg, 0, e, 0, KINDS[kind]], self.shape(kind), scale)
        return self._pool[key]

    def frame(self, b, n, s, kind):
        """uint16 (Ft, H, d) draw for rollout b, frame n, denoise step s (-1 = prefill)."""
        if self.wl.cfg == 5:
            return self.pool_entry(self.pool_index(b, n, s), kind)
        scale = self.q_scale if kind == "q" else 1.0
        return _draw([self.wl.cfg, b, n, s + 1, KINDS[kind]], self.shape(kind), scale)

    def chunk(self, b, n0, n_frames, s, kind):
        """Frames n0 .. n0+n_frames-1 stacked token-major: (n_frames*Ft, H, d)."""
        return np.concatenate([self.frame(b, n0 + j, s, kind) for j in range(n_frames)], axis=0)

    def batch_chunk(self, n0s, n_frames, s, kind):
        """Per-rollout chunks stacked on a leading batch axis; n0s[b] None -> zeros."""
        shp = (n_frames * self.wl.ft,) + self.shape(kind)[1:]
        out = np.zeros((len(n0s),) + shp, dtype=np.uint16)
        for b, n0 in enumerate(n0s):
            if n0 is not None:
                out[b] = self.chunk(b, n0, n_frames, s, kind)
        return out


SPECIAL_BF16 = (0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80,
                0x7FC0, 0xFFC1, 0x3F80, 0xBF80)


def full_range_bits(seed, shape):
    """Uniformly random bf16 bit patterns (every exponent, subnormals, inf, NaN),
    with the special patterns above planted at the start."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xB16]))
    x = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    flat = x.reshape(-1)
    flat[:len(SPECIAL_BF16)] = SPECIAL_BF16
    return x
