"""3D rotary position embedding at absolute (t, h, w) (test infrastructure only).

The pages carry frame positions across requests (DreamZero single-GPU page,
"Architecture" and "Sequential requests") and describe outputs as
(height, width, time) volumes of latents laid out frame by frame
(Cosmos3-H-Dreams model card, "Output"; DreamZero page, request schema), but
they fix no positional-encoding convention.  The convention below is the
reading used throughout; every choice is stated so that bit-exact comparison
has a meaning:

* positions: token r of the frame with id n in a sequence whose origin is t0
  sits at t = t0 + n, h = r // frame_w, w = r % frame_w;
* several camera views (AlpaDreams write-up, sections VII-VIII: a four-view
  model whose views one Transformer attends together) make a frame of
  V * frame_h * frame_w tokens, view after view; each view keeps its own
  (h, w) grid and all views of a frame share t: token r sits at
  h = (r % (frame_h * frame_w)) // frame_w, w = r % frame_w (the pages say
  nothing about encoding the view itself -- a learned view embedding would be
  added outside this attention path);
* the head dimension d is cut into three bands [t | h | w]; by default
  d_h = d_w = 2 * floor(d / 6) and d_t = d - d_h - d_w;
* in a band of width d_a starting at element off_a, pair j (0 <= j < d_a/2)
  is the element pair (off_a + 2j, off_a + 2j + 1); its inverse frequency is
  theta ** (-(2j) / d_a), evaluated with the C library ``pow`` in fp64;
* the angle is pos * inv_freq in fp64; the table entries are the C library
  ``cos``/``sin`` of that angle in fp64, each rounded once to fp32;
* the rotation is y0 = x0*c - x1*s, y1 = x0*s + x1*c evaluated in fp64 --
  a bf16 value times an fp32 value is exact in fp64, so the subtraction or
  addition is the only rounding -- followed by one round-to-nearest-even
  straight to bf16.
"""

import math

import numpy as np

from . import bf16


def band_sizes(d, rope_dims=None):
    """(d_t, d_h, d_w) band widths; ``rope_dims`` overrides the default split."""
    if rope_dims is not None and any(rope_dims):
        dt, dh, dw = (int(v) for v in rope_dims)
    else:
        dh = dw = 2 * (d // 6)
        dt = d - dh - dw
    if dt + dh + dw != d or min(dt, dh, dw) < 0 or dt % 2 or dh % 2 or dw % 2:
        raise ValueError("rope bands must be even, non-negative and sum to d")
    return dt, dh, dw


def inv_freqs(theta, d_a):
    """Inverse frequencies of the d_a/2 pairs of one band (fp64, C pow)."""
    return [math.pow(theta, -(2.0 * j) / d_a) for j in range(d_a // 2)]


def table_row(pos, theta, d_a, round_fp32=True):
    """(cos, sin) of one band at integer position ``pos``.

    Returned as float64 arrays whose values are the fp32-rounded libm results
    (``round_fp32=False`` keeps the fp64 values; used only by identity checks).
    """
    c = np.empty(d_a // 2, dtype=np.float64)
    s = np.empty(d_a // 2, dtype=np.float64)
    for j, f in enumerate(inv_freqs(theta, d_a)):
        ang = float(pos) * f
        cv, sv = math.cos(ang), math.sin(ang)
        if round_fp32:
            cv, sv = float(np.float32(cv)), float(np.float32(sv))
        c[j], s[j] = cv, sv
    return c, s


def token_positions(n_frames, frame_h, frame_w, t_first, n_views=1):
    """(t, h, w) of every token of ``n_frames`` consecutive frames, token-major;
    a frame holds ``n_views`` views of frame_h x frame_w tokens."""
    fv = frame_h * frame_w
    ft = n_views * fv
    r = np.arange(n_frames * ft)
    t = t_first + r // ft
    hw = (r % ft) % fv
    return t.astype(np.int64), (hw // frame_w).astype(np.int64), (hw % frame_w).astype(np.int64)


def per_token_tables(t, h, w, d, theta=10000.0, rope_dims=None, round_fp32=True):
    """cos/sin per token and per pair: two float64 arrays of shape (T, d/2)."""
    dt, dh, dw = band_sizes(d, rope_dims)
    T = len(t)
    cos = np.empty((T, d // 2))
    sin = np.empty((T, d // 2))
    col = 0
    for pos_arr, d_a in ((t, dt), (h, dh), (w, dw)):
        npair = d_a // 2
        if npair == 0:
            continue
        uniq, inv = np.unique(pos_arr, return_inverse=True)
        ctab = np.empty((len(uniq), npair))
        stab = np.empty((len(uniq), npair))
        for k, p in enumerate(uniq):
            ctab[k], stab[k] = table_row(int(p), theta, d_a, round_fp32)
        cos[:, col:col + npair] = ctab[inv]
        sin[:, col:col + npair] = stab[inv]
        col += npair
    return cos, sin


def rotate_f64(x, t, h, w, theta=10000.0, rope_dims=None, round_fp32=True):
    """Rotated vectors in fp64, before the final rounding to bf16.

    x: float64 array (T, H, d) -- token-major, heads, head dim.
    t, h, w: int arrays (T,) of positions.
    """
    T, H, d = x.shape
    cos, sin = per_token_tables(t, h, w, d, theta, rope_dims, round_fp32)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    c = cos[:, None, :]
    s = sin[:, None, :]
    y = np.empty_like(x)
    # Exact products in fp64, one rounding in the add/subtract.
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def rotate(x_bits, t, h, w, theta=10000.0, rope_dims=None):
    """Rotate bf16 token vectors at absolute positions; returns bf16 bits."""
    x = bf16.bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    return bf16.f64_to_bits(rotate_f64(x, t, h, w, theta, rope_dims))


def rotate_frames(x_bits, frame_h, frame_w, t_first, theta=10000.0, rope_dims=None, n_views=1):
    """Rotate ``n_frames`` consecutive frames starting at absolute t ``t_first``."""
    T = x_bits.shape[0]
    ft = n_views * frame_h * frame_w
    if T % ft:
        raise ValueError("token count is not a whole number of frames")
    t, h, w = token_positions(T // ft, frame_h, frame_w, t_first, n_views)
    return rotate(x_bits, t, h, w, theta, rope_dims)
