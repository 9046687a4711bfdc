"""Helpers shared by the GPU tests: host<->device bf16 bits and error metrics."""

import numpy as np
import torch

# Tolerance on bf16 attention outputs against the fp64 oracle: max-abs 2e-2 and
# mean-abs 2e-3 (the stated acceptance bar), plus a relative-L2 bound of 1e-2.
# With N(0,1) inputs the softmax is nearly flat and |O| ~ sqrt(e/Nk) is small,
# so absolute bounds alone would pass a kernel that drops a whole frame
# (relative-L2 ~0.2); bf16 rounding of P and of O gives ~3e-3.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


def dev(bits):
    """uint16 numpy bits -> bf16 CUDA tensor (same shape)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    """bf16 tensor -> uint16 numpy bits."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def errors(got_bits, ref):
    g = bf16_to_f64(got_bits)
    d = np.abs(g - ref)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    return float(d.max()), float(d.mean()), rel


# Inputs outside the N(0,1) workloads (queries scaled x8: a peaked softmax
# with |O| up to max|V| ~ 5) meet the arithmetic's own limit first.  P is
# rounded to bf16 before P.V and O is written in bf16, each with unit
# roundoff u = 2^-8, so even an exact fp32 pipeline is off by up to
# u * (sum_k p_k |v_k| / l) + u * |O| <= u * (max|V| + |O|): ~0.03 at
# |O| = 4, where bf16 values are 2^-5 apart.  For such inputs an element may
# use that bound (plus 1e-3 for the fp32 sums and exponentials) where it is
# above MAX_ABS; the mean-abs and relative-L2 gates stay as they are.
BF16_U = 2.0 ** -8


def assert_close(got_bits, ref, what="", vmax=None):
    """The acceptance bar; with vmax (max |V| of the case's inputs), the
    per-element bound is max(MAX_ABS, u * (|ref| + vmax) + 1e-3)."""
    mx, mean, rel = errors(got_bits, ref)
    assert np.all(np.isfinite(bf16_to_f64(got_bits))), what
    if vmax is None:
        ok_elem = mx <= MAX_ABS
    else:
        bound = np.maximum(MAX_ABS, BF16_U * (np.abs(ref) + vmax) + 1e-3)
        ok_elem = bool(np.all(np.abs(bf16_to_f64(got_bits) - ref) <= bound))
    assert ok_elem and mean <= MEAN_ABS and rel <= REL_L2, \
        "%s: max %.3g mean %.3g relL2 %.3g" % (what, mx, mean, rel)
    return mx, mean, rel
