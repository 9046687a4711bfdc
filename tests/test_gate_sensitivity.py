"""The GPU parity gate catches plausible attention bugs (CPU, oracle only).

Mutations are planted in the oracle's key list -- a dropped sink frame, a
duplicated window frame, the chunk's own keys left out -- and the mutated
output, rounded to bf16, is put through the same gate the GPU tests use
(tests/gpu_util.assert_close).  With N(0,1) queries the softmax is nearly
flat, so the absolute bounds alone can let such a bug through; the
relative-L2 bound and the sharp-query variant (Q x 8) must not.
"""

import numpy as np
import pytest

from gpu_util import assert_close
from oracle import attention as oatt
from oracle import bf16 as obf16
from oracle.rollout import Rollout
from wm_synth import Source, Workload


def _case(q_scale):
    wl = Workload(90, "gate", 1, 2, 2, 128, 6, 8, 1, 1, 3, 0, 6, 1)
    src = Source(wl, q_scale=q_scale)
    ro = Rollout(2, 2, 128, 6, 8, 1, 3)
    for n in range(5):
        ro.commit(src.frame(0, n, 0, "k"), src.frame(0, n, 0, "v"), 1)
    q = ro.rope(src.frame(0, 5, 0, "q"), 1)
    k = ro.rope(src.frame(0, 5, 0, "k"), 1)
    v = src.frame(0, 5, 0, "v")
    kb, vb = ro.keys_values(k, v, 1)
    return obf16.bits_to_f64(q), obf16.bits_to_f64(kb), obf16.bits_to_f64(vb), wl.ft


def _mutants(k, v, ft):
    frames = k.shape[0] // ft  # sink, 3 window frames, own chunk
    sl = lambda f: slice(f * ft, (f + 1) * ft)
    drop_sink = (np.concatenate([k[sl(f)] for f in range(1, frames)]),
                 np.concatenate([v[sl(f)] for f in range(1, frames)]))
    dup_window = (np.concatenate([k, k[sl(2)]]), np.concatenate([v, v[sl(2)]]))
    no_own = (k[:(frames - 1) * ft], v[:(frames - 1) * ft])
    return {"drop_sink": drop_sink, "dup_window": dup_window, "no_own_chunk": no_own}


@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_correct_output_passes_and_mutations_fail(q_scale):
    q, k, v, ft = _case(q_scale)
    # the GPU tests' gate: scaled queries may also use the bf16 bound
    vmax = float(np.abs(v).max()) if q_scale != 1.0 else None
    ref = oatt.attend(q, k, v)
    assert_close(obf16.f64_to_bits(ref), ref, "unmutated", vmax)
    for name, (km, vm) in _mutants(k, v, ft).items():
        bad = obf16.f64_to_bits(oatt.attend(q, km, vm))
        with pytest.raises(AssertionError):
            assert_close(bad, ref, name, vmax)
