"""CPU oracle for streaming block-causal chunk attention over a bounded KV ring.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or runs this package; only the tests, the
package's ``smoke()`` check and the CPU-baseline leg of ``bench.py`` do.

It is a deliberately plain, slow, fp64 restatement of what the hot path
computes, written from the source pages:

* ``ring``      -- the bounded per-rollout cache: sinks + FIFO window, kept as
                   a Python deque (FlashDreams blog post, "Bounded Memory for
                   Infinite Rollouts"; Cosmos3-H-Dreams model card, "Software
                   Integration": static-shape KV cache).
* ``rope``      -- 3D rotary positions at absolute (t, h, w); the pages fix no
                   RoPE convention, so the one used here is stated in full in
                   ``oracle.rope``.
* ``attention`` -- softmax attention of a chunk's queries over an explicitly
                   concatenated key list (sinks, window, own chunk) in
                   temporal order, plus the equivalent masked full-sequence
                   formulation (Cosmos3-H-Dreams model card, "Model
                   Architecture": block-causal student with a KV cache;
                   AlpaDreams write-up, section VII: each new frame is
                   predicted from the earlier, already denoised frames and
                   the frame still being denoised).
* ``rollout``   -- a whole rollout: prefill, chunks of few-step denoising,
                   commit after the last step (FlashDreams blog post,
                   "Hot-Path Generation, Background State Updates").

It shares no code with the HIP path.  Random inputs come in as arguments.
"""

from . import bf16, ring, rope, attention, rollout  # noqa: F401
