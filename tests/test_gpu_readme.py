"""The Python usage example in README.md runs as written on the GPU, and its
ring holds the frames the example says it does."""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_readme_example_runs(capsys):
    src = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", src, re.S)
    assert len(blocks) == 1
    scope = {}
    exec(compile(blocks[0], "README.md example", "exec"), scope)
    printed = capsys.readouterr().out.splitlines()
    # a first chunk of 3 frames: frames 0..2 go to slots 0..2 (1 sink + window), nothing evicted
    assert printed[0] == "{'written': [(0, 0, 0), (1, 1, 1), (2, 2, 2)], 'evicted': []}"
    assert printed[1] == "{'retained': [(0, 0, 0), (1, 1, 1), (2, 2, 2)], 'n_committed': 3, 't0': 0}"
    assert len(scope["outs"]) == scope["D"]


def test_readme_example_names_exist():
    """On the CPU: every ring method and package name the example uses is
    part of the binding."""
    import autoregressive_video_world_amd as wm

    src = open(os.path.join(ROOT, "README.md")).read()
    code = re.findall(r"```python\n(.*?)```", src, re.S)[0]
    compile(code, "README.md example", "exec")
    methods = set(re.findall(r"\bring\.(\w+)\(", code))
    assert methods and all(hasattr(wm.KVRing, m) for m in methods), methods
    names = set(re.findall(r"\bwm\.(\w+)", code))
    assert all(hasattr(wm, n) for n in names), names
    # the lower-level calls the text names
    for m in ("rope3d", "rope3d_pair", "chunk_attn", "append_evict", "rollout_graph"):
        assert "`%s`" % m in src and hasattr(wm.KVRing, m), m
