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
