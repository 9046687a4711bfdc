"""The library's host code under AddressSanitizer and ThreadSanitizer (no GPU).

A host-sanitized copy of libwm.so (device code unchanged, rebuilt here when
a source or the build script is newer) is loaded through WM_LIB by a child
pytest run of the host ABI tests (eight threads calling at once among them),
with the sanitizer's runtime preloaded.  Any sanitizer report fails the run
(halt_on_error), and the copy must really be instrumented: its undefined
symbols include the sanitizer's hooks.  Under AddressSanitizer the
interpreter allocates through malloc (PYTHONMALLOC=malloc), so the buffers
Python hands the library (report and view structs) carry redzones too.  Leak
detection is off: the interpreter itself keeps allocations until exit.
"""

import glob
import os
import subprocess
import sys

import pytest

from autoregressive_video_world_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = ["tests/test_abi_host.py"]
HOOK = {"address": "__asan_report_load", "thread": "__tsan_read"}


def fresh_lib(kind):
    lib = os.path.join(_build.BUILD, "san_" + kind, "libwm.so")
    deps = _build.sources() + glob.glob(os.path.join(_build.CSRC, "*.hpp")) + \
        glob.glob(os.path.join(ROOT, "include", "*.h")) + [_build.__file__]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(d) for d in deps):
        _build.build(sanitize=kind)
    return lib


@pytest.mark.slow
@pytest.mark.parametrize("kind", ["address", "thread"])
def test_host_code_under_sanitizer(kind):
    lib = fresh_lib(kind)
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                               check=True).stdout
    assert HOOK[kind] in undefined, "the %s build is not instrumented" % kind
    preload = [_build.sanitizer_runtime(kind)]
    if os.environ.get("LD_PRELOAD"):
        preload.append(os.environ["LD_PRELOAD"])   # the runtime must come first
    env = dict(os.environ, WM_LIB=lib, LD_PRELOAD=" ".join(preload),
               PYTHONMALLOC="malloc" if kind == "address" else "pymalloc",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + FILES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "Sanitizer" not in out, out[-6000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]
