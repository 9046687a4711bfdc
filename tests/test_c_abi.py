"""The boundary from C: include/wm.h compiles as strict C99; a C program
linked against libwm.so drives a metadata-only ring (CPU), and another one
allocates device memory with hipMalloc and runs a rollout step (GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "autoregressive_video_world_amd")
LIB = os.path.join(PKG, "libwm.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_consumer(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libwm.so is not built; run __graft_entry__.build()")
    exe = str(tmp_path / "c_abi_consumer")
    hip_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_consumer.c"),
           "-o", exe, "-L" + PKG, "-lwm", "-Wl,-rpath," + PKG, "-L" + hip_lib, "-Wl,-rpath," + hip_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_device_consumer(tmp_path):
    """One rollout step from C on a ring where every query sees one key:
    the output equals V bit for bit."""
    if not os.path.exists(LIB):
        pytest.fail("libwm.so is not built; run __graft_entry__.build()")
    exe = str(tmp_path / "c_abi_device_consumer")
    hip_inc, hip_lib = "/opt/rocm/include", "/opt/rocm/lib"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-isystem", hip_inc,
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_device_consumer.c"),
           "-o", exe, "-L" + PKG, "-lwm", "-Wl,-rpath," + PKG, "-L" + hip_lib, "-lamdhip64",
           "-Wl,-rpath," + hip_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)
