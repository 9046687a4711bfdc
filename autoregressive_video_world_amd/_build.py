"""Build libwm.so (the C-ABI library with its gfx950 kernels) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled.  No fast-math anywhere: the host RoPE tables must be the
plain libm values.

``build(sanitize="address")`` or ``"thread"`` builds a second copy whose host
code (the C ABI, ring bookkeeping, argument checks, launch set-up) carries
AddressSanitizer or ThreadSanitizer; device code is compiled exactly as in
the normal build.  It goes to ``_build/san_<kind>/libwm.so``, never over the
in-package library, and is meant for host-only tests: the process that loads
it must start with the sanitizer runtime preloaded (``sanitizer_runtime``
gives its path).  ``python -m autoregressive_video_world_amd._build address``
builds it from the command line.
"""

import concurrent.futures
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


# Extra flags per source file (relative to csrc/).  The attention kernel is
# built without NaN semantics so that max() needs no NaN-quieting instructions.
PER_FILE = {os.path.join("kernels", "chunk_attn.hip"): ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


SANITIZERS = ("address", "thread")


def _san_flags(kind):
    # -Xarch_host before every flag: the sanitizer applies to host code only
    return ["-Xarch_host", "-fsanitize=" + kind, "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def sanitizer_runtime(kind):
    """Path of the shared sanitizer runtime of hipcc's clang (for LD_PRELOAD)."""
    name = {"address": "libclang_rt.asan-x86_64.so", "thread": "libclang_rt.tsan-x86_64.so"}[kind]
    r = subprocess.run([HIPCC, "--print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/" + name))
    if not hits:
        raise RuntimeError("no %s runtime found for hipcc's clang" % kind)
    return hits[-1]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) +
                  glob.glob(os.path.join(CSRC, "kernels", "*.hip")))


def _compile(src, out_dir, extra):
    obj = os.path.join(out_dir, os.path.relpath(src, CSRC).replace(os.sep, "_") + ".o")
    cmd = [HIPCC] + COMMON + PER_FILE.get(os.path.relpath(src, CSRC), []) + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose=False, sanitize=None):
    """Compile every source and link ``libwm.so``; returns its path.

    sanitize: None (the product library, in the package), or "address" /
    "thread" for a host-sanitized copy under _build/san_<kind>/."""
    if sanitize is None:
        out_dir, lib, extra, link_extra = BUILD, LIB, [], ["-Wl,--no-undefined"]
    elif sanitize in SANITIZERS:
        out_dir = os.path.join(BUILD, "san_" + sanitize)
        lib = os.path.join(out_dir, "libwm.so")
        # the runtime comes from the preloaded shared library at run time
        extra, link_extra = _san_flags(sanitize), ["-Xarch_host", "-fsanitize=" + sanitize, "-shared-libsan"]
    else:
        raise ValueError("sanitize must be None, 'address' or 'thread'")
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    # --no-undefined: a kernel whose host stub the compiler did not emit
    # fails the build here instead of at the first launch
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + link_extra + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    import sys
    build(verbose=True, sanitize=sys.argv[1] if len(sys.argv) > 1 else None)
