"""Build libbeam_moe.so (gfx950) in-tree with hipcc.

    python -m group_limited_routing_amd.build [--asan]

Each HIP source compiles to an object in parallel, then one link step makes
the shared library next to this file. Every HIP compile disables packed fp32
instructions (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know that feature, which is harmless.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libbeam_moe.so")
SOURCES = ["beam_moe.hip", "router.hip", "permute.hip", "expert_gemm.hip", "backward.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # drop hipcc's harmless host-side note about the packed-fp32 feature
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, "\n".join(lines)


# Host-only AddressSanitizer build (the argument checks and host logic of the
# C ABI, run on the CPU): the host pass is instrumented, the gfx950 code is
# not. The library leaves the sanitizer's symbols undefined; a process loads
# it with the sanitizer runtime preloaded (asan_runtime()).
ASAN_LIB_PATH = os.path.join(BUILD_DIR, "asan", "libbeam_moe_asan.so")
ASAN_CFLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-g"]


def asan_runtime():
    """Path of the AddressSanitizer runtime that matches hipcc's clang, or None."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(verbose=False, asan=False):
    out_dir = os.path.join(BUILD_DIR, "asan") if asan else BUILD_DIR
    os.makedirs(out_dir, exist_ok=True)
    flags = CFLAGS + (ASAN_CFLAGS if asan else [])
    objs = [os.path.join(out_dir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            raise RuntimeError("hipcc failed: " + " ".join(cmd))
    lib_path = ASAN_LIB_PATH if asan else LIB_PATH
    tmp = lib_path + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv))
