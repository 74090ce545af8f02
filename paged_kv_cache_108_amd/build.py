"""Build libpkv.so in-tree: host C++ with g++, device code with hipcc for gfx950.

``python -m paged_kv_cache_108_amd.build`` (or ``build()``) always recompiles.
"""

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale of the
    # output accumulators is then plain VALU work, with no AGPR round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "argument unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False, out=LIB, extra_hip_flags=()):
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        host_o = os.path.join(tmp, "host.o")
        dev_o = os.path.join(tmp, "device.o")
        _run([cxx, "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
              os.path.join(CSRC, "host.cpp"), "-o", host_o], verbose)
        _run([hipcc, *HIP_FLAGS, *extra_hip_flags, "-I", INCLUDE, "-c",
              os.path.join(CSRC, "device.hip"), "-o", dev_o], verbose)
        tmp_so = os.path.join(tmp, "libpkv.so")
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", host_o, dev_o, "-o", tmp_so],
             verbose)
        shutil.move(tmp_so, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


# The host part alone (allocator, table and slot builders, hashes), built with
# AddressSanitizer and UndefinedBehaviorSanitizer for CPU test runs. It is
# loaded with PKV_LIB pointing at it, PKV_HOST_ONLY=1 and the sanitizer
# runtimes preloaded (see tests/test_host_sanitizers.py). No device code is in it.
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host_sanitized(out, verbose=False):
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    _run([cxx, *SAN_FLAGS, "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", "-I", INCLUDE,
          os.path.join(CSRC, "host.cpp"), "-o", out], verbose)
    return out


def sanitizer_runtimes():
    """Paths of the compiler's ASan and UBSan runtimes, to preload."""
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    paths = []
    for name in ("libasan.so", "libubsan.so"):
        r = subprocess.run([cxx, f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
        paths.append(r.stdout.strip())
    return paths


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(os.path.join(HERE, "libpkv_host_san.so"), verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
