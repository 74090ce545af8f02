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


# The attention kernels are instantiated once per (cache type, head dim) in
# attn_inst.hip, each its own translation unit: 0/1/2 = f32/bf16/fp8 caches.
INSTANCES = [(kv, d) for kv in (0, 1, 2) for d in (64, 128)]
# host code (g++): the allocator, builders and hashes; the decode work plan
HOST_SOURCES = ["host.cpp", "plan.cpp"]


def build(verbose=False, out=LIB, extra_hip_flags=(), jobs=None):
    """Compile every translation unit (in parallel) and link libpkv.so."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    jobs = jobs or min(8, os.cpu_count() or 1, int(os.environ.get("MAX_JOBS", "8")))
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        cmds, objs = [], []
        for name in HOST_SOURCES:
            o = os.path.join(tmp, name.replace(".cpp", ".o"))
            cmds.append([cxx, "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
                         os.path.join(CSRC, name), "-o", o])
            objs.append(o)
        for kv, d in INSTANCES:
            o = os.path.join(tmp, f"attn_{kv}_{d}.o")
            cmds.append([hipcc, *HIP_FLAGS, *extra_hip_flags, f"-DPKV_INST_KV={kv}", f"-DPKV_INST_D={d}",
                         "-I", INCLUDE, "-c", os.path.join(CSRC, "attn_inst.hip"), "-o", o])
            objs.append(o)
        dev_o = os.path.join(tmp, "device.o")
        cmds.append([hipcc, *HIP_FLAGS, *extra_hip_flags, "-I", INCLUDE, "-c",
                     os.path.join(CSRC, "device.hip"), "-o", dev_o])
        objs.append(dev_o)
        # the longest compiles first
        cmds = cmds[len(HOST_SOURCES):] + cmds[:len(HOST_SOURCES)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp_so = os.path.join(tmp, "libpkv.so")
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_so], verbose)
        shutil.move(tmp_so, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


# The host part alone (allocator, table and slot builders, hashes, the decode
# work plan), built with
# AddressSanitizer and UndefinedBehaviorSanitizer for CPU test runs. It is
# loaded with PKV_LIB pointing at it, PKV_HOST_ONLY=1 and the sanitizer
# runtimes preloaded (see tests/test_host_sanitizers.py). No device code is in it.
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host_sanitized(out, verbose=False):
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    _run([cxx, *SAN_FLAGS, "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", "-I", INCLUDE,
          *[os.path.join(CSRC, n) for n in HOST_SOURCES], "-o", out], verbose)
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
