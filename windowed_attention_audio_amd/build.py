"""Builds libmt.so (the HIP kernels and the C ABI) for gfx950 in-tree.

    python -m windowed_attention_audio_amd.build [--host-check]

--host-check instead builds _build/host_abi_check: the C ABI (api.cpp)
compiled with g++ under AddressSanitizer and UndefinedBehaviorSanitizer,
linked with the stub launchers of csrc/host_stubs.cpp (no GPU code; every
"device" pointer is host memory and each launcher touches the ends of the
ranges its kernel would access) and the driver tests/host_abi_check.cpp,
which calls every rejection path of every entry point and valid calls on
exactly sized buffers.  The CPU test-suite builds and runs it.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmt.so")

SOURCES = ["api.cpp", "mel.hip", "conv1.hip", "gemm.hip", "norm.hip", "attn.hip", "misc.hip", "decoder.hip"]
ARCH = "gfx950"


def hipcc():
    for p in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found")


def flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        # no packed-fp32 instructions in generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
        "-Wno-pass-failed",
    ]


# Per-file code-generation options.  attn.hip: matrix-core results in
# ordinary VGPRs rather than accumulation registers -- the softmax rescales
# the accumulators every key chunk, and each access to an accumulation
# register would cost a v_accvgpr move (measured: 368 moves per four chunks).
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    return obj, out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    subprocess.run([sys.executable, os.path.join(PKG, "gen_tables.py"),
                    os.path.join(CSRC, "mel_tables.inc")], check=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (o, msg) in results:
            if msg:
                print(msg)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libmt.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


HOST_CHECK = os.path.join(BUILD, "host_abi_check")


def rocm_include():
    root = os.environ.get("ROCM_PATH") or os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    return os.path.join(root, "include")


def build_host_check():
    """The sanitizer build of the C ABI on the host (see the module docstring);
    returns the path of the executable."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = HOST_CHECK + ".tmp"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-D__align__(x)=__attribute__((aligned(x)))",
           "-DHIP_SYMBOL(x)=x", "-I", rocm_include(), "-I", INCLUDE, "-I", CSRC,
           "-x", "c++", os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_stubs.cpp"),
           os.path.join(ROOT, "tests", "host_abi_check.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the host check failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, HOST_CHECK)
    return HOST_CHECK


if __name__ == "__main__":
    if "--host-check" in sys.argv[1:]:
        print(build_host_check())
    else:
        print(build(verbose=True))
