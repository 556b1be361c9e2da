"""Build libbasiskv.so (gfx950) in-tree with hipcc.

    python -m sparse_decode_attention_latent_amd.build [--sanitize]

Compiles every csrc/*.hip to an object under _build/ and links them into
sparse_decode_attention_latent_amd/libbasiskv.so.  Packed-FP32 instruction
selection is disabled for the device code.

The sanitizer build (build_sanitized, also run by build()) compiles the
host side of every source with AddressSanitizer and UndefinedBehaviorSanitizer
and every source with -Werror into libbasiskv_san.so;
tests/test_abi_sanitized.py runs the ABI tests (host-side validation, no
kernel launch) against it.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbasiskv.so")
BUILD_SAN = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "libbasiskv_san.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-function", "-Wno-unused-result",
                "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + DEVICE_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop those lines
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _compile_san(src):
    obj = os.path.join(BUILD_SAN, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + HOST_SAN_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed on {src}:\n{r.stderr}")
    return obj


# the host side instrumented (-O1, frame pointers), warnings as errors; the
# device side as in the product build
HOST_SAN_FLAGS = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Xarch_host", "-O1",
                  "-Xarch_device", "-O3", "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                  "-Wall", "-Werror", "-Wno-unused-function", "-Wno-unused-result",
                  "-Wno-unknown-warning-option",
                  "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def asan_runtime():
    """Path of the AddressSanitizer runtime the sanitizer build links against
    (to be preloaded into an uninstrumented Python)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    return r.stdout.strip()


def build_sanitized(verbose=True):
    os.makedirs(BUILD_SAN, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile_san, srcs))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "-shared-libsan", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer link failed:\n" + r.stderr)
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_sanitized(verbose)
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        build_sanitized()
    else:
        build()
