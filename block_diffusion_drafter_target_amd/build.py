"""Build libdflash.so (gfx950) from csrc/ with hipcc.

    python -m block_diffusion_drafter_target_amd.build [--sanitize]

Every call recompiles every source; objects go to ``_build/`` at the repo root
and the shared library next to this file, where the binding loads it.

``--sanitize`` (``build_sanitized()``) builds a second copy of the library,
``_build/sanitize/libdflash_san.so``, whose host code is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (device code is built as
usual); the CPU tests load it with the sanitizer runtime preloaded to check
the C ABI's argument handling.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdflash.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# hipcc may pick packed fp32 instructions for float2 math on its own; they are
# switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"] + DEVICE_FLAGS


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


SAN_DIR = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libdflash_san.so")
# host-side only: each -fsanitize= goes to the host compilation pass
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime that the sanitized library links to."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def _compile_san(src: str) -> str:
    obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + SAN_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized) failed on {src}:\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = True) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile_san, srcs))
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", "-o", tmp] + SAN_FLAGS + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB} from {len(srcs)} sources")
    return SAN_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host-side stub the compiler dropped
    # (a host-pass failure inside a template it reports nowhere) is a link
    # error here, not a load error on the GPU
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
