"""Build liblowram.so for gfx950 in-tree with hipcc (no GPU needed).

Usage: python -m long_context_decode_lowram_amd.build [-v] [--sanitize]
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblowram.so")

SOURCES = ["api.cpp", "decode_common.hip", "decode_generic.hip", "decode_mfma.hip", "rank.hip", "prefill_mfma.hip",
           "xkv.hip", "fit.hip"]
# Packed fp32 instructions are switched off for all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-x", "hip", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
PER_FILE = {"rank.hip": ["-ffp-contract=off"], "prefill_mfma.hip": ["-ffp-contract=off"]}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose=False):
    """Compile every source and link liblowram.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
# layer (api.cpp: argument checks, workspace carving, launch sequence), linked
# with the normal kernel objects. Device code is built without sanitizers.
SAN_HOST = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "san", "liblowram.so")


def asan_runtime():
    """The compiler's shared ASan runtime, which must be preloaded into the
    process that loads the sanitized library."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("shared ASan runtime not found")
    return path


def build_sanitized(verbose=False):
    """Compile api.cpp with host sanitizers and link it with the other
    objects into _build/san/liblowram.so (run build() first)."""
    os.makedirs(os.path.join(BUILD, "san"), exist_ok=True)
    obj = os.path.join(BUILD, "san", "api.o")
    cmd = [hipcc(), *[f for f in COMMON if f != "-O3"], *SAN_HOST, "-c", os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized api.cpp failed:\n{r.stdout}\n{r.stderr}")
    others = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "api.cpp"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing}")
    link = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", obj, *others, "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB]
    if verbose:
        print(" ".join(cmd), "\n", " ".join(link), flush=True)
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
