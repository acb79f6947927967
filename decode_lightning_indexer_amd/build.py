"""Build libess.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each .hip (and host-only .cpp) source under csrc/ compiles to an object in
_build/ (in parallel),
then the objects link into decode_lightning_indexer_amd/libess.so.  No GPU is
needed: hipcc cross-compiles for gfx950.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libess.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 VALU ops stay off (host pass warns it does not know the
    # feature; that warning is harmless).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source additions: MFMA results in VGPRs (not accumulation registers).
# The indexer reads every MFMA result in its epilogue, so no copy precedes
# each read (measured 8-12 % faster at 32K and 128K).  The attention
# rescales its output accumulators under a branch; with them in
# accumulation registers the compiler moved all of them to VGPRs and back
# on every tile.
EXTRA = {
    "index_scores.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


# Host-only C++ (no device code): compiled as plain C++ by the same driver.
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
              "-x", "c++"]


# Host-code sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for a
# checking build of the library's host paths: every flag applies to the host
# compilation only (-Xarch_host), the GPU code is built as usual.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src, cc, verbose, out_dir=BUILD, extra_flags=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    extra = EXTRA.get(os.path.basename(src), []) + list(extra_flags)
    flags = HOST_FLAGS if src.endswith(".cpp") else FLAGS
    cmd = [cc, *flags, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The library with its host code under ASan + UBSan, for the CPU tests
    of the host paths (argument checks, the host replay).  It resolves the
    sanitizer runtime at load time: load it with that runtime preloaded
    (sanitizer_runtime()).  Returns the library's path (in _build/)."""
    cc = hipcc()
    out = os.path.join(BUILD, "asan")
    os.makedirs(out, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc, verbose, out, SANITIZE), srcs))
    lib = os.path.join(out, "libess_asan.so")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(lib + ".tmp", lib)
    return lib


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too)."""
    cc = hipcc()
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "llvm",
                                     "bin", "clang"), "--print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("AddressSanitizer runtime not found")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose=True))
