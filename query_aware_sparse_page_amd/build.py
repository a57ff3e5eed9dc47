"""Builds libqsa.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libqsa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed fp32 instructions stay off (scalar/float2 code only).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wl,-rpath,/opt/rocm/lib",
]


# A second build for checking the host code: the host half of every source
# under AddressSanitizer and UndefinedBehaviorSanitizer (each -fsanitize
# applies to the host compilation only; the device code is unchanged). It
# needs the sanitizer runtime preloaded (sanitizer_runtime()).
SAN_LIB = os.path.join(PKG, "_sanitized", "libqsa.so")
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-shared-libsan", "-g",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def sanitizer_runtime() -> str:
    """The ASan (+UBSan) runtime the sanitized build links against."""
    clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path):
        raise RuntimeError("sanitizer runtime not found")
    return path


def build(verbose: bool = False, sanitize: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    flags = HIPCC_FLAGS + (SAN_FLAGS if sanitize else [])
    cmd = [hipcc, *flags, "-I", os.path.join(ROOT, "include"), "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
