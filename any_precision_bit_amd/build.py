"""Builds libpw.so (the HIP kernels plus the C ABI) in-tree for gfx950 with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "pw_api.cpp"), os.path.join(HERE, "csrc", "pw_plan.cpp"),
        os.path.join(HERE, "csrc", "pw_kernels.hip")]
LIB = os.path.join(HERE, "libpw.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # keep packed-fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + SRCS + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])
    os.replace(tmp, LIB)
    return LIB


# Host sources of the C ABI (argument checks, page table, workspace layout,
# launch sequencing, planner): the part an AddressSanitizer / UBSan build covers.
HOST_SRCS = SRCS[:2]
KERNEL_SRC = SRCS[2]
# Sanitizer flags apply to host code only (no GPU sanitizer build).
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """libpw with AddressSanitizer and UBSan on the host sources, in out_dir (for
    CPU tests of the ABI's host layer; load it with the clang ASan runtime
    preloaded, see asan_runtime())."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-O3")] + ["-O1", "-g"]
    objs = []
    for src in SRCS:
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        extra = SAN_HOST_FLAGS if src in HOST_SRCS else []
        cmd = [hipcc] + flags + extra + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])
        objs.append(obj)
    lib = os.path.join(out_dir, "libpw_san.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + SAN_HOST_FLAGS + objs + ["-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stderr[-8000:])
    return lib


def asan_runtime() -> str:
    """The clang ASan runtime that hipcc's host code links against."""
    import glob

    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return found[-1]


if __name__ == "__main__":
    print(build(verbose=True))
