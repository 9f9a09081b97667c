"""Build the kvq shared library (HIP for gfx950) in-tree.

    python -m decode_attention_paged_split_amd.build

compiles csrc/*.hip and csrc/*.cpp with hipcc and links libkvq.so next to this file;
``--sanitize`` links _build/sanitize/libkvq_san.so, whose host code runs under ASan + UBSan.
Every HIP translation unit is built with packed-FP32 instructions disabled (the
compiler then never emits v_pk_{add,mul,fma}_f32).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvq.so")
ARCH = os.environ.get("KVQ_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file code generation: the matrix engine's head-dim-256 kernels run a few per cent faster with
# these of the compiler's instruction-scheduling strategies (measured on MI355X: pair kernel 84.1 ->
# 82.3 us on the 4-bit GQA-8 workload, split kernel 691 -> 672 us on the 4-row one); every other
# file keeps the default, which measured best for it.
FILE_FLAGS = {"partial_mfma_pair.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
              "partial_mfma_split.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the kvq library needs ROCm's hipcc to build")
    return p


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + FILE_FLAGS.get(os.path.basename(src), []) + ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    # the host pass warns that it does not know the packed-fp32 feature: expected
    noise = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source and link libkvq.so; returns its path.  incremental: recompile only the
    sources whose object is older than the source or than any header (a development shortcut)."""
    objdir = os.path.join(ROOT, "_build", "kvq")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    todo = list(zip(srcs, objs))
    if incremental:
        headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
        headers.append(os.path.join(ROOT, "include", "kvq.h"))
        newest_h = max(os.path.getmtime(h) for h in headers)
        todo = [(s, o) for s, o in todo if not os.path.exists(o) or
                os.path.getmtime(o) < max(os.path.getmtime(s), newest_h)]
    workers = max(1, min(len(todo), int(os.environ.get("MAX_JOBS", "8"))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda so: _compile(*so), todo))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libkvq.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI's host code (argument
# validation, pool handles, workspace carving, the per-device scratch table), for CPU tests.  Only
# the host pass is instrumented (every sanitizer flag follows -Xarch_host); device code is unchanged.
SAN_SOURCES = ("api.cpp", "noalloc.hip")
SAN_FLAGS = ["-O1", "-g",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(ROOT, "_build", "sanitize", "libkvq_san.so")


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of ROCm's clang (a process loading the sanitized library
    needs it preloaded, since the Python interpreter is not instrumented)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not found:
            raise RuntimeError("the shared AddressSanitizer runtime was not found")
        path = found[-1]
    return path


def build_sanitized(verbose: bool = True) -> str:
    """Link SAN_LIB from the sanitized host sources and the regular objects of the other sources
    (built by build() first when missing); returns its path."""
    objdir = os.path.join(ROOT, "_build", "kvq")
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    plain = [os.path.join(objdir, f + ".o") for f in srcs if f not in SAN_SOURCES]
    if not all(os.path.exists(o) for o in plain):
        build(verbose=verbose, incremental=True)
    sandir = os.path.dirname(SAN_LIB)
    os.makedirs(sandir, exist_ok=True)
    san = []
    for f in SAN_SOURCES:
        src, obj = os.path.join(CSRC, f), os.path.join(sandir, f + ".o")
        cmd = [_hipcc()] + [c for c in COMMON if c != "-O3"] + SAN_FLAGS
        if f.endswith(".hip"):
            cmd += DEVICE + ["-x", "hip"]
        r = subprocess.run(cmd + ["-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"sanitized compile of {f} failed")
        san.append(obj)
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-o", SAN_LIB] + plain + san
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of the sanitized library failed")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build(incremental="--incremental" in sys.argv[1:])
