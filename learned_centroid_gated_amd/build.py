"""Build libfocus.so (the Focus C-ABI library) for gfx950 with hipcc, in-tree.

    python -m learned_centroid_gated_amd.build [--jobs N]

Every source under csrc/ is compiled for --offload-arch=gfx950 and linked into
learned_centroid_gated_amd/libfocus.so. Packed fp32 arithmetic is disabled in device code.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfocus.so")
ARCH = "gfx950"

SOURCES = ["focus_api.hip", "assign_kernels.hip", "bucket_kernels.hip", "attention_kernels.hip",
           "decode_kernels.hip", "train_kernels.hip"]

CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the Focus library needs ROCm's hipcc to build")


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msg = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(jobs=None, verbose=False):
    """Compile every source and link libfocus.so. Always rebuilds. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitized variant of the library for checking the C-ABI layer on a machine without a GPU:
# focus_api.hip (argument validation, workspace carving, launch order) is compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer on its host code only; the kernels' objects are
# the normal build's. Load it with the sanitizer runtime preloaded (sanitizer_runtime()).
SAN_LIB = os.path.join(BUILD, "libfocus_san.so")
SAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()


def sanitizer_runtime():
    """Path of the AddressSanitizer runtime that a plain interpreter must preload."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime was not found next to hipcc")
    return path


def build_sanitized(verbose=False):
    """Compile focus_api.hip with host-side ASan and UBSan and link it with the other objects
    of the normal build (built first if missing). Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES[1:]:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj if os.path.exists(obj) else _compile(src, verbose))
    san_obj = os.path.join(BUILD, "focus_api_san.o")
    cflags = [f for f in CFLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [hipcc(), *cflags, *SAN_FLAGS, "-Xarch_host", "-fno-omit-frame-pointer", "-c",
           os.path.join(CSRC, "focus_api.hip"), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized build of focus_api.hip failed:\n{r.stdout}{r.stderr}")
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, san_obj,
                        *objs, "-o", SAN_LIB], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
    sys.exit(0)
