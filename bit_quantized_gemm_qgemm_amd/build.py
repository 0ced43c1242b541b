"""Build libqgemm.so (HIP, gfx950) in-tree.

Every .hip file under csrc/ is compiled to an object with hipcc and the
objects are linked into bit_quantized_gemm_qgemm_amd/libqgemm.so.

Flags:
  --offload-arch=gfx950      MI355X only
  -ffp-contract=off          no implicit fma: the int8 quantization and the
                             W8A8 epilogue are bit-exact IEEE sequences; the
                             GEMM kernels use explicit fma where they want one
  -packed-fp32-ops disabled  packed fp32 instructions are not generated
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments preloaded into scalar registers at dispatch (a kernel
    # otherwise loads them from the argument segment, one or more dependent
    # round trips before its first address is known): measured on MI355X,
    # 1-6 % off the 5-20 us memory-bound kernels, no change on the long ones
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (each -fsanitize
# behind -Xarch_host: the device code is built as usual), against the shared
# sanitizer runtime of the toolchain's clang, which the loading process must
# preload; for checking runs of the host tests only.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libasan"]
SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-shared-libasan"]


def _compile(src, verbose, objdir=OBJ, extra=()):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + list(extra) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj


def build(verbose: bool = False, out: str = LIB, host_sanitize: bool = False) -> str:
    objdir = OBJ + ("_san" if host_sanitize else "")
    extra = SAN_FLAGS if host_sanitize else []
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, objdir, extra), srcs))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + (SAN_LINK if host_sanitize else [])
    cmd += ["-o", out + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
