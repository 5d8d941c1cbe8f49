"""Build libbdiff.so in-tree with hipcc for gfx950.

    python -m block_diffusion_vlm_amd.build

Every HIP source under csrc/ is compiled to an object in _build/ (in
parallel) and linked into block_diffusion_vlm_amd/libbdiff.so.  The build
always recompiles, so a call after a source change never links stale code.

    python -m block_diffusion_vlm_amd.build host-sanitized

builds the host side alone (no device code) with AddressSanitizer and
UndefinedBehaviorSanitizer into _build/libbdiff_host_asan.so, for running
the argument validation of every entry point on a machine without a GPU
(the library's sanitizer runtime must then be preloaded: host_asan_runtime()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libbdiff.so"
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all device code: hipcc would
# otherwise emit v_pk_* float ops from ordinary float code.  MFMA results are
# kept in architectural registers (the compiler's VGPR form of the MFMA
# instructions): by default it places them in accumulation registers and
# copies them to and fro, about 900 copies in the block-attention split kernel
# (304 registers, one wave per SIMD; 200 and two waves in this form) and 1,000
# in the dual-stream backward.  Measured A/B on one box: backward 319-320
# against 332-334 us, the decode step +0.4-0.5%, the rest unchanged.  The
# compiler's other scheduling strategies (max-ilp, iterative-ilp,
# max-memory-clause) and its automatic wave priorities measured slower on
# the backward (322-329 us) and no better elsewhere.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


# Host-only sanitizer build: each -fsanitize= applies to the host pass only.
HOST_SAN_FLAGS = [
    "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]
HOST_SAN_LIB = BUILD / "libbdiff_host_asan.so"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libbdiff")
    return exe


def sources():
    return sorted(CSRC.glob("*.hip"))


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


def host_asan_runtime() -> Path:
    """The AddressSanitizer runtime of the compiler hipcc drives (it also
    carries the UndefinedBehaviorSanitizer handlers)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    p = Path(r.stdout.strip())
    if r.returncode != 0 or not p.is_absolute() or not p.exists():
        raise RuntimeError("the compiler's AddressSanitizer runtime was not found")
    return p


def build_host_sanitized(verbose: bool = True) -> Path:
    """Host code of every source with ASan + UBSan, linked without device code."""
    san = BUILD / "host_asan"
    san.mkdir(parents=True, exist_ok=True)

    def one(src: Path) -> Path:
        obj = san / (src.stem + ".o")
        r = subprocess.run([hipcc(), *HOST_SAN_FLAGS, "-c", str(src), "-o", str(obj)],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host sanitizer build failed on {src.name}:\n{r.stderr}")
        return obj

    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(one, srcs))
    r = subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, objs),
                        "-o", str(HOST_SAN_LIB)], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host sanitizer link failed:\n{r.stderr}")
    if verbose:
        print(f"built {HOST_SAN_LIB} (host code only, ASan + UBSan)", file=sys.stderr)
    return HOST_SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "host-sanitized":
        build_host_sanitized()
    else:
        build()
